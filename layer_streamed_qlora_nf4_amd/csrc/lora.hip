// Rank-r LoRA kernels for gfx950: the down-projection U = s X A^T, the
// gradient projection G = s dY B, the adapter gradients dA = G^T X and
// dB = dY^T U (LS-docs "Honest scope": plain LoRA; About: only the adapters
// train), and the per-step transposed copy of the adapters.
//
// Each product is one launch.  Where a launch splits its reduction over
// workgroups (the input dimension for U and G, the tokens for dA and dB), every
// workgroup writes a float32 partial and the last workgroup of its group to
// arrive (an integer counter) sums the group's partials in a fixed order
// (chunk or token-range order) and writes the result: no float atomics, and
// the sum does not depend on which workgroup arrives last, so a resident and a
// streamed run give identical bits (LS-docs "Bit-exact is two claims, not one").
// The counters live in the caller's workspace, are zeroed once by the caller
// (zero_counters) and are returned to zero by each last workgroup.
#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "layer.h"
#include "layer_ops.h"

namespace lsq {
namespace {

constexpr int NT = 256;          // 4 waves
constexpr int KCHUNK = 512;      // reduction columns per workgroup of the down / G projections

__device__ __forceinline__ bf16x8 as_frag(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The float32 partials of a split reduction cross XCDs, whose L2 caches are
// not coherent with each other.  They are therefore written and read as
// device-scope relaxed atomics (stores and loads that are coherent at the
// device level: they write through and read past the XCD's L2), which needs
// no cache-wide write-back or invalidation; only completion order matters.
__device__ __forceinline__ void put_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// v[i] = 0 + p[e_i] + p[e_i + stride] + ... + p[e_i + (count - 1) stride] over
// partials, in k order, for the E elements e_i = e0 + i step below n (v[i] = 0
// past n).  The loads of E elements x 8 partials are all issued before the
// first sum, so a last workgroup's reduction costs count / 8 memory round
// trips per E elements rather than one per element.
template <int E>
__device__ __forceinline__ void ordered_partial_sums(float (&v)[E], const float* p, int64_t stride, int e0, int step,
                                                     int n, int count) {
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = 0.f;
  for (int kb = 0; kb < count; kb += 8) {
    float t[E][8];
#pragma unroll
    for (int i = 0; i < E; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + i * step;
        t[i][j] = (kb + j < count && e < n) ? get_partial(p + e + (int64_t)(kb + j) * stride) : 0.f;
      }
#pragma unroll
    for (int i = 0; i < E; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (kb + j < count) v[i] += t[i][j];
  }
}

// Call after this workgroup's put_partial stores: true, in every thread, for
// the one workgroup of the n sharing *counter that arrives last.  Every
// thread waits for its stores to complete at device scope before the
// barrier, so the count is taken only once the workgroup's partials are
// visible to any XCD; the last workgroup reads them with get_partial after
// its count returned, and puts the counter back to zero for the next launch.
__device__ __forceinline__ bool last_arriver(int* counter, int n) {
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == n - 1;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

// RT 16-row tiles of S = X W^T for a skinny W [nw, K] (nw <= 64) over the
// reduction columns [kb0, kb0 + KCHUNK): the 4 waves take 128 columns each
// (4 MFMA steps of 32; every load issued before the first MFMA; addresses
// clamped into the operands, values masked) and meet in red[wave] [16 RT][64].
// A wave loads its W fragments once for all RT row tiles, so W's bytes per
// workgroup are spread over 16 RT rows of X.  Each row tile's accumulation
// (k order inside the wave, then the four waves in order) does not depend on
// RT.
template <int RT>
__device__ __forceinline__ void skinny_block(const uint16_t* __restrict__ X, int64_t ldx, int M, int m0, int K,
                                             int kb0, int kend, const uint16_t* __restrict__ W, int64_t ldw, int nw,
                                             float (&red)[4][16 * RT][64]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nct = (nw + 15) / 16;
  const int kb = kb0 + wave * (KCHUNK / 4), ke = min(kend, kb + KCHUNK / 4);
  const int g = lane >> 4;
  constexpr int NS = KCHUNK / 4 / 32;
  f32x4 acc[RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[t][ct] = f32x4{0, 0, 0, 0};
  uint4 av[RT][NS], bv[NS][4];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int kk = kb + 32 * i + 8 * g, kkc = min(kk, K - 8);
    const bool kin = kk < ke;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = m0 + 16 * t + (lane & 15);
      const uint4 x = *reinterpret_cast<const uint4*>(X + (int64_t)min(row, M - 1) * ldx + kkc);
      av[t][i] = (row < M && kin) ? x : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (ct >= nct) break;
      const int c = ct * 16 + (lane & 15);
      const uint4 w = *reinterpret_cast<const uint4*>(W + (int64_t)min(c, nw - 1) * ldw + kkc);
      bv[i][ct] = (c < nw && kin) ? w : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (ct >= nct) break;
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t][ct] = mfma(as_frag(av[t][i]), as_frag(bv[i][ct]), acc[t][ct]);
    }
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (ct >= nct) break;
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][16 * t + 4 * g + v][ct * 16 + (lane & 15)] = acc[t][ct][v];
    }
  __syncthreads();
}

// ------------------------------------------------------------- down: U = s X A^T
struct DownArgs {
  const uint16_t* X;
  int64_t ldx;
  int M, K, rr, nch;
  const uint16_t* A;   // [rr, K]
  float s;
  uint16_t* U;         // [M, ldu] bf16
  int64_t ldu;
  float* U32;          // [M, ldu32] float32 (nullable)
  int64_t ldu32;
  float* part;         // [row blocks][nch][16 RT][rr]
  int* cnt;            // one per row block
};

// Grid (row blocks of 16 RT, chunks of KCHUNK input columns).
template <int RT>
__global__ void __launch_bounds__(NT) lora_down_kernel(DownArgs a) {
  __shared__ float red[4][16 * RT][64];
  const int rb = blockIdx.x, chunk = blockIdx.y, m0 = rb * 16 * RT, tid = threadIdx.x;
  skinny_block<RT>(a.X, a.ldx, a.M, m0, a.K, chunk * KCHUNK, a.K, a.A, a.K, a.rr, red);
  const int n = 16 * RT * a.rr;
  auto finish = [&](int e, float v) {
    const int r = e / a.rr, c = e % a.rr;
    v *= a.s;
    a.U[(int64_t)(m0 + r) * a.ldu + c] = f32_to_bf16_bits(v);
    if (a.U32) a.U32[(int64_t)(m0 + r) * a.ldu32 + c] = v;
  };
  if (a.nch == 1) {
    for (int e = tid; e < n; e += NT) {
      const int r = e / a.rr, c = e % a.rr;
      if (m0 + r < a.M) finish(e, 0.f + (((red[0][r][c] + red[1][r][c]) + red[2][r][c]) + red[3][r][c]));
    }
    return;
  }
  float* base = a.part + (int64_t)rb * a.nch * n;
  for (int e = tid; e < n; e += NT) {
    const int r = e / a.rr, c = e % a.rr;
    put_partial(base + (int64_t)chunk * n + e, ((red[0][r][c] + red[1][r][c]) + red[2][r][c]) + red[3][r][c]);
  }
  if (!last_arriver(a.cnt + rb, a.nch)) return;
  constexpr int E = 4;
  for (int e0 = tid; e0 < n; e0 += E * NT) {
    float v[E];
    ordered_partial_sums<E>(v, base, n, e0, NT, n, a.nch);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = e0 + i * NT;
      if (e < n && m0 + e / a.rr < a.M) finish(e, v[i]);
    }
  }
}

// ------------------------------------------------------------- G = s dY_seg B_seg
// Reduction chunks of KCHUNK columns inside each segment of dY's columns;
// chunk c of the launch belongs to the segment whose chunk range holds it.
struct GArgs {
  const uint16_t* dY;
  int64_t ldy;
  int M, N, r, nseg;
  int seg_end[4];
  const uint16_t* Bt;  // B transposed [r, N]
  float s;
  uint16_t* G;         // [M, ldg] bf16: segment s at columns [s r, s r + r)
  int64_t ldg;
  float* G32;          // [M, ldg32] (nullable)
  int64_t ldg32;
  float* part;         // [row blocks][total chunks][16 RT][r]
  int* cnt;            // [row blocks][nseg]
  int nch;             // total chunks
};

__device__ __forceinline__ int seg_chunks(int len) { return (len + KCHUNK - 1) / KCHUNK; }

// Grid (row blocks of 16 RT, chunks).
template <int RT>
__global__ void __launch_bounds__(NT) lora_g_kernel(GArgs a) {
  __shared__ float red[4][16 * RT][64];
  const int rb = blockIdx.x, chunk = blockIdx.y, m0 = rb * 16 * RT, tid = threadIdx.x;
  // this chunk's segment, its column range and the segment's first chunk
  int sg = 0, c0 = 0, nb = 0, ne = a.seg_end[0];
  int first = 0, begin = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= a.nseg) break;
    const int end = a.seg_end[i], nc = seg_chunks(end - begin);
    if (chunk >= first && chunk < first + nc) {
      sg = i;
      c0 = first;
      nb = begin;
      ne = end;
    }
    first += nc;
    begin = end;
  }
  const int nsc = seg_chunks(ne - nb);
  skinny_block<RT>(a.dY, a.ldy, a.M, m0, a.N, nb + (chunk - c0) * KCHUNK, ne, a.Bt, a.N, a.r, red);
  const int n = 16 * RT * a.r;
  auto finish = [&](int e, float v) {
    const int rr = e / a.r, c = e % a.r;
    v *= a.s;
    a.G[(int64_t)(m0 + rr) * a.ldg + sg * a.r + c] = f32_to_bf16_bits(v);
    if (a.G32) a.G32[(int64_t)(m0 + rr) * a.ldg32 + sg * a.r + c] = v;
  };
  if (nsc == 1) {
    for (int e = tid; e < n; e += NT) {
      const int rr = e / a.r, c = e % a.r;
      if (m0 + rr < a.M) finish(e, 0.f + (((red[0][rr][c] + red[1][rr][c]) + red[2][rr][c]) + red[3][rr][c]));
    }
    return;
  }
  float* base = a.part + ((int64_t)rb * a.nch + c0) * n;
  for (int e = tid; e < n; e += NT) {
    const int rr = e / a.r, c = e % a.r;
    put_partial(base + (int64_t)(chunk - c0) * n + e,
                ((red[0][rr][c] + red[1][rr][c]) + red[2][rr][c]) + red[3][rr][c]);
  }
  if (!last_arriver(a.cnt + rb * a.nseg + sg, nsc)) return;
  constexpr int E = 4;
  for (int e0 = tid; e0 < n; e0 += E * NT) {
    float v[E];
    ordered_partial_sums<E>(v, base, n, e0, NT, n, nsc);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = e0 + i * NT;
      if (e < n && m0 + e / a.r < a.M) finish(e, v[i]);
    }
  }
}

// ------------------------------------------------------------- dA = G^T X, dB = dY^T U
// The adapter gradients of one linear group in one launch, on the matrix
// cores.  out[a][b] = sum over tokens of S[m][a] L[m][b] is an MFMA product
// with the tokens as its reduction: each k-step stages 64 tokens of L (128
// columns) and of S (all small indices) in LDS transposed, token-major per
// column, so a lane's 8 reduction values are contiguous.  S is float32 (the
// unrounded G or U); it enters the bf16 MFMA as a hi/lo pair (hi = bf16(S),
// lo = bf16(S - hi)), which carries 16 of its 24 mantissa bits into an exact
// product with L's bf16 values and float32 accumulation.
//
// Tasks (derived from the arguments, in this order): dA of the stacked group
// (S = G, L = X; one task, or one per segment when the stacked rank exceeds
// 64), then dB of each segment (S = U_seg, L = dY_seg).  Each workgroup owns
// every small index of 128 columns of one task over one token range; with
// several ranges, the last range of a column tile to finish sums the tile's
// range partials in range order.
struct GradsArgs {
  const float* G;       // [M, ldg] float32, segments' columns stacked
  int64_t ldg;
  const float* U;       // [M, ldu] float32
  int64_t ldu;
  const uint16_t* X;    // [M, ldx] bf16, Kx columns
  int64_t ldx;
  const uint16_t* dY;   // [M, ldy] bf16, seg_end[nseg - 1] columns
  int64_t ldy;
  int Kx, r, nseg, M;
  int seg_end[3];
  float* gA;            // [nseg r, Kx]
  float* gB;            // [N, r]
  int accumulate, splits, per;
  float* part;          // [column tiles][splits][64][128]
  int* cnt;             // one per column tile
};
constexpr int TNM_COLS = 128, TNM_TOK = 64;
// Element offset of (column, token) in the staged L tile: unpadded 128-byte
// column rows whose 16-byte chunks of 8 tokens are permuted per column (chunk
// index XOR (col ^ 5 (col >> 3)) & 7), and of (small index, token) in the
// staged S tile: 256-byte rows of 16 chunks of 4 tokens, chunk index XOR
// row & 15.  Measured on gfx950 (SQ_LDS_BANK_CONFLICT): the fragment reads of
// both tiles are conflict-free, and the L staging writes (one thread: 8
// columns 8 apart, 4 tokens) cost 4 conflict cycles each instead of the 60
// of rows padded to 144 bytes; the S reads cost 4 in rows padded to 272 bytes.
__device__ __forceinline__ int lt_off(int col, int tok) {
  return col * TNM_TOK + ((((tok >> 3) ^ col ^ (5 * (col >> 3))) & 7) << 3) + (tok & 7);
}
__device__ __forceinline__ int st_off(int row, int tok) {
  return row * TNM_TOK + ((((tok >> 2) ^ row) & 15) << 2) + (tok & 3);
}

struct Task {
  const float* S;
  int64_t lds;
  int ns;
  const uint16_t* L;
  int64_t ldl;
  int nl;
  float* out;
  int64_t ldo;
  int small_rows;
  int tile0;
};

__device__ __forceinline__ Task grads_task(const GradsArgs& a, int tile) {
  const bool split_a = a.nseg * a.r > 64;
  Task t{};
  int t0 = 0;
  // dA tasks
  const int na = split_a ? a.nseg : 1;
  const int tiles_a = (a.Kx + TNM_COLS - 1) / TNM_COLS;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i >= na) break;
    if (tile >= t0) {
      t.S = a.G + (split_a ? i * a.r : 0);
      t.lds = a.ldg;
      t.ns = split_a ? a.r : a.nseg * a.r;
      t.L = a.X;
      t.ldl = a.ldx;
      t.nl = a.Kx;
      t.out = a.gA + (split_a ? (int64_t)i * a.r * a.Kx : 0);
      t.ldo = a.Kx;
      t.small_rows = 1;
      t.tile0 = t0;
    }
    t0 += tiles_a;
  }
  // dB tasks
  int nb = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i >= a.nseg) break;
    const int ne = a.seg_end[i];
    if (tile >= t0) {
      t.S = a.U + i * a.r;
      t.lds = a.ldu;
      t.ns = a.r;
      t.L = a.dY + nb;
      t.ldl = a.ldy;
      t.nl = ne - nb;
      t.out = a.gB + (int64_t)nb * a.r;
      t.ldo = a.r;
      t.small_rows = 0;
      t.tile0 = t0;
    }
    t0 += (ne - nb + TNM_COLS - 1) / TNM_COLS;
    nb = ne;
  }
  return t;
}

__global__ void __launch_bounds__(NT) lora_grads_kernel(GradsArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t LT[TNM_COLS * TNM_TOK];   // [column][token] by lt_off, bf16
  __shared__ __attribute__((aligned(16))) float ST[64 * TNM_TOK];               // [small index][token] by st_off
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Task tk = grads_task(a, blockIdx.x);
  const int b0 = (blockIdx.x - tk.tile0) * TNM_COLS;
  const int ns = tk.ns;
  const int m_lo = blockIdx.y * a.per;
  const int m_hi = min(a.M, m_lo + a.per);
  // this thread's L micro-tile (4 tokens x 8 columns) and S row (one token, 16 small indices)
  const int lr = 4 * (tid >> 4), lc = 8 * (tid & 15);
  const int scol = b0 + lc;
  const int sa = 16 * wave;
  // Two register sets of staged operands, by k-step parity: the loads of
  // k-step k + 2 go out while k-step k + 1 waits in the other set, so two
  // k-steps of each workgroup are in flight while it computes.
  uint4 lv[2][4];
  float4 sv[2][4];
  auto load = [&](int m0, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + lr + i;
      const uint16_t* row = tk.L + (int64_t)m * tk.ldl + scol;
      if (m < m_hi && scol + 8 <= tk.nl) {
        lv[set][i] = *reinterpret_cast<const uint4*>(row);
      } else if (m < m_hi && scol + 4 <= tk.nl) {
        const uint2 h = *reinterpret_cast<const uint2*>(row);
        lv[set][i] = make_uint4(h.x, h.y, 0u, 0u);
      } else {
        lv[set][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    const int m = m0 + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int aa = sa + 4 * q;
      sv[set][q] = (m < m_hi && aa < ns) ? *reinterpret_cast<const float4*>(tk.S + (int64_t)m * tk.lds + aa)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&](int set) __attribute__((always_inline)) {
    const uint4(&l)[4] = lv[set];
    const uint32_t w[4][4] = {{l[0].x, l[0].y, l[0].z, l[0].w}, {l[1].x, l[1].y, l[1].z, l[1].w},
                              {l[2].x, l[2].y, l[2].z, l[2].w}, {l[3].x, l[3].y, l[3].z, l[3].w}};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int sel = (c & 1) ? 0x07060302 : 0x05040100;   // high or low bf16 of each token's word
      const uint32_t lo = __builtin_amdgcn_perm(w[1][c >> 1], w[0][c >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(w[3][c >> 1], w[2][c >> 1], sel);
      *reinterpret_cast<u32x2*>(&LT[lt_off(lc + c, lr)]) = u32x2{lo, hi};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ST[st_off(sa + 4 * q + 0, lane)] = sv[set][q].x;
      ST[st_off(sa + 4 * q + 1, lane)] = sv[set][q].y;
      ST[st_off(sa + 4 * q + 2, lane)] = sv[set][q].z;
      ST[st_off(sa + 4 * q + 3, lane)] = sv[set][q].w;
    }
  };
  const int J = (ns + 15) / 16;
  f32x4 acc[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g][0] = acc[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The tokens' products in k-step order, one k-step staged in LDS at a time.
  auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int t0 = 32 * kb + 8 * (lane >> 4);
      bf16x8 bfr[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        bfr[c] = *reinterpret_cast<const bf16x8*>(&LT[lt_off(32 * wave + 16 * c + (lane & 15), t0)]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g >= J) break;
        const int srow = 16 * g + (lane & 15);
        const float4 f0 = *reinterpret_cast<const float4*>(&ST[st_off(srow, t0)]);
        const float4 f1 = *reinterpret_cast<const float4*>(&ST[st_off(srow, t0 + 4)]);
        const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          hw[t] = pack_bf16x2(f[2 * t], f[2 * t + 1]);
          lw[t] = pack_bf16x2(f[2 * t] - bf_lo(hw[t]), f[2 * t + 1] - bf_hi(hw[t]));
        }
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        const bf16x8 alo = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          acc[g][c] = mfma(ahi, bfr[c], acc[g][c]);
          acc[g][c] = mfma(alo, bfr[c], acc[g][c]);
        }
      }
    }
  };
  auto step = [&](int m0, int set) __attribute__((always_inline)) {
    __syncthreads();   // the previous k-step's fragment reads are done
    store(set);
    __syncthreads();
    if (m0 + 2 * TNM_TOK < m_hi) load(m0 + 2 * TNM_TOK, set);
    compute();
  };
  load(m_lo, 0);
  if (m_lo + TNM_TOK < m_hi) load(m_lo + TNM_TOK, 1);
  for (int m0 = m_lo; m0 < m_hi; m0 += 2 * TNM_TOK) {
    step(m0, 0);
    if (m0 + TNM_TOK >= m_hi) break;
    step(m0 + TNM_TOK, 1);
  }
  // lane holds C[4 (lane >> 4) + v][lane & 15]: small index row, column
  auto put = [&](int aa, int b, float v) {
    const int64_t o = tk.small_rows ? (int64_t)aa * tk.ldo + b : (int64_t)b * tk.ldo + aa;
    tk.out[o] = a.accumulate ? tk.out[o] + v : v;
  };
  if (a.splits == 1) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g >= J) break;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int b = b0 + 32 * wave + 16 * c + (lane & 15);
        if (b >= tk.nl) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int aa = 16 * g + 4 * (lane >> 4) + v;
          if (aa < ns) put(aa, b, acc[g][c][v]);
        }
      }
    }
    return;
  }
  // this range's partial of the tile: [ns][128], then the last range sums them in range order
  constexpr int PT = 64 * TNM_COLS;
  float* base = a.part + (int64_t)blockIdx.x * a.splits * PT;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g >= J) break;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int bl = 32 * wave + 16 * c + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int aa = 16 * g + 4 * (lane >> 4) + v;
        put_partial(base + (int64_t)blockIdx.y * PT + aa * TNM_COLS + bl, acc[g][c][v]);
      }
    }
  }
  if (!last_arriver(a.cnt + blockIdx.x, a.splits)) return;
  constexpr int E = 8;
  const int n = ns * TNM_COLS;
  for (int e0 = tid; e0 < n; e0 += E * NT) {
    float v[E];
    ordered_partial_sums<E>(v, base, PT, e0, NT, n, a.splits);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = e0 + i * NT;
      if (e >= n) break;
      const int aa = e / TNM_COLS, bl = e % TNM_COLS;
      if (b0 + bl < tk.nl) put(aa, b0 + bl, v[i]);
    }
  }
}

// ------------------------------------------------------------- adapter transposes
// Per layer of an adapter arena (layer_elems apart): A_g [rr_g, K_g] -> [K_g, rr_g]
// and B_g [N_g, r] -> [r, N_g] at the same offsets of the output arena, so the
// G projection and the backward GEMM read 8 consecutive reduction values per
// lane.  One thread per output element (coalesced writes; the strided reads
// of these small blocks come from cache).  Grid (elements, layers).
struct TransposeArgs {
  const uint16_t* src;
  uint16_t* dst;
  int64_t layer_elems;
  int nblk;
  int64_t off[8];
  int rows[8], cols[8];   // of the source block
  int64_t end[8];         // cumulative element counts
};
__global__ void adapter_transpose_kernel(TransposeArgs a) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.end[a.nblk - 1]) return;
  int64_t off = a.off[0], start = 0;
  int rows = a.rows[0], cols = a.cols[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    if (i < a.nblk && e >= a.end[i - 1]) {
      off = a.off[i];
      start = a.end[i - 1];
      rows = a.rows[i];
      cols = a.cols[i];
    }
  }
  const int64_t k = e - start;             // output element [cols][rows]
  const int64_t j = k / rows, i = k % rows;
  const int64_t lb = (int64_t)blockIdx.y * a.layer_elems + off;
  a.dst[lb + k] = a.src[lb + i * cols + j];
}

}  // namespace

// ================================================================ launchers
size_t counters_bytes(int n) { return ((size_t)std::max(n, 1) * sizeof(int) + 255) / 256 * 256; }

int zero_counters(int* cnt, int n, hipStream_t s) { return zero_words(cnt, n, 1, n, s); }

// Row tiles per workgroup of the down and G projections: the largest of 4, 2
// and 1 that still gives the launch kSkinnyBlocks workgroups (about two per
// CU), so that small launches keep every CU loading and large ones read the
// skinny operand once per 64 or 32 rows instead of once per 16.
constexpr int kSkinnyBlocks = 512;
static int skinny_rt(int M, int nch) {
  for (int rt = 4; rt > 1; rt /= 2)
    if ((int64_t)((M + 16 * rt - 1) / (16 * rt)) * nch >= kSkinnyBlocks) return rt;
  return 1;
}
// Partial rows of a split launch: M rounded up to 64 covers every row tiling.
static int64_t skinny_part_rows(int M) { return ((int64_t)M + 63) / 64 * 64; }

int lora_down_counters(int M) { return (M + 15) / 16; }
size_t lora_down_ws_bytes(int M, int K, int rr) {
  const int nch = (K + KCHUNK - 1) / KCHUNK;
  return nch > 1 ? (size_t)skinny_part_rows(M) * nch * rr * sizeof(float) : 0;
}

int lora_down(const uint16_t* X, int64_t ldx, int M, int K, const uint16_t* A, int rr, float s, uint16_t* U,
              int64_t ldu, float* U32, int64_t ldu32, float* ws, size_t ws_bytes, int* cnt, hipStream_t st) {
  LSQ_CHECK(rr >= 1 && rr <= 64 && K >= 32 && K % 32 == 0, LSQ_ERR_SHAPE, "lora_down: rank %d / K %d unsupported", rr,
            K);
  if (M == 0) return LSQ_OK;
  const int nch = (K + KCHUNK - 1) / KCHUNK;
  LSQ_CHECK(nch == 1 || (ws && ws_bytes >= lora_down_ws_bytes(M, K, rr) && cnt), LSQ_ERR_WORKSPACE,
            "lora_down: workspace too small");
  DownArgs a{X, ldx, M, K, rr, nch, A, s, U, ldu, U32, ldu32, ws, cnt};
  const int rt = skinny_rt(M, nch);
  const dim3 grid((M + 16 * rt - 1) / (16 * rt), nch);
  int tok = prof_begin(st);
  if (rt == 4) lora_down_kernel<4><<<grid, NT, 0, st>>>(a);
  else if (rt == 2) lora_down_kernel<2><<<grid, NT, 0, st>>>(a);
  else lora_down_kernel<1><<<grid, NT, 0, st>>>(a);
  prof_end(tok, st, PROF_LORA, 2.0 * M * (double)K * rr, 2.0 * M * (double)K + 2.0 * rr * K + 2.0 * M * rr);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

static int g_total_chunks(int nseg, const SegEnds& segs) {
  int n = 0;
  for (int i = 0; i < nseg; ++i) n += (segs.end[i] - (i ? segs.end[i - 1] : 0) + KCHUNK - 1) / KCHUNK;
  return n;
}
int lora_g_counters(int M, int nseg) { return (M + 15) / 16 * nseg; }
size_t lora_g_ws_bytes(int M, int N, int r) {
  // chunks <= N / KCHUNK + one partial chunk per segment (at most 4)
  return (size_t)skinny_part_rows(M) * ((N + KCHUNK - 1) / KCHUNK + 4) * r * sizeof(float);
}

int lora_g(const uint16_t* dY, int64_t ldy, int M, int N, const uint16_t* Bt, int r, int nseg, const SegEnds& segs,
           float s, uint16_t* G, int64_t ldg, float* G32, int64_t ldg32, float* ws, size_t ws_bytes, int* cnt,
           hipStream_t st) {
  LSQ_CHECK(r >= 1 && r <= 64 && r % 8 == 0 && nseg >= 1 && nseg <= 4 && N >= 8 && N % 8 == 0 &&
                segs.end[nseg - 1] == N,
            LSQ_ERR_SHAPE, "lora_g: bad rank/segments/N");
  for (int i = 0; i < nseg; ++i)
    LSQ_CHECK(segs.end[i] > (i ? segs.end[i - 1] : 0) && segs.end[i] % 8 == 0, LSQ_ERR_SHAPE,
              "lora_g: segment %d is empty or not a multiple of 8", i);
  if (M == 0) return LSQ_OK;
  LSQ_CHECK(ws && ws_bytes >= lora_g_ws_bytes(M, N, r) && cnt, LSQ_ERR_WORKSPACE, "lora_g: workspace too small");
  GArgs a{};
  a.dY = dY;
  a.ldy = ldy;
  a.M = M;
  a.N = N;
  a.r = r;
  a.nseg = nseg;
  for (int i = 0; i < 4; ++i) a.seg_end[i] = i < nseg ? segs.end[i] : N;
  a.Bt = Bt;
  a.s = s;
  a.G = G;
  a.ldg = ldg;
  a.G32 = G32;
  a.ldg32 = ldg32;
  a.part = ws;
  a.cnt = cnt;
  a.nch = g_total_chunks(nseg, segs);
  const int rt = skinny_rt(M, a.nch);
  const dim3 grid((M + 16 * rt - 1) / (16 * rt), a.nch);
  int tok = prof_begin(st);
  if (rt == 4) lora_g_kernel<4><<<grid, NT, 0, st>>>(a);
  else if (rt == 2) lora_g_kernel<2><<<grid, NT, 0, st>>>(a);
  else lora_g_kernel<1><<<grid, NT, 0, st>>>(a);
  prof_end(tok, st, PROF_LORA, 2.0 * M * (double)N * r, 2.0 * M * (double)N + 2.0 * N * r + 2.0 * M * r * nseg);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

// Token ranges of a lora_grads launch: enough column-tile x range workgroups
// to keep about four per CU loading (each walks its range 64 tokens at a
// time), at least 128 tokens per range, at most 8 ranges.
static int grads_tiles(int Kx, int r, int nseg, const int* seg_end) {
  const int na = nseg * r > 64 ? nseg : 1;
  int t = na * ((Kx + TNM_COLS - 1) / TNM_COLS);
  for (int i = 0; i < nseg; ++i) t += (seg_end[i] - (i ? seg_end[i - 1] : 0) + TNM_COLS - 1) / TNM_COLS;
  return t;
}
static int grads_splits(int tiles, int M) { return std::max(1, std::min({8, (1024 + tiles - 1) / tiles, M / 128})); }
int lora_grads_counters(int Kx, int r, int nseg, const int* seg_end) { return grads_tiles(Kx, r, nseg, seg_end); }
size_t lora_grads_ws_bytes(int Kx, int r, int nseg, const int* seg_end, int M) {
  const int tiles = grads_tiles(Kx, r, nseg, seg_end);
  const int sp = grads_splits(tiles, M);
  return sp > 1 ? (size_t)tiles * sp * 64 * TNM_COLS * sizeof(float) : 0;
}

int lora_grads(const GradGroup& g, int M, int accumulate, float* ws, size_t ws_bytes, int* cnt, hipStream_t st) {
  LSQ_CHECK(g.nseg >= 1 && g.nseg <= 3 && g.r >= 8 && g.r <= 64 && g.r % 8 == 0 && g.Kx % 8 == 0, LSQ_ERR_SHAPE,
            "lora_grads: %d segments of rank %d over %d columns unsupported", g.nseg, g.r, g.Kx);
  LSQ_CHECK(g.ldx % 8 == 0 && g.ldy % 8 == 0 && g.ldg % 4 == 0 && g.ldu % 4 == 0 && aligned16(g.X) &&
                aligned16(g.dY) && aligned16(g.G) && aligned16(g.U),
            LSQ_ERR_SHAPE, "lora_grads: operands must be in 16-byte rows");
  for (int i = 0; i < g.nseg; ++i)
    LSQ_CHECK(g.seg_end[i] > (i ? g.seg_end[i - 1] : 0) && g.seg_end[i] % 8 == 0, LSQ_ERR_SHAPE,
              "lora_grads: segment %d is empty or not a multiple of 8", i);
  const int N = g.seg_end[g.nseg - 1];
  if (M == 0) {
    if (accumulate) return LSQ_OK;
    if (int e = zero_words(g.gA, g.Kx, g.nseg * g.r, g.Kx, st)) return e;
    return zero_words(g.gB, g.r, N, g.r, st);
  }
  const int tiles = grads_tiles(g.Kx, g.r, g.nseg, g.seg_end);
  GradsArgs a{};
  a.G = g.G;
  a.ldg = g.ldg;
  a.U = g.U;
  a.ldu = g.ldu;
  a.X = g.X;
  a.ldx = g.ldx;
  a.dY = g.dY;
  a.ldy = g.ldy;
  a.Kx = g.Kx;
  a.r = g.r;
  a.nseg = g.nseg;
  a.M = M;
  for (int i = 0; i < 3; ++i) a.seg_end[i] = i < g.nseg ? g.seg_end[i] : N;
  a.gA = g.gA;
  a.gB = g.gB;
  a.accumulate = accumulate;
  a.splits = grads_splits(tiles, M);
  a.per = M;
  if (a.splits > 1) {
    LSQ_CHECK(ws && ws_bytes >= lora_grads_ws_bytes(g.Kx, g.r, g.nseg, g.seg_end, M) && cnt, LSQ_ERR_WORKSPACE,
              "lora_grads: needs %zu bytes of workspace", lora_grads_ws_bytes(g.Kx, g.r, g.nseg, g.seg_end, M));
    a.per = ((M + a.splits - 1) / a.splits + TNM_TOK - 1) / TNM_TOK * TNM_TOK;
    a.splits = (M + a.per - 1) / a.per;   // every range holds tokens
    a.part = ws;
    a.cnt = cnt;
  }
  const double nsa = (double)g.nseg * g.r;
  const double flops = 2.0 * M * nsa * g.Kx + 2.0 * M * (double)N * g.r;
  const double bytes = 4.0 * M * nsa + 2.0 * M * g.Kx + 4.0 * nsa * g.Kx + 4.0 * M * nsa + 2.0 * M * N + 4.0 * N * g.r;
  int tok = prof_begin(st);
  lora_grads_kernel<<<dim3(tiles, a.splits), NT, 0, st>>>(a);
  prof_end(tok, st, PROF_LORA, flops, bytes);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int adapter_transpose(const lsq_model_cfg* c, const uint16_t* lora, uint16_t* lora_t, int n_layers, hipStream_t st) {
  lsq_lora_layout L;
  lora_layout(c, &L);
  const int r = c->lora_r;
  const int H = c->hidden, Nq = c->n_heads * c->head_dim, Nkv = c->n_kv_heads * c->head_dim, I = c->intermediate;
  const int gN[4] = {Nq + 2 * Nkv, H, 2 * I, H}, gK[4] = {H, Nq, H, I}, rr[4] = {3 * r, r, 2 * r, r};
  TransposeArgs a{};
  a.src = lora;
  a.dst = lora_t;
  a.layer_elems = (int64_t)L.layer_elems;
  a.nblk = 8;
  int64_t acc = 0;
  for (int g = 0; g < 4; ++g) {
    a.off[g] = (int64_t)L.a_off[g];
    a.rows[g] = rr[g];
    a.cols[g] = gK[g];
    acc += (int64_t)rr[g] * gK[g];
    a.end[g] = acc;
  }
  for (int g = 0; g < 4; ++g) {
    a.off[4 + g] = (int64_t)L.b_off[g];
    a.rows[4 + g] = gN[g];
    a.cols[4 + g] = r;
    acc += (int64_t)gN[g] * r;
    a.end[4 + g] = acc;
  }
  if (n_layers <= 0) return LSQ_OK;
  int tok = prof_begin(st);
  adapter_transpose_kernel<<<dim3((unsigned)((acc + 255) / 256), n_layers), 256, 0, st>>>(a);
  prof_end(tok, st, PROF_OTHER, 0.0, 4.0 * acc * n_layers);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

}  // namespace lsq
