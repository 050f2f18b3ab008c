// NF4-LoRA linear kernels for gfx950: the fused dequantize + GEMM + LoRA
// forward, the transposed-decode backward for dX, and the skinny LoRA GEMMs.
//
// The pages run the base linear through bitsandbytes (a fused 4-bit GEMM for
// few rows, dequantize + matmul otherwise, and a backward that always
// dequantises because no transposed 4-bit GEMM exists: LS-docs "Bit-exact is
// two claims, not one"; "v0.76.0 changes the code").  Here both directions
// decode NF4 inside the GEMM: packed codes and float32 absmax stream from HBM
// (0.5625 B per weight), each workgroup decodes its weight tile once into LDS
// as bf16 (the forward's main kernel looks levels up with byte permutes of a
// per-row table in registers, the others through a 16-entry table in LDS),
// and bf16 MFMA 16x16x32 tiles with
// float32 accumulation consume it.  The LoRA up-projection U B^T (forward) and
// G A (backward) ride in the same accumulators.  The kernel chosen depends on
// (M, N, K, r) only, so resident and streamed runs execute identical code.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include <hip/hip_ext.h>

#include "common.h"
#include "gemm.h"
#include "layer_ops.h"
#include "nf4_levels.h"

namespace lsq {
namespace {

constexpr int BK = 64;          // reduction step = one NF4 block
constexpr int kTile = 256;      // output tile edge of every GEMM kernel (256 x 256, 8 waves)
constexpr int NTHREADS = 256;   // 4 waves

// ------------------------------------------------------------------ LDS tiles
// A tile row r holds 64 bf16 of the reduction dimension as 8 chunks of 16 B;
// chunk c of row r lives at chunk position c ^ (r & 7), so the 8 lanes of a
// 128-bit LDS pass read 8 different bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }
// Transposed weight tile (backward): row = output column k, 64 reduction values.
// The swizzle also folds in 5 (k >> 3) so the transposing writes (rows 8
// apart) spread over banks too.  Measured on gfx950 with
// SQ_LDS_BANK_CONFLICT, both the fragment reads (16 consecutive rows) and the
// transposing 8-byte writes are conflict-free with this form; folding in
// k >> 3 unmultiplied cost 4 conflict cycles per fragment read.
__device__ __forceinline__ int swzt(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row ^ (5 * (row >> 3))) & 7)) << 3);
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base, int idx) {
  return *reinterpret_cast<const bf16x8*>(base + idx);
}
__device__ __forceinline__ bf16x8 u4_as_frag(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// XCD-aware work order.  Workgroups are handed to the 8 XCDs round-robin in
// dispatch order (x fastest), and each XCD has its own L2.  A launch of
// `tiles` output tiles x `splits` reduction ranges is therefore renumbered so
// that each XCD receives one contiguous run of (split, tile) pairs in
// split-major order: with one range, a run of neighbouring tiles (column-major,
// so the tiles that share a weight slab read it into one L2); with several,
// the tiles of one reduction range, whose activation and weight columns then
// leave HBM once instead of once per XCD.
struct TileSplit {
  int tile, split;
};
__device__ __forceinline__ TileSplit xcd_order(int tiles, int splits) {
  const int g = blockIdx.x + blockIdx.y * gridDim.x;
  const int total = tiles * splits;
  const int v = (total & 7) ? g : (g & 7) * (total >> 3) + (g >> 3);
  return TileSplit{v % tiles, v / tiles};
}

// Decode 8 packed bytes' worth... one 32-bit word = 8 NF4 codes (bytes in
// memory order, even element in the high nibble) into 4 bf16 pairs.
__device__ __forceinline__ void decode_word(uint32_t w, float a, const float* lut, uint32_t out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t byte = (w >> (8 * j)) & 0xFFu;
    float v0 = lut[byte >> 4] * a;
    float v1 = lut[byte & 15u] * a;
    out[j] = pack_bf16x2(v0, v1);
  }
}

// The same decode with the level table in registers: the 16 levels times one
// absmax, rounded to bf16, split into byte planes (the low bytes of levels
// 4g..4g+3 in lo[g], their high bytes in hi[g]).  A code then becomes its bf16
// value through byte permutes (v_perm_b32: selector byte s < 8 takes byte s of
// {src0, src1}, src1 the low word), with no LDS reads; the values are the same
// fp32 products rounded once to bf16 as decode_word gives.
struct NF4Planes {
  uint32_t lo[4], hi[4];
};
__device__ __forceinline__ NF4Planes nf4_planes(float a) {
  NF4Planes p;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t d0 = pack_bf16x2(kNF4LevelsDev[4 * g] * a, kNF4LevelsDev[4 * g + 1] * a);
    const uint32_t d1 = pack_bf16x2(kNF4LevelsDev[4 * g + 2] * a, kNF4LevelsDev[4 * g + 3] * a);
    p.lo[g] = __builtin_amdgcn_perm(d1, d0, 0x06040200u);
    p.hi[g] = __builtin_amdgcn_perm(d1, d0, 0x07050301u);
  }
  return p;
}
// Four codes, one per byte of x, to bf16 pairs (code of byte 0, byte 1) and
// (byte 2, byte 3): each plane is looked up in levels 0-7 and 8-15 with the
// code's low 3 bits, and bit 3 picks which of the two bytes is kept.
__device__ __forceinline__ void nf4_lookup4(const NF4Planes& p, uint32_t x, uint32_t& o01, uint32_t& o23) {
  const uint32_t s = x & 0x07070707u;
  const uint32_t pick = ((x >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(p.lo[3], p.lo[2], s),
                                            __builtin_amdgcn_perm(p.lo[1], p.lo[0], s), pick);
  const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(p.hi[3], p.hi[2], s),
                                            __builtin_amdgcn_perm(p.hi[1], p.hi[0], s), pick);
  o01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  o23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}
// decode_word's output (4 bf16 pairs in element order) from the planes.
__device__ __forceinline__ void decode_word_regs(uint32_t w, const NF4Planes& p, uint32_t out[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;   // odd, even elements
  nf4_lookup4(p, __builtin_amdgcn_perm(hi, lo, 0x01050004u), out[0], out[1]);
  nf4_lookup4(p, __builtin_amdgcn_perm(hi, lo, 0x03070206u), out[2], out[3]);
}

// LoRA up-projection folded into the tile: acc += U_seg B^T, one or more
// extra 32-wide reduction steps (split 0 only).  r0, c0: the wave's first row
// and column.
template <int TM, int TN>
__device__ __forceinline__ void fwd_lora_up(const FwdParams& p, f32x4 (&acc)[TM][TN], int r0, int c0, int lane,
                                            int split) {
  if (p.r <= 0 || split != 0) return;
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col0 = c0 + j * 16;
    if (col0 >= p.N) continue;
    int s = 0;
    while (s + 1 < p.nseg && col0 >= p.seg_end[s]) ++s;
    const int ucol = p.seg_ucol[s];
    const int col = col0 + (lane & 15);
    for (int kc = 0; kc < p.r; kc += 32) {
      const int kk = kc + 8 * g;
      uint4 bv = (col < p.N && kk < p.r) ? *reinterpret_cast<const uint4*>(p.Bl + (int64_t)col * p.r + kk)
                                         : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = r0 + i * 16 + (lane & 15);
        uint4 av = (row < p.M && kk < p.r) ? *reinterpret_cast<const uint4*>(p.U + (int64_t)row * p.ldu + ucol + kk)
                                           : make_uint4(0, 0, 0, 0);
        acc[i][j] = mfma16(u4_as_frag(av), u4_as_frag(bv), acc[i][j]);
      }
    }
  }
}

// Epilogue: lane holds C[4 (lane >> 4) + v][lane & 15] of each 16x16 tile.
// Split-K launches write fp32 partials; otherwise bias, residual and the
// output conversion are applied here.
template <int TM, int TN, int EPI>
__device__ __forceinline__ void fwd_store(const FwdParams& p, const f32x4 (&acc)[TM][TN], int r0, int c0, int lane,
                                          int split) {
  if (p.splits > 1) {
    float* part = p.part + (int64_t)split * p.M * p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = c0 + j * 16 + (lane & 15);
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = r0 + i * 16 + 4 * (lane >> 4) + v;
          if (row < p.M) part[(int64_t)row * p.N + col] = acc[i][j][v];
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = c0 + j * 16 + (lane & 15);
    if (col >= p.N) continue;
    const float bias = p.bias ? bf16_bits_to_f32(p.bias[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + i * 16 + 4 * (lane >> 4) + v;
        if (row >= p.M) continue;
        float val = acc[i][j][v] + bias;
        const int64_t o = (int64_t)row * p.ldc + col;
        if (EPI == EPI_BF16) {
          static_cast<uint16_t*>(p.out)[o] = f32_to_bf16_bits(val);
        } else if (EPI == EPI_F32) {
          static_cast<float*>(p.out)[o] = val;
        } else {
          static_cast<float*>(p.out)[o] = p.resid[o] + val;
        }
      }
    }
  }
}

// Workgroup barrier that waits for this wave's LDS traffic only: global loads
// still in flight (the next k-step's prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// =========================================================== forward (NT)
// C[M, N] = X[M, K] W[N, K]^T + U_seg[M, r] Bl[N, r]^T (+ bias) (+ resid)

// Ping-pong forward: 256 x 256 tile, 8 waves in two groups of 4 (one wave
// per SIMD in each).  Group g owns tile rows [128 g, 128 g + 128) and loads /
// decodes that half of the A and B tiles.  Each k-step has two halves split by
// barriers: in half h, group h runs its MFMAs on the current LDS buffer while
// the other group writes its share of the next k-step into the other buffer
// and issues the global loads of the one after.  A SIMD therefore always has
// one wave feeding the matrix unit and one doing NF4 decode on the VALU.
template <int WKIND, int EPI>
__global__ void __launch_bounds__(512, 1) gemm_fwd_pp_kernel(FwdParams p) {
  constexpr int BM = 256, BN = 256, WM = 64, WN = 128, TM = WM / 16, TN = WN / 16, GT = 256;
  constexpr int A_CH = 128 * 8 / GT;                                  // 16-B A chunks per thread
  constexpr int B_CH = (WKIND == LSQ_W_NF4) ? 128 * 2 / GT : 128 * 8 / GT;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * 64];
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, gtid = tid & (GT - 1);
  const int wm = grp * 2 + ((wave >> 1) & 1), wn = wave & 1;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles_m = (p.M + BM - 1) / BM;
  const TileSplit ts = xcd_order(tiles_m * tiles_n, p.splits);
  const int t = ts.tile;
  const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
  if (tid < 16) lut[tid] = kNF4LevelsDev[tid];

  const int K = p.K, nk_all = K / BK, Kw = p.Kw, nkw = Kw / BK;
  const int split = ts.split;
  const int per = (nk_all + p.splits - 1) / p.splits;
  const int kbeg = min(nk_all, split * per), nk = min(nk_all, kbeg + per);

  uint4 ra[A_CH], rb[B_CH];
  float rabs[B_CH];
  const int arow0 = grp * 128;   // this group's share: rows [arow0, arow0 + 128) of both tiles

  auto load_share = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    int gt = gtid;   // opaque copy: addresses are rebuilt per call, not held in registers
    asm volatile("" : "+v"(gt));
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = gt + i * GT, row = arow0 + (q >> 3), c = q & 7, m = m0 + row;
      ra[i] = (m < p.M) ? *reinterpret_cast<const uint4*>(p.X + (int64_t)m * p.ldx + k0 + c * 8)
                        : make_uint4(0, 0, 0, 0);
    }
    const int kq = kt - (kt >= nkw ? nkw : 0), kq0 = kq * BK;   // the weight's reduction step
    if (WKIND == LSQ_W_NF4) {
      const uint8_t* W = static_cast<const uint8_t*>(p.W);
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int q = gt + i * GT, n = n0 + arow0 + (q >> 1), h = q & 1;
        const bool ok = n < p.N;
        rb[i] = ok ? *reinterpret_cast<const uint4*>(W + (int64_t)n * (Kw / 2) + kq0 / 2 + h * 16)
                   : make_uint4(0, 0, 0, 0);
        rabs[i] = ok ? p.absmax[(int64_t)n * (Kw / 64) + kq] : 0.f;
      }
    } else {
      const uint16_t* W = static_cast<const uint16_t*>(p.W);
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int q = gt + i * GT, n = n0 + arow0 + (q >> 3), c = q & 7;
        rb[i] = (n < p.N) ? *reinterpret_cast<const uint4*>(W + (int64_t)n * Kw + kq0 + c * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_share = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = gtid + i * GT, row = arow0 + (q >> 3), c = q & 7;
      *reinterpret_cast<uint4*>(&As[buf][swz(row, c)]) = ra[i];
    }
    if (WKIND == LSQ_W_NF4) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int q = gtid + i * GT, row = arow0 + (q >> 1), h = q & 1;
        const uint32_t words[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t o[4];
          decode_word(words[w], rabs[i], lut, o);
          *reinterpret_cast<uint4*>(&Bs[buf][swz(row, h * 4 + w)]) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int q = gtid + i * GT, row = arow0 + (q >> 3), c = q & 7;
        *reinterpret_cast<uint4*>(&Bs[buf][swz(row, c)]) = rb[i];
      }
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_step = [&](int cur) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[TM], bfr[TN];
      const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = lds_frag(As[cur], swz(wm * WM + i * 16 + (lane & 15), chunk));
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = lds_frag(Bs[cur], swz(wn * WN + j * 16 + (lane & 15), chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  };

  // Prologue: both groups fill buffer 0 with k-step kbeg and prefetch kbeg + 1.
  if (kbeg < nk) load_share(kbeg);
  __syncthreads();  // lut
  if (kbeg < nk) store_share(0);
  if (kbeg + 1 < nk) load_share(kbeg + 1);
  lds_barrier();

  for (int kt = kbeg; kt < nk; ++kt) {
    const int cur = (kt - kbeg) & 1;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (grp == half) {
        mfma_step(cur);
      } else if (kt + 1 < nk) {
        store_share(cur ^ 1);
        if (kt + 2 < nk) load_share(kt + 2);
      }
      lds_barrier();
    }
  }

  fwd_lora_up<TM, TN>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, split);
  fwd_store<TM, TN, EPI>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, split);
}

// ------------------------------------------------- buffer resources and LDS DMA
// A raw buffer resource over [base, base + bytes): loads past the end return
// zeros, which pads ragged tiles without a compare per load.  Offsets are 32-bit
// bytes, so the host only routes operands below 2 GiB here.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// s_waitcnt vmcnt(N) through the builtin (not inline asm), so that the
// compiler's own wait insertion sees it and knows which DMA writes are done.
// gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ lds_ptr_t as_lds(void* p) { return (lds_ptr_t)(p); }
// Copy 64 lanes x 16 B from the buffer into LDS at lds + 16 * lane (the DMA
// writes LDS without passing through VGPRs; out-of-range chunks land as zeros).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, as_lds(lds), 16, voff, soff, 0, 0);
}

// ============================================ forward, NF4, activations by DMA
// The ping-pong schedule above with the activation tile moved off the VGPR
// path: each wave copies its group's share of the next k-step's X tile
// straight into LDS (buffer loads with the LDS modifier, issued as its MFMA
// half begins and waited for at the end of its decode half), so the decode
// half only unpacks NF4 codes.  It does so from registers (nf4_planes, one
// table per thread and k-step: a thread's 32 codes share one absmax), which
// leaves LDS to the fragment reads, the decoded tile and the DMA; the level
// table lookups were half of this kernel's LDS instructions.  Lane l of a
// DMA fills LDS bytes 16 l of an 8-row block, i.e. row l / 8, swizzled chunk
// slot l % 8; it therefore loads
// logical chunk (l % 8) ^ (row % 8).  The two LDS stages are separate arrays
// and the k loop is unrolled by two so that every access names its stage
// statically (the compiler can then tell DMA writes to one stage from reads of
// the other and does not drain the DMA queue before each fragment read).
//
// BN is the tile's width in output columns (256, or 224 or 192 where 256-wide
// tiles would leave part of a round of 256 workgroups idle, e.g. N = 6144 at
// 2048 rows gives 192 tiles of 256 but 256 of 192).  Each group decodes BN / 2
// weight rows; the spare threads of a narrower tile load a duplicate row and
// skip the store.
//
// PAIR: the input is a hi/lo pair X = [X_hi | X_lo] over one weight (K = 2 Kw).
// Without PAIR the reduction runs over the hi steps, then reads the weight
// again for the lo steps.  With PAIR the steps alternate, hi then lo of the
// same 64-wide weight block, and both read one decoded block: the block of
// the next pair is decoded over the two decode halves of the current pair
// (16 of a thread's 32 codes in each), so the weight is unpacked once for
// two k-steps of matrix work.  A split covers whole pairs.
template <int EPI, int BN, bool PAIR>
__global__ void __launch_bounds__(512, 1) gemm_fwd_nf4_dma_kernel(FwdParams p) {
  static_assert(BN % 32 == 0 && BN <= 256, "two 16-column-aligned wave columns per tile");
  constexpr int BM = 256, WM = 64, WN = BN / 2, TM = WM / 16, TN = WN / 16, GT = 256;
  __shared__ __attribute__((aligned(16))) uint16_t As0[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t As1[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[BN * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs1[BN * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wig = wave & 3, gtid = tid & (GT - 1);
  const int wm = grp * 2 + ((wave >> 1) & 1), wn = wave & 1;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles_m = (p.M + BM - 1) / BM;
  // Column-major tile order: the M tiles that share a weight slab are
  // neighbours, so xcd_order puts them on one XCD and the slab leaves HBM once.
  const TileSplit ts = xcd_order(tiles_m * tiles_n, p.splits);
  const int t = ts.tile;
  const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;

  const int K = p.K, nk_all = K / BK, Kw = p.Kw, nkw = Kw / BK;
  const int split = ts.split;
  const int per = PAIR ? 2 * ((nkw + p.splits - 1) / p.splits) : (nk_all + p.splits - 1) / p.splits;
  const int kbeg = min(nk_all, split * per), nk = min(nk_all, kbeg + per);

  // X rows [m0, M), packed codes and absmax of weight rows [n0, N).
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.X + (int64_t)m0 * p.ldx, (uint32_t)((p.M - m0) * p.ldx * 2));
  const __amdgpu_buffer_rsrc_t rw =
      buffer_rsrc(static_cast<const uint8_t*>(p.W) + (int64_t)n0 * (Kw / 2), (uint32_t)((p.N - n0) * (Kw / 2)));
  const __amdgpu_buffer_rsrc_t rs =
      buffer_rsrc(p.absmax + (int64_t)n0 * (Kw / 64), (uint32_t)((p.N - n0) * (Kw / 64) * 4));

  // This wave's four 8-row blocks of its group's 128 X rows.
  const int xrow0 = grp * 128 + wig * 32;
  const uint32_t x_voff = (uint32_t)(((xrow0 + (lane >> 3)) * p.ldx + (((lane & 7) ^ (lane >> 3)) * 8)) * 2);
  const uint32_t x_blk = (uint32_t)(8 * p.ldx * 2);
  // This thread's 32 codes (row, half of the 64-wide block) and their scale.
  const bool bact = BN == 256 || gtid < BN;
  const int brow = grp * WN + (bact ? (gtid >> 1) : WN - 1), bh = gtid & 1;
  const uint32_t w_voff = (uint32_t)(brow * (Kw / 2) + bh * 16);
  const uint32_t s_voff = (uint32_t)(brow * (Kw / 64) * 4);

  auto dma_x = [&](int kt, uint16_t* as) __attribute__((always_inline)) {
    // PAIR: step kt reads X_hi (even kt) or X_lo (odd kt) of weight block kt / 2
    const uint32_t koff = PAIR ? (uint32_t)((kt & 1) * Kw * 2 + (kt >> 1) * 128) : (uint32_t)(kt * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rx, as + (xrow0 + i * 8) * 64, x_voff, koff + i * x_blk);
  };
  // Two register sets for the prefetched codes, by k-step parity (PAIR: by
  // block parity), so a decode half can issue the loads of the step (block)
  // after next before it unpacks the next one.
  uint4 rb[2];
  float rab[2];
  auto load_blk = [&](int kq, int set) __attribute__((always_inline)) {   // kq: the weight's block
    rb[set] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff, (uint32_t)(kq * 32), 0));
    rab[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, s_voff, (uint32_t)(kq * 4), 0));
  };
  auto load_b = [&](int kt, int set) __attribute__((always_inline)) {
    load_blk(kt - (kt >= nkw ? nkw : 0), set);   // the second pass reads the weight again
  };
  // Decode words [w0, w0 + nw) of the set's 4 (8 codes each) into the tile.
  auto store_words = [&](uint16_t* bs, int set, int w0, int nw) __attribute__((always_inline)) {
    const uint32_t words[4] = {rb[set].x, rb[set].y, rb[set].z, rb[set].w};
    if (!bact) return;
    const NF4Planes pl = nf4_planes(rab[set]);
#pragma unroll
    for (int w = w0; w < w0 + nw; ++w) {
      uint32_t o[4];
      decode_word_regs(words[w], pl, o);
      *reinterpret_cast<uint4*>(&bs[swz(brow, bh * 4 + w)]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  auto store_b = [&](uint16_t* bs, int set) __attribute__((always_inline)) { store_words(bs, set, 0, 4); };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_step = [&](const uint16_t* as, const uint16_t* bs) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[TM], bfr[TN];
      const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = lds_frag(as, swz(wm * WM + i * 16 + (lane & 15), chunk));
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = lds_frag(bs, swz(wn * WN + j * 16 + (lane & 15), chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  };

  // The two halves of a k-step on stage (as, bs) while stage (an, bn) receives
  // k-step kt + 1.  A wave's DMA of X(kt + 1) goes out at the end of its MFMA
  // half, after the half's fragment reads, and is waited for before the
  // barrier that closes its decode half, a full MFMA half later; the only
  // vector-memory operations issued after it are the two B loads of kt + 2.
  // Each group runs its own loop (group 0: MFMA then decode, group 1 the other
  // way round) over pairs of k-steps with no branches inside: loads past the
  // last k-step are clamped to it and land in the stage nobody reads any more.
  // (Straight-line halves also let the compiler see that every DMA is waited
  // for before the stage it wrote is read, so it adds no waits of its own.)
  auto mfma_half = [&](int kt, const uint16_t* as, const uint16_t* bs, uint16_t* an)
      __attribute__((always_inline)) {
    mfma_step(as, bs);
    __builtin_amdgcn_sched_barrier(0);
    dma_x(min(kt + 1, nk - 1), an);
    lds_barrier();
  };
  // set: register set holding k-step kt's codes (parity relative to kbeg);
  // k-step kt + 1 is in the other one.
  auto decode_half = [&](int kt, uint16_t* bn, int set) __attribute__((always_inline)) {
    load_b(min(kt + 2, nk - 1), set);
    store_b(bn, set ^ 1);
    wait_vmcnt<2>();
    lds_barrier();
  };
  // The last k-step of an odd count: no DMA, and the decode half only waits.
  auto last_mfma = [&](const uint16_t* as, const uint16_t* bs) __attribute__((always_inline)) {
    mfma_step(as, bs);
    lds_barrier();
  };
  auto last_wait = [&]() __attribute__((always_inline)) {
    wait_vmcnt<0>();
    lds_barrier();
  };

  if constexpr (PAIR) {
    // Pairs of steps (hi, lo) of one block read one B stage; the block
    // after it is decoded into the other stage over the pair's two decode
    // halves (the first also loads the codes of the block after that), so the
    // loop runs over two pairs, one per B stage.  bl: the split's last block;
    // loads past it are clamped and decoded into the stage nobody reads any
    // more.
    const int bl = (nk - 1) >> 1;
    auto dec_first = [&](uint16_t* bn, int set, int lset, int blk) __attribute__((always_inline)) {
      load_blk(min(blk, bl), lset);
      store_words(bn, set, 0, 2);
      wait_vmcnt<2>();
      lds_barrier();
    };
    auto dec_second = [&](uint16_t* bn, int set) __attribute__((always_inline)) {
      store_words(bn, set, 2, 2);
      wait_vmcnt<0>();
      lds_barrier();
    };
    // Prologue: stage 0 gets block kbeg / 2 and X of step kbeg; registers the next block.
    if (kbeg < nk) {
      dma_x(kbeg, As0);
      load_blk(kbeg >> 1, 0);
    }
    if (kbeg < nk) {
      load_blk(min((kbeg >> 1) + 1, bl), 1);
      store_b(Bs0, 0);
    }
    wait_vmcnt<0>();
    lds_barrier();

    int kt = kbeg;
    if (grp == 0) {
      for (; kt + 3 < nk; kt += 4) {
        mfma_half(kt, As0, Bs0, As1);
        dec_first(Bs1, 1, 0, (kt >> 1) + 2);
        mfma_half(kt + 1, As1, Bs0, As0);
        dec_second(Bs1, 1);
        mfma_half(kt + 2, As0, Bs1, As1);
        dec_first(Bs0, 0, 1, (kt >> 1) + 3);
        mfma_half(kt + 3, As1, Bs1, As0);
        dec_second(Bs0, 0);
      }
      if (kt < nk) {   // one pair left, on stage 0
        mfma_half(kt, As0, Bs0, As1);
        last_wait();
        last_mfma(As1, Bs0);
        last_wait();
      }
    } else {
      for (; kt + 3 < nk; kt += 4) {
        dec_first(Bs1, 1, 0, (kt >> 1) + 2);
        mfma_half(kt, As0, Bs0, As1);
        dec_second(Bs1, 1);
        mfma_half(kt + 1, As1, Bs0, As0);
        dec_first(Bs0, 0, 1, (kt >> 1) + 3);
        mfma_half(kt + 2, As0, Bs1, As1);
        dec_second(Bs0, 0);
        mfma_half(kt + 3, As1, Bs1, As0);
      }
      if (kt < nk) {
        last_wait();
        mfma_half(kt, As0, Bs0, As1);
        last_wait();
        last_mfma(As1, Bs0);
      }
    }
  } else {
    // Prologue: stage 0 gets k-step kbeg (X by DMA, codes decoded), registers kbeg + 1.
    if (kbeg < nk) {
      dma_x(kbeg, As0);
      load_b(kbeg, 0);
    }
    if (kbeg < nk) {
      load_b(min(kbeg + 1, nk - 1), 1);
      store_b(Bs0, 0);
    }
    wait_vmcnt<0>();
    lds_barrier();

    int kt = kbeg;
    if (grp == 0) {
      for (; kt + 1 < nk; kt += 2) {
        mfma_half(kt, As0, Bs0, As1);
        decode_half(kt, Bs1, 0);
        mfma_half(kt + 1, As1, Bs1, As0);
        decode_half(kt + 1, Bs0, 1);
      }
      if (kt < nk) {
        last_mfma(As0, Bs0);
        last_wait();
      }
    } else {
      for (; kt + 1 < nk; kt += 2) {
        decode_half(kt, Bs1, 0);
        mfma_half(kt, As0, Bs0, As1);
        decode_half(kt + 1, Bs0, 1);
        mfma_half(kt + 1, As1, Bs1, As0);
      }
      if (kt < nk) {
        last_wait();
        last_mfma(As0, Bs0);
      }
    }
  }
  wait_vmcnt<0>();   // the clamped DMA / loads of the final pair

  fwd_lora_up<TM, TN>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, split);
  fwd_store<TM, TN, EPI>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, split);
}

// ==================================== forward, bf16 weights, both operands by DMA
// With nothing to decode there is no second half to ping-pong against: all
// eight waves run MFMAs on the 256 x 256 tile (a 64 x 128 wave tile each), and
// each wave copies 32 rows of both the X and the W tile of the next k-step
// into the other LDS stage by DMA while it computes on the current one, with
// one barrier per k-step.  The DMA lane mapping and swizzle are those of the
// NF4 kernel above; the stages are again separate arrays named statically.
template <int EPI>
__global__ void __launch_bounds__(512, 1) gemm_fwd_bf16_dma_kernel(FwdParams p) {
  constexpr int BM = 256, BN = 256, WM = 64, WN = 128, TM = WM / 16, TN = WN / 16;
  __shared__ __attribute__((aligned(16))) uint16_t As0[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t As1[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[BN * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs1[BN * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles_m = (p.M + BM - 1) / BM;
  const TileSplit ts = xcd_order(tiles_m * tiles_n, p.splits);
  const int t = ts.tile;
  const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;

  const int K = p.K, nk_all = K / BK, Kw = p.Kw, nkw = Kw / BK;
  const int split = ts.split;
  const int per = (nk_all + p.splits - 1) / p.splits;
  const int kbeg = min(nk_all, split * per), nk = min(nk_all, kbeg + per);

  // X rows [m0, M) and W rows [n0, N): rows past the end read as zeros.
  const uint16_t* W = static_cast<const uint16_t*>(p.W);
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.X + (int64_t)m0 * p.ldx, (uint32_t)((p.M - m0) * p.ldx * 2));
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + (int64_t)n0 * Kw, (uint32_t)((int64_t)(p.N - n0) * Kw * 2));
  // This wave's four 8-row blocks of each tile: rows [32 wave, 32 wave + 32).
  const int row0 = wave * 32;
  const int lchunk = ((lane & 7) ^ (lane >> 3)) * 8;
  const uint32_t x_voff = (uint32_t)(((row0 + (lane >> 3)) * p.ldx + lchunk) * 2);
  const uint32_t x_blk = (uint32_t)(8 * p.ldx * 2);
  const uint32_t w_voff = (uint32_t)(((row0 + (lane >> 3)) * Kw + lchunk) * 2);
  const uint32_t w_blk = (uint32_t)(8 * Kw * 2);
  auto dma = [&](int kt, uint16_t* as, uint16_t* bs) __attribute__((always_inline)) {
    const int kq = kt - (kt >= nkw ? nkw : 0);   // the weight's reduction step
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rx, as + (row0 + i * 8) * 64, x_voff, (uint32_t)(kt * 128) + i * x_blk);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rw, bs + (row0 + i * 8) * 64, w_voff, (uint32_t)(kq * 128) + i * w_blk);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_step = [&](const uint16_t* as, const uint16_t* bs) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[TM], bfr[TN];
      const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = lds_frag(as, swz(wm * WM + i * 16 + (lane & 15), chunk));
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = lds_frag(bs, swz(wn * WN + j * 16 + (lane & 15), chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  };

  // Stage 0 holds k-step kt at the top of each pair; the DMA into a stage is
  // issued only after the barrier that closed the last reads of it.  A DMA
  // past the last k-step is clamped to it and lands in a stage nobody reads.
  if (kbeg < nk) dma(kbeg, As0, Bs0);
  wait_vmcnt<0>();
  lds_barrier();
  int kt = kbeg;
  // (sched_barrier keeps the compiler from sinking the DMA issue to the end
  // of the MFMAs, right before its wait.)
  for (; kt + 1 < nk; kt += 2) {
    dma(kt + 1, As1, Bs1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(As0, Bs0);
    wait_vmcnt<0>();
    lds_barrier();
    dma(min(kt + 2, nk - 1), As0, Bs0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(As1, Bs1);
    wait_vmcnt<0>();
    lds_barrier();
  }
  if (kt < nk) mfma_step(As0, Bs0);

  fwd_lora_up<TM, TN>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, split);
  fwd_store<TM, TN, EPI>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, split);
}

template <int TM, int TO, int EPI>
__device__ __forceinline__ void bwd_store(const BwdParams& p, const f32x4 (&acc)[TM][TO], int r0, int c0, int lane,
                                          int split);

// =========================================================== backward (NN)
// C[M, K] = dY[M, N] W[N, K] + G[M, rr] Al[rr, K] (+ resid)
// The weight slab (64 rows of W) is decoded straight into a transposed LDS
// tile Bt[k][n] so that each lane's 8 reduction values are contiguous.

// Backward epilogue (lane layout as in fwd_store); columns are the weight's
// input dimension K.
template <int TM, int TO, int EPI>
__device__ __forceinline__ void bwd_store(const BwdParams& p, const f32x4 (&acc)[TM][TO], int r0, int c0, int lane,
                                          int split) {
  const int K = p.K;
  if (p.splits > 1) {
    float* part = p.part + (int64_t)split * p.M * K;
#pragma unroll
    for (int j = 0; j < TO; ++j) {
      const int col = c0 + j * 16 + (lane & 15);
      if (col >= K) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = r0 + i * 16 + 4 * (lane >> 4) + v;
          if (row < p.M) part[(int64_t)row * K + col] = acc[i][j][v];
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TO; ++j) {
    const int col = c0 + j * 16 + (lane & 15);
    if (col >= K) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + i * 16 + 4 * (lane >> 4) + v;
        if (row >= p.M) continue;
        const int64_t o = (int64_t)row * p.ldc + col;
        const float val = acc[i][j][v];
        if (EPI == EPI_BF16) {
          static_cast<uint16_t*>(p.out)[o] = f32_to_bf16_bits(val);
        } else if (EPI == EPI_F32) {
          static_cast<float*>(p.out)[o] = val;
        } else {
          static_cast<float*>(p.out)[o] = p.resid[o] + val;
        }
      }
    }
  }
}

// LoRA term of the backward folded into the tile: acc += G[:, 0:rr] Al, one
// or more extra 32-wide reduction steps (split 0 only), with Al read from its
// transposed copy AlT [K, rr] so each lane's 8 reduction values are contiguous.
template <int TM, int TO>
__device__ __forceinline__ void bwd_lora_up(const BwdParams& p, f32x4 (&acc)[TM][TO], int r0, int c0, int lane,
                                            int split) {
  if (p.rr <= 0 || split != 0) return;
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < TO; ++j) {
    const int col = c0 + j * 16 + (lane & 15);
    for (int kc = 0; kc < p.rr; kc += 32) {
      const int kk = kc + 8 * g;
      const uint4 bv = (col < p.K && kk < p.rr) ? *reinterpret_cast<const uint4*>(p.AlT + (int64_t)col * p.rr + kk)
                                                : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = r0 + i * 16 + (lane & 15);
        const uint4 av = (row < p.M && kk < p.rr) ? *reinterpret_cast<const uint4*>(p.G + (int64_t)row * p.ldg + kk)
                                                  : make_uint4(0, 0, 0, 0);
        acc[i][j] = mfma16(u4_as_frag(av), u4_as_frag(bv), acc[i][j]);
      }
    }
  }
}

// Transposed micro-tile coordinates of the backward weight slab (BO output
// columns x 64 reduction rows): micro-tile u covers rows 4 rg .. 4 rg + 3 and
// columns 8 q .. 8 q + 7; lanes 8 apart in q, neighbouring rg pairs in a pass.
template <int BO>
__device__ __forceinline__ void bwd_mt_coords(int u, int& rg, int& q) {
  q = (u & 7) | (((u >> 4) & ((BO / 8 / 8) - 1)) << 3);
  rg = ((u >> 3) & 1) | ((u >> (4 + __builtin_ctz(BO / 64))) << 1);
}

// Decode (or copy) one micro-tile held in registers and write it transposed
// into Bt: column c of the micro-tile becomes 4 consecutive reduction values.
template <bool NF4, int RB>
__device__ __forceinline__ void bwd_store_mt(uint16_t* Bt, int rg, int q, const uint32_t (&rb)[RB], const float* lut) {
  // rb: NF4 -> codes of rows 0..3 in rb[0..3], their absmax bits in rb[4..7];
  //     bf16 -> rows 0..3 as four 16-byte groups.
  uint32_t pairs[4][4];  // pairs[rr][j] = (col 2j, col 2j+1) of row rr
  if (NF4) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) decode_word(rb[rr], __uint_as_float(rb[4 + rr]), lut, pairs[rr]);
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int w = 0; w < 4; ++w) pairs[rr][w] = rb[(4 * rr + w) % RB];
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int sel = (c & 1) ? 0x07060302 : 0x05040100;  // high or low halves
    const uint32_t lo = __builtin_amdgcn_perm(pairs[1][c >> 1], pairs[0][c >> 1], sel);
    const uint32_t hi = __builtin_amdgcn_perm(pairs[3][c >> 1], pairs[2][c >> 1], sel);
    const int krow = q * 8 + c, nbase = rg * 4;
    *reinterpret_cast<u32x2*>(Bt + swzt(krow, nbase >> 3) + (nbase & 7)) = u32x2{lo, hi};
  }
}

// Ping-pong backward: the forward's schedule over the NN product.  Group g
// runs the MFMAs of rows [128 g, 128 g + 128) and produces half of the next
// k-step: its own dY (or G) rows and half of the weight slab's micro-tiles.
template <int WKIND, int EPI>
__global__ void __launch_bounds__(512, 1) gemm_bwd_pp_kernel(BwdParams p) {
  constexpr int BM = 256, BO = 256, WM = 64, WO = 128, TM = WM / 16, TO = WO / 16, GT = 256;
  constexpr int A_CH = 128 * 8 / GT;           // 16-B dY chunks per thread
  constexpr int MT_TOTAL = (64 / 4) * (BO / 8);
  static_assert(MT_TOTAL == 2 * GT, "one micro-tile per producer thread");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[2][BO * 64];
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, gtid = tid & (GT - 1);
  const int wm = grp * 2 + ((wave >> 1) & 1), wo = wave & 1;
  const int tiles_o = (p.K + BO - 1) / BO;
  const int tiles_m = (p.M + BM - 1) / BM;
  const TileSplit ts = xcd_order(tiles_m * tiles_o, p.splits);
  const int t = ts.tile;
  const int m0 = (t / tiles_o) * BM, o0 = (t % tiles_o) * BO;
  if (tid < 16) lut[tid] = kNF4LevelsDev[tid];

  const int K = p.K;
  const int nk_all = (p.N + BK - 1) / BK;   // the LoRA term is added after the main loop
  const int split = ts.split;
  const int per = (nk_all + p.splits - 1) / p.splits;
  const int kbeg = min(nk_all, split * per), nk = min(nk_all, kbeg + per);

  const int arow0 = grp * 128;
  int mrg, mq;
  bwd_mt_coords<BO>(grp * GT + gtid, mrg, mq);
  constexpr int RB = (WKIND == LSQ_W_NF4) ? 8 : 16;
  uint4 ra[A_CH];
  uint32_t rb[RB];   // the micro-tile: NF4 codes + absmax bits, or bf16 rows (see bwd_store_mt)

  auto load_share = [&](int kt) __attribute__((always_inline)) {
    const int r0 = kt * BK;
    int gt = gtid, lq = mq, lrg = mrg;   // opaque copies: addresses are rebuilt per call, not held
    asm volatile("" : "+v"(gt), "+v"(lq), "+v"(lrg));
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = gt + i * GT, row = arow0 + (q >> 3), c = q & 7;
      const int m = m0 + row, rcol = r0 + c * 8;
      ra[i] = (m < p.M && rcol < p.N) ? *reinterpret_cast<const uint4*>(p.dY + (int64_t)m * p.ldy + rcol)
                                      : make_uint4(0, 0, 0, 0);
    }
    const int kcol = o0 + lq * 8;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int n = r0 + lrg * 4 + rr;
      const bool ok = n < p.N && kcol < K;
      if (WKIND == LSQ_W_NF4) {
        const uint8_t* W = static_cast<const uint8_t*>(p.W);
        rb[rr] = ok ? *reinterpret_cast<const uint32_t*>(W + (int64_t)n * (K / 2) + kcol / 2) : 0u;
        rb[4 + rr] = ok ? __float_as_uint(p.absmax[(int64_t)n * (K / 64) + kcol / 64]) : 0u;
      } else {
        const uint16_t* W = static_cast<const uint16_t*>(p.W);
        const uint4 v = ok ? *reinterpret_cast<const uint4*>(W + (int64_t)n * K + kcol) : make_uint4(0, 0, 0, 0);
        rb[(4 * rr) % RB] = v.x;
        rb[(4 * rr + 1) % RB] = v.y;
        rb[(4 * rr + 2) % RB] = v.z;
        rb[(4 * rr + 3) % RB] = v.w;
      }
    }
  };

  auto store_share = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = gtid + i * GT, row = arow0 + (q >> 3), c = q & 7;
      *reinterpret_cast<uint4*>(&As[buf][swz(row, c)]) = ra[i];
    }
    int q = mq;
    asm volatile("" : "+v"(q));
    bwd_store_mt<WKIND == LSQ_W_NF4, RB>(Bt[buf], mrg, q, rb, lut);
  };

  f32x4 acc[TM][TO];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TO; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_step = [&](int cur) __attribute__((always_inline)) {
    // The transposed tile's swizzle differs per 16-row block; recompute its
    // addresses here (an empty asm hides the base from loop-invariant code
    // motion) instead of holding 16 of them in registers across the loop.
    int brow = wo * WO + (lane & 15);
    asm volatile("" : "+v"(brow));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[TM], bfr[TO];
      const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = lds_frag(As[cur], swz(wm * WM + i * 16 + (lane & 15), chunk));
#pragma unroll
      for (int j = 0; j < TO; ++j) bfr[j] = lds_frag(Bt[cur], swzt(brow + j * 16, chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TO; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  };

  if (kbeg < nk) load_share(kbeg);
  __syncthreads();  // lut
  if (kbeg < nk) store_share(0);
  if (kbeg + 1 < nk) load_share(kbeg + 1);
  lds_barrier();

  for (int kt = kbeg; kt < nk; ++kt) {
    const int cur = (kt - kbeg) & 1;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (grp == half) {
        mfma_step(cur);
      } else if (kt + 1 < nk) {
        store_share(cur ^ 1);
        if (kt + 2 < nk) load_share(kt + 2);
      }
      lds_barrier();
    }
  }
  bwd_lora_up<TM, TO>(p, acc, m0 + wm * WM, o0 + wo * WO, lane, split);
  bwd_store<TM, TO, EPI>(p, acc, m0 + wm * WM, o0 + wo * WO, lane, split);
}

// ============================================ backward, NF4, dY tile by DMA
// The forward DMA kernel's schedule over the NN product dX = dY W: the dY tile
// reaches LDS by DMA, the weight slab's micro-tiles (4 rows of 8 codes each,
// per producer thread) come through buffer loads into two register sets and
// are decoded and written transposed, and the LoRA term G A joins in the
// epilogue.  Weight rows past N read as zeros, which also cancels the dY
// columns past N that the DMA brings in on the last reduction step.
//
// BO is the tile's width in output columns: 256, or 224 where 256-wide tiles
// would leave part of a round of workgroups idle (K = 14336 at 2048 rows: 448
// tiles of 256, two rounds of 256 workgroups with a quarter idle, but 512 of
// 224).  The producer threads keep the 256-wide micro-tile map; those whose
// micro-tile column falls past a narrower tile load a duplicate and skip the
// store.
template <int WK, int EPI, int BO>
__device__ __forceinline__ void gemm_bwd_dma_body(const BwdParams& p) {
  constexpr bool NF4 = WK == LSQ_W_NF4;
  constexpr int BM = 256, WM = 64, WO = BO / 2, TM = WM / 16, TO = WO / 16, GT = 256;
  static_assert(BO % 32 == 0 && BO <= 256, "two 16-column-aligned wave columns per tile");
  static_assert((64 / 4) * (256 / 8) == 2 * GT, "one micro-tile per producer thread at the full width");
  __shared__ __attribute__((aligned(16))) uint16_t As0[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t As1[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bt0[BO * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bt1[BO * 64];
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wig = wave & 3, gtid = tid & (GT - 1);
  const int wm = grp * 2 + ((wave >> 1) & 1), wo = wave & 1;
  const int tiles_o = (p.K + BO - 1) / BO;
  const int tiles_m = (p.M + BM - 1) / BM;
  const TileSplit ts = xcd_order(tiles_m * tiles_o, p.splits);
  const int t = ts.tile;   // column-major, as in the forward
  const int m0 = (t % tiles_m) * BM, o0 = (t / tiles_m) * BO;
  if (NF4 && tid < 16) lut[tid] = kNF4LevelsDev[tid];

  const int K = p.K;
  const int nk_all = (p.N + BK - 1) / BK;
  const int split = ts.split;
  const int per = (nk_all + p.splits - 1) / p.splits;
  const int kbeg = min(nk_all, split * per), nk = min(nk_all, kbeg + per);

  const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(p.dY + (int64_t)m0 * p.ldy, (uint32_t)((p.M - m0) * p.ldy * 2));
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.W, (uint32_t)((int64_t)p.N * (NF4 ? K / 2 : 2 * K)));
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.absmax, (uint32_t)((int64_t)p.N * (K / 64) * 4));

  const int yrow0 = grp * 128 + wig * 32;
  const uint32_t y_voff = (uint32_t)(((yrow0 + (lane >> 3)) * p.ldy + (((lane & 7) ^ (lane >> 3)) * 8)) * 2);
  const uint32_t y_blk = (uint32_t)(8 * p.ldy * 2);
  int mrg, mq;
  bwd_mt_coords<256>(grp * GT + gtid, mrg, mq);
  const bool mact = BO == 256 || mq < BO / 8;
  if (!mact) mq = BO / 8 - 1;
  const int kcol = o0 + mq * 8;
  const uint32_t w_voff = NF4 ? (uint32_t)(mrg * 4 * (K / 2) + kcol / 2) : (uint32_t)((mrg * 4 * K + kcol) * 2);
  const uint32_t s_voff = (uint32_t)((mrg * 4 * (K / 64) + kcol / 64) * 4);
  const uint32_t w_row = NF4 ? (uint32_t)(K / 2) : (uint32_t)(2 * K), w_step = 64 * w_row;
  const uint32_t s_step = (uint32_t)(64 * (K / 64) * 4), s_row = (uint32_t)((K / 64) * 4);

  auto dma_y = [&](int kt, uint16_t* as) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(ry, as + (yrow0 + i * 8) * 64, y_voff, (uint32_t)(kt * 128) + i * y_blk);
  };
  // Per set: NF4, the codes of the micro-tile's 4 rows, then their absmax
  // bits (8 loads); bf16, the 4 rows of 8 values (4 loads of 16 bytes).
  constexpr int RB = NF4 ? 8 : 16, NLOAD = NF4 ? 8 : 4;
  uint32_t rb[2][RB];
  auto load_b = [&](int kt, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if constexpr (NF4) {
        rb[set][rr] = __builtin_amdgcn_raw_buffer_load_b32(rw, w_voff, (uint32_t)kt * w_step + rr * w_row, 0);
        rb[set][4 + rr] = __builtin_amdgcn_raw_buffer_load_b32(rs, s_voff, (uint32_t)kt * s_step + rr * s_row, 0);
      } else {
        const uint4 v = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff, (uint32_t)kt * w_step + rr * w_row, 0));
        rb[set][4 * rr] = v.x;
        rb[set][4 * rr + 1] = v.y;
        rb[set][4 * rr + 2] = v.z;
        rb[set][4 * rr + 3] = v.w;
      }
    }
  };
  auto store_b = [&](uint16_t* bt, int set) __attribute__((always_inline)) {
    int q = mq;
    asm volatile("" : "+v"(q));
    if (mact) bwd_store_mt<NF4, RB>(bt, mrg, q, rb[set], lut);
  };

  f32x4 acc[TM][TO];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TO; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_step = [&](const uint16_t* as, const uint16_t* bt) __attribute__((always_inline)) {
    int brow = wo * WO + (lane & 15);
    asm volatile("" : "+v"(brow));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[TM], bfr[TO];
      const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = lds_frag(as, swz(wm * WM + i * 16 + (lane & 15), chunk));
#pragma unroll
      for (int j = 0; j < TO; ++j) bfr[j] = lds_frag(bt, swzt(brow + j * 16, chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TO; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  };

  // Same half structure as the forward DMA kernel; eight B loads per decode half.
  auto mfma_half = [&](int kt, const uint16_t* as, const uint16_t* bt, uint16_t* an)
      __attribute__((always_inline)) {
    mfma_step(as, bt);
    __builtin_amdgcn_sched_barrier(0);
    dma_y(min(kt + 1, nk - 1), an);
    lds_barrier();
  };
  auto decode_half = [&](int kt, uint16_t* bn, int set) __attribute__((always_inline)) {
    load_b(min(kt + 2, nk - 1), set);
    store_b(bn, set ^ 1);
    wait_vmcnt<NLOAD>();
    lds_barrier();
  };
  auto last_mfma = [&](const uint16_t* as, const uint16_t* bt) __attribute__((always_inline)) {
    mfma_step(as, bt);
    lds_barrier();
  };
  auto last_wait = [&]() __attribute__((always_inline)) {
    wait_vmcnt<0>();
    lds_barrier();
  };

  if (kbeg < nk) {
    dma_y(kbeg, As0);
    load_b(kbeg, 0);
  }
  __syncthreads();  // lut
  if (kbeg < nk) {
    load_b(min(kbeg + 1, nk - 1), 1);
    store_b(Bt0, 0);
  }
  wait_vmcnt<0>();
  lds_barrier();

  int kt = kbeg;
  if (grp == 0) {
    for (; kt + 1 < nk; kt += 2) {
      mfma_half(kt, As0, Bt0, As1);
      decode_half(kt, Bt1, 0);
      mfma_half(kt + 1, As1, Bt1, As0);
      decode_half(kt + 1, Bt0, 1);
    }
    if (kt < nk) {
      last_mfma(As0, Bt0);
      last_wait();
    }
  } else {
    for (; kt + 1 < nk; kt += 2) {
      decode_half(kt, Bt1, 0);
      mfma_half(kt, As0, Bt0, As1);
      decode_half(kt + 1, Bt0, 1);
      mfma_half(kt + 1, As1, Bt1, As0);
    }
    if (kt < nk) {
      last_wait();
      last_mfma(As0, Bt0);
    }
  }
  wait_vmcnt<0>();

  bwd_lora_up<TM, TO>(p, acc, m0 + wm * WM, o0 + wo * WO, lane, split);
  bwd_store<TM, TO, EPI>(p, acc, m0 + wm * WM, o0 + wo * WO, lane, split);
}

template <int EPI, int BO>
__global__ void __launch_bounds__(512, 1) gemm_bwd_nf4_dma_kernel(BwdParams p) {
  gemm_bwd_dma_body<LSQ_W_NF4, EPI, BO>(p);
}
// The same schedule over bf16 weights: each producer thread copies (instead
// of decoding) its 4 x 8 micro-tile and writes it transposed.
template <int EPI>
__global__ void __launch_bounds__(512, 1) gemm_bwd_bf16_dma_kernel(BwdParams p) {
  gemm_bwd_dma_body<LSQ_W_BF16, EPI, 256>(p);
}

__global__ void bf16_to_f32_kernel(const uint16_t* __restrict__ src, int64_t n, float* __restrict__ dst) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) dst[e] = bf16_bits_to_f32(src[e]);
}

// B [N, r] -> Bt [r, N] (bf16), so the G kernel reads 8 reduction values
// contiguously.  One thread per output element: the writes are coalesced and
// the strided reads of the (small) source come from cache.
__global__ void transpose_rows_kernel(const uint16_t* __restrict__ B, int N, int r, uint16_t* __restrict__ Bt) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)N * r) return;
  const int64_t j = e / N, n = e % N;
  Bt[e] = B[n * r + j];
}


// =========================================================== float32 variants
// The float32 tier: dequantized weights are the exact float32 products and
// every product is accumulated in float32, one output per thread in a fixed
// order.  Used for the single-linear float32 checks, not on the hot path.
__device__ __forceinline__ float w_f32(const lsq::WeightRef& W, int n, int k) {
  if (W.kind == LSQ_W_NF4) {
    const uint8_t byte = static_cast<const uint8_t*>(W.data)[(int64_t)n * (W.K / 2) + k / 2];
    const uint32_t code = (k & 1) ? (byte & 15u) : (byte >> 4);
    return kNF4LevelsDev[code] * W.absmax[(int64_t)n * (W.K / 64) + k / 64];
  }
  return bf16_bits_to_f32(static_cast<const uint16_t*>(W.data)[(int64_t)n * W.K + k]);
}

__global__ void f32_lora_down_kernel(const float* X, int M, int K, const float* A, int r, float s, float* U) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= M * r) return;
  int m = e / r, j = e % r;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(X[(int64_t)m * K + k], A[(int64_t)j * K + k], acc);
  U[e] = s * acc;
}

__global__ void f32_linear_fwd_kernel(const float* X, int M, lsq::WeightRef W, const float* U, const float* Bl, int r,
                                      const uint16_t* bias, float* Y) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)M * W.N) return;
  int m = e / W.N, n = e % W.N;
  float acc = 0.f;
  for (int k = 0; k < W.K; ++k) acc = fmaf(X[(int64_t)m * W.K + k], w_f32(W, n, k), acc);
  float lo = 0.f;
  for (int j = 0; j < r; ++j) lo = fmaf(U[(int64_t)m * r + j], Bl[(int64_t)n * r + j], lo);
  Y[e] = acc + lo + (bias ? bf16_bits_to_f32(bias[n]) : 0.f);
}

__global__ void f32_g_kernel(const float* dY, int M, int N, const float* Bl, int r, float s, float* G) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= M * r) return;
  int m = e / r, j = e % r;
  float acc = 0.f;
  for (int n = 0; n < N; ++n) acc = fmaf(dY[(int64_t)m * N + n], Bl[(int64_t)n * r + j], acc);
  G[e] = s * acc;
}

__global__ void f32_linear_dx_kernel(const float* dY, int M, lsq::WeightRef W, const float* G, const float* A, int r,
                                     float* dX) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)M * W.K) return;
  int m = e / W.K, k = e % W.K;
  float acc = 0.f;
  for (int n = 0; n < W.N; ++n) acc = fmaf(dY[(int64_t)m * W.N + n], w_f32(W, n, k), acc);
  float lo = 0.f;
  for (int j = 0; j < r; ++j) lo = fmaf(G[(int64_t)m * r + j], A[(int64_t)j * W.K + k], lo);
  dX[e] = acc + lo;
}

// C[a, b] (+)= sum_m P[m, a] Q[m, b]   (dA = G^T X with P = G; dB = dY^T U with P = dY)
__global__ void f32_tn_kernel(const float* P, int na, const float* Q, int nb, int M, float* C, int accumulate) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)na * nb) return;
  int a = e / nb, b = e % nb;
  float acc = 0.f;
  for (int m = 0; m < M; ++m) acc = fmaf(P[(int64_t)m * na + a], Q[(int64_t)m * nb + b], acc);
  C[e] = accumulate ? C[e] + acc : acc;
}

// out[m, n] = epilogue(sum over splits of part[s, m, n], in split order) (+ bias) (+ resid)
template <int EPI>
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                     const uint16_t* __restrict__ bias, const float* __restrict__ resid,
                                     void* __restrict__ out, int64_t ldc) {
  const int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (e >= total) return;
  const float4 v = split_sum4(part, splits, total, e);
  const int64_t row = e / N, col = e % N;
  float r[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (bias) r[i] += bf16_bits_to_f32(bias[col + i]);
    const int64_t o = row * ldc + col + i;
    if (EPI == EPI_BF16)
      static_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(r[i]);
    else if (EPI == EPI_F32)
      static_cast<float*>(out)[o] = r[i];
    else
      static_cast<float*>(out)[o] = resid[o] + r[i];
  }
}

// The DMA kernels address their operands with 32-bit byte offsets.
bool fwd_dma_ok(const FwdParams& p) {
  const int64_t lim = int64_t(1) << 31;
  return (int64_t)p.M * p.ldx * 2 < lim && (int64_t)p.N * (p.Kw / 2) < lim && p.ldx % 8 == 0;
}
bool fwd_bf16_dma_ok(const FwdParams& p) {
  const int64_t lim = int64_t(1) << 31;
  return (int64_t)p.M * p.ldx * 2 < lim && (int64_t)p.N * p.Kw * 2 < lim && p.ldx % 8 == 0;
}
bool bwd_dma_ok(const BwdParams& p) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t row_bytes = p.kind == LSQ_W_NF4 ? p.K / 2 : 2 * (int64_t)p.K;
  return (int64_t)p.M * p.ldy * 2 < lim && ((int64_t)p.N + 64) * row_bytes < lim && p.ldy % 8 == 0;
}

// The forward kernels take their operands by DMA when they fit 32-bit offsets
// (the NF4 one its activations, the bf16 one both operands); larger operands
// and the backward's bf16 weights use the register-path kernels.
// e0, e1: the timing events attached to the dispatch (null when timing is off).
template <int EPI, bool PAIR>
void launch_fwd_nf4(const FwdParams& p, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.bn == 192)
    hipExtLaunchKernelGGL(gemm_fwd_nf4_dma_kernel<EPI, 192, PAIR>, grid, block, 0, s, e0, e1, 0, p);
  else if (p.bn == 224)
    hipExtLaunchKernelGGL(gemm_fwd_nf4_dma_kernel<EPI, 224, PAIR>, grid, block, 0, s, e0, e1, 0, p);
  else
    hipExtLaunchKernelGGL(gemm_fwd_nf4_dma_kernel<EPI, 256, PAIR>, grid, block, 0, s, e0, e1, 0, p);
}

template <int WK, int EPI>
void launch_fwd(const FwdParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int tiles = ((p.M + kTile - 1) / kTile) * ((p.N + p.bn - 1) / p.bn);
  const dim3 grid(tiles, p.splits), block(512);
  if (WK == LSQ_W_BF16 && fwd_bf16_dma_ok(p))
    hipExtLaunchKernelGGL(gemm_fwd_bf16_dma_kernel<EPI>, grid, block, 0, s, e0, e1, 0, p);
  else if (WK != LSQ_W_NF4 || !fwd_dma_ok(p))
    hipExtLaunchKernelGGL(gemm_fwd_pp_kernel<WK, EPI>, grid, block, 0, s, e0, e1, 0, p);
  else if constexpr (EPI == EPI_F32) {
    if (p.Kw != p.K)   // the hi/lo pair of the q/k/v product
      launch_fwd_nf4<EPI, true>(p, grid, block, s, e0, e1);
    else
      launch_fwd_nf4<EPI, false>(p, grid, block, s, e0, e1);
  } else {
    launch_fwd_nf4<EPI, false>(p, grid, block, s, e0, e1);
  }
}

template <int WK, int EPI>
void launch_bwd(const BwdParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int tiles = ((p.M + kTile - 1) / kTile) * ((p.K + p.bo - 1) / p.bo);
  const dim3 grid(tiles, p.splits), block(512);
  if (WK == LSQ_W_NF4 && bwd_dma_ok(p) && p.bo == 224)
    hipExtLaunchKernelGGL(gemm_bwd_nf4_dma_kernel<EPI, 224>, grid, block, 0, s, e0, e1, 0, p);
  else if (WK == LSQ_W_NF4 && bwd_dma_ok(p))
    hipExtLaunchKernelGGL(gemm_bwd_nf4_dma_kernel<EPI, 256>, grid, block, 0, s, e0, e1, 0, p);
  else if (WK == LSQ_W_BF16 && bwd_dma_ok(p))
    hipExtLaunchKernelGGL(gemm_bwd_bf16_dma_kernel<EPI>, grid, block, 0, s, e0, e1, 0, p);
  else
    hipExtLaunchKernelGGL(gemm_bwd_pp_kernel<WK, EPI>, grid, block, 0, s, e0, e1, 0, p);
}

void launch_reduce(const float* part, int splits, int M, int N, const uint16_t* bias, const float* resid, void* out,
                   int64_t ldc, int epi, hipStream_t s) {
  const int64_t n4 = ((int64_t)M * N) / 4;
  const unsigned grid = (unsigned)((n4 + 255) / 256);
  if (epi == EPI_BF16)
    splitk_reduce_kernel<EPI_BF16><<<grid, 256, 0, s>>>(part, splits, M, N, bias, resid, out, ldc);
  else if (epi == EPI_F32)
    splitk_reduce_kernel<EPI_F32><<<grid, 256, 0, s>>>(part, splits, M, N, bias, resid, out, ldc);
  else
    splitk_reduce_kernel<EPI_F32_RESID><<<grid, 256, 0, s>>>(part, splits, M, N, bias, resid, out, ldc);
}

template <int WK>
void dispatch_fwd_epi(const FwdParams& p, int epi, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (epi == EPI_BF16) launch_fwd<WK, EPI_BF16>(p, s, e0, e1);
  else if (epi == EPI_F32) launch_fwd<WK, EPI_F32>(p, s, e0, e1);
  else launch_fwd<WK, EPI_F32_RESID>(p, s, e0, e1);
}

template <int WK>
void dispatch_bwd_epi(const BwdParams& p, int epi, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (epi == EPI_BF16) launch_bwd<WK, EPI_BF16>(p, s, e0, e1);
  else if (epi == EPI_F32) launch_bwd<WK, EPI_F32>(p, s, e0, e1);
  else launch_bwd<WK, EPI_F32_RESID>(p, s, e0, e1);
}

}  // namespace

// ------------------------------------------------------------------ launchers
// Tile width and split count of a launch from a small cost model.  A launch
// runs in rounds of 256 workgroups (one tile per CU), each round as long as
// its split's reduction steps at ~40% of one CU's MFMA peak for a 256-wide
// tile; a narrower tile (224 or 192 output columns, NF4 DMA kernels only)
// does proportionally less per step except for the activation DMA (about
// 15%); every extra split writes and re-reads an fp32 partial of the whole
// output, priced at 4 TB/s.  A split must win by 3% and a narrower tile by
// 5% (on gfx950 the clock rises a little when CUs idle in a partly filled
// round).  Examples: N = 28672 at 512 rows, 224 tiles of 256 but 256 of 224;
// at 2048 rows 3.5 rounds of 256 but 4 full rounds of 224; N = 6144 at 2048
// rows, 192 tiles of 256 but 256 of 192; the q/k/v product at 512 rows (a
// 128-step reduction over the hi/lo input), 240 workgroups of 256 split 5
// ways but 256 of 192 split 4 ways.  The width never changes a result (every
// output element sums the same products in the same order); the split count
// sets the order of the final fp32 sums.
static GemmPlan plan_tiles(int tm, int n_cols, int ksteps, double out_elems, int narrowest) {
  const double step_us = 2.0 * kTile * kTile * BK / (0.4 * 2.5e15 / 256) * 1e6;
  GemmPlan best{kTile, 1};
  double best_t = 1e30;
  for (int w : {kTile, 224, 192}) {
    if (w < narrowest) break;
    const double work = 0.15 + 0.85 * w / kTile, need = w == kTile ? 0.97 : 0.95;
    for (int sp = 1; sp <= 8; ++sp) {
      if (sp > 1 && ksteps / sp < 4) break;
      const double rounds = (double)((tm * ((n_cols + w - 1) / w) * sp + 255) / 256);
      const double steps = (double)((ksteps + sp - 1) / sp);
      const double t = rounds * steps * step_us * work + (sp > 1 ? 8.0 * sp * out_elems / 4e6 : 0.0);
      if (t < best_t * need) {
        best_t = t;
        best = GemmPlan{w, sp};
      }
    }
  }
  return best;
}

GemmPlan gemm_fwd_plan(int M, int N, int K, bool narrow) {
  return plan_tiles((M + kTile - 1) / kTile, N, K / 64, (double)M * N, narrow ? 192 : kTile);
}
GemmPlan gemm_bwd_plan(int M, int N, int K, bool narrow) {
  return plan_tiles((M + kTile - 1) / kTile, K, (N + 63) / 64, (double)M * K, narrow ? 224 : kTile);
}
// Workspace of gemm_bwd: the split-K partials, for whichever kernel the
// launch can take.
static size_t gemm_bwd_part_bytes(int M, int N, int K) {
  const int sp = std::max(gemm_bwd_plan(M, N, K, true).splits, gemm_bwd_plan(M, N, K, false).splits);
  return sp > 1 ? ((size_t)sp * M * K * sizeof(float) + 255) / 256 * 256 : 0;
}
size_t gemm_fwd_ws_bytes(int M, int N, int K) {
  const int sp = std::max(gemm_fwd_plan(M, N, K, true).splits, gemm_fwd_plan(M, N, K, false).splits);
  return sp > 1 ? (size_t)sp * M * N * sizeof(float) : 0;
}
size_t gemm_bwd_ws_bytes(int M, int N, int K, int rr) {
  (void)rr;   // the LoRA term is added after the main loop, outside the split reduction
  return gemm_bwd_part_bytes(M, N, K);
}

int gemm_fwd(const FwdParams& p_in, int epi, hipStream_t s, void* ws, size_t ws_bytes, int* deferred_splits) {
  FwdParams p = p_in;
  LSQ_CHECK(p.K % 64 == 0, LSQ_ERR_SHAPE, "gemm: K=%d must be a multiple of 64", p.K);
  if (p.Kw == 0) p.Kw = p.K;
  LSQ_CHECK(p.Kw == p.K || 2 * p.Kw == p.K, LSQ_ERR_SHAPE, "gemm: the weight is read once or twice along K");
  LSQ_CHECK(p.r == 0 || (p.r % 8 == 0 && p.ldu % 8 == 0), LSQ_ERR_SHAPE, "gemm: LoRA rank must be a multiple of 8");
  if (p.M == 0 || p.N == 0) return LSQ_OK;
  const GemmPlan plan = gemm_fwd_plan(p.M, p.N, p.K, p.kind == LSQ_W_NF4 && fwd_dma_ok(p));
  p.bn = plan.bn;
  p.splits = plan.splits;
  if (p.splits > 1) {
    LSQ_CHECK(ws && ws_bytes >= gemm_fwd_ws_bytes(p.M, p.N, p.K) && p.N % 4 == 0, LSQ_ERR_WORKSPACE,
              "gemm_fwd: split-K needs %zu bytes of workspace", gemm_fwd_ws_bytes(p.M, p.N, p.K));
    p.part = static_cast<float*>(ws);
  }
  // algorithmic work of the product itself (a hi/lo input is two passes over one product)
  const double flops = 2.0 * p.M * p.N * (double)p.Kw + 2.0 * p.M * (double)p.N * p.r;
  const double wbytes = (p.kind == LSQ_W_NF4 ? 0.5625 : 2.0) * p.N * (double)p.Kw;
  const double bytes = wbytes + 2.0 * p.M * p.K + (epi == EPI_BF16 ? 2.0 : (epi == EPI_F32 ? 4.0 : 8.0)) * p.M * (double)p.N;
  // The profiler times the tile kernel alone (events on its dispatch); a split-K
  // reduction is credited separately.
  hipEvent_t e0, e1;
  int tok = prof_begin_kernel(&e0, &e1);
  if (p.kind == LSQ_W_NF4) dispatch_fwd_epi<LSQ_W_NF4>(p, epi, s, e0, e1);
  else dispatch_fwd_epi<LSQ_W_BF16>(p, epi, s, e0, e1);
  prof_end_kernel(tok, p.kind == LSQ_W_NF4 ? PROF_GEMM_FWD : PROF_GEMM_BF16, flops, bytes);
  if (deferred_splits) *deferred_splits = p.splits;
  if (p.splits > 1 && !deferred_splits) {
    tok = prof_begin(s);
    launch_reduce(p.part, p.splits, p.M, p.N, p.bias, p.resid, p.out, p.ldc, epi, s);
    prof_end(tok, s, PROF_OTHER, 0.0, 4.0 * p.splits * p.M * (double)p.N + 2.0 * p.M * (double)p.N);
  }
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int gemm_bwd(const BwdParams& p_in, int epi, hipStream_t s, void* ws, size_t ws_bytes, int* deferred_splits) {
  BwdParams p = p_in;
  LSQ_CHECK(p.K % 64 == 0, LSQ_ERR_SHAPE, "gemm: K=%d must be a multiple of 64", p.K);
  LSQ_CHECK(p.N % 8 == 0 && p.rr % 8 == 0 && p.ldy % 8 == 0 && p.ldg % 8 == 0, LSQ_ERR_SHAPE,
            "gemm_bwd: N=%d and rank %d must be multiples of 8", p.N, p.rr);
  if (p.M == 0 || p.K == 0) return LSQ_OK;
  const GemmPlan plan = gemm_bwd_plan(p.M, p.N, p.K, p.kind == LSQ_W_NF4 && bwd_dma_ok(p));
  p.bo = plan.bn;
  p.splits = plan.splits;
  const size_t need = gemm_bwd_ws_bytes(p.M, p.N, p.K, p.rr);
  LSQ_CHECK(need == 0 || (ws && ws_bytes >= need), LSQ_ERR_WORKSPACE, "gemm_bwd: needs %zu bytes of workspace",
            need);
  LSQ_CHECK(p.rr == 0 || p.AlT, LSQ_ERR_INVALID, "gemm_bwd: the LoRA term needs the transposed A");
  if (p.splits > 1) p.part = static_cast<float*>(ws);
  const double flops = 2.0 * p.M * p.N * (double)p.K + 2.0 * p.M * (double)p.rr * p.K;
  const double wbytes = (p.kind == LSQ_W_NF4 ? 0.5625 : 2.0) * p.N * (double)p.K;
  const double bytes = wbytes + 2.0 * p.M * p.N + (epi == EPI_BF16 ? 2.0 : (epi == EPI_F32 ? 4.0 : 8.0)) * p.M * (double)p.K;
  hipEvent_t e0, e1;
  int tok = prof_begin_kernel(&e0, &e1);
  if (p.kind == LSQ_W_NF4) dispatch_bwd_epi<LSQ_W_NF4>(p, epi, s, e0, e1);
  else dispatch_bwd_epi<LSQ_W_BF16>(p, epi, s, e0, e1);
  prof_end_kernel(tok, p.kind == LSQ_W_NF4 ? PROF_GEMM_BWD : PROF_GEMM_BF16, flops, bytes);
  if (deferred_splits) *deferred_splits = p.splits;
  if (p.splits > 1 && !deferred_splits) {
    tok = prof_begin(s);
    launch_reduce(p.part, p.splits, p.M, p.K, nullptr, p.resid, p.out, p.ldc, epi, s);
    prof_end(tok, s, PROF_OTHER, 0.0, 4.0 * p.splits * p.M * (double)p.K + 2.0 * p.M * (double)p.K);
  }
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

}  // namespace lsq

// ================================================================== C ABI
namespace {
using namespace lsq;

int check_weight(const lsq_weight* W) {
  LSQ_CHECK(W && W->data, LSQ_ERR_INVALID, "weight: null");
  LSQ_CHECK(W->kind == LSQ_W_NF4 || W->kind == LSQ_W_BF16, LSQ_ERR_INVALID, "weight: bad kind %d", W->kind);
  LSQ_CHECK(W->kind == LSQ_W_BF16 || W->absmax, LSQ_ERR_INVALID, "weight: NF4 needs absmax");
  LSQ_CHECK(W->n_out > 0 && W->n_in > 0 && W->n_in % 64 == 0 && W->n_out < (1 << 30) && W->n_in < (1 << 30),
            LSQ_ERR_SHAPE, "weight: n_in must be a positive multiple of 64 (got %lld x %lld)", (long long)W->n_out,
            (long long)W->n_in);
  LSQ_CHECK(aligned16(W->data) && (!W->absmax || aligned16(W->absmax)), LSQ_ERR_ALIGN, "weight: unaligned pointer");
  return LSQ_OK;
}

WeightRef ref_of(const lsq_weight* W) {
  return WeightRef{W->kind, W->data, W->absmax, (int)W->n_out, (int)W->n_in};
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of one linear call, carved in a fixed order (base null: sizes only).
struct LinWs {
  void* U;            // [M, r] in dtype: U (recomputed or forward scratch)
  void* G;            // [M, r] in dtype
  float* U32;         // [M, r] float32 (bf16 dtype): the unrounded U and G
  float* G32;
  float* lw;          // partials of the down / G projections
  size_t lw_bytes;
  float* gw;          // partials of the adapter-gradient reduction
  size_t gw_bytes;
  uint16_t* Bt;       // B^T [r, N]
  uint16_t* At;       // A^T [K, r]
  int* cnt;           // arrival counters
  int ncnt;
  void* part;         // split-K partials of the GEMM
  size_t part_bytes;
  size_t total;
};
LinWs carve_lin(void* base, int M, int N, int K, int r, int dtype) {
  LinWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* q = base ? p + off : nullptr;
    off += align256(std::max<size_t>(bytes, 1));
    return q;
  };
  const size_t el = dtype == LSQ_F32 ? 4 : 2;
  w.U = take((size_t)M * r * el);
  w.G = take((size_t)M * r * el);
  if (dtype != LSQ_F32) {
    w.U32 = static_cast<float*>(take((size_t)M * r * 4));
    w.G32 = static_cast<float*>(take((size_t)M * r * 4));
    w.lw_bytes = std::max(lora_down_ws_bytes(M, K, r), lora_g_ws_bytes(M, N, r));
    w.lw = static_cast<float*>(take(w.lw_bytes));
    const int se[1] = {N};
    w.gw_bytes = lora_grads_ws_bytes(K, r, 1, se, M);
    w.gw = static_cast<float*>(take(w.gw_bytes));
    w.Bt = static_cast<uint16_t*>(take((size_t)N * r * 2));
    w.At = static_cast<uint16_t*>(take((size_t)K * r * 2));
    w.ncnt = std::max({lora_down_counters(M), lora_g_counters(M, 1), lora_grads_counters(K, r, 1, se)});
    w.cnt = static_cast<int*>(take(counters_bytes(w.ncnt)));
  }
  w.part_bytes = std::max(gemm_fwd_ws_bytes(M, N, K), gemm_bwd_ws_bytes(M, N, K, r));
  w.part = take(w.part_bytes);
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

size_t nf4_lora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dtype) {
  return carve_lin(nullptr, (int)M, (int)N, (int)K, r, dtype).total + 256;
}

int nf4_lora_linear_fwd(const lsq_weight* W, const void* bias, const void* X, int64_t M, const void* A,
                        const void* B, int32_t r, float scale, int32_t dtype, void* Y, void* U_out, void* ws,
                        size_t ws_bytes, void* stream) {
  if (int e = check_weight(W)) return e;
  LSQ_CHECK(dtype == LSQ_F32 || W->n_out % 8 == 0, LSQ_ERR_SHAPE,
            "linear: the bf16 kernels need n_out to be a multiple of 8 (got %lld)", (long long)W->n_out);
  LSQ_CHECK(X && A && B && Y, LSQ_ERR_INVALID, "linear_fwd: null pointer");
  LSQ_CHECK(dtype == LSQ_BF16 || dtype == LSQ_F32, LSQ_ERR_INVALID, "linear_fwd: bad dtype");
  LSQ_CHECK(M >= 0 && M < (1 << 30) && r >= 8 && r <= 64 && r % 8 == 0, LSQ_ERR_SHAPE,
            "linear_fwd: need 0 <= M, r in {8, 16, ..., 64} (got M=%lld r=%d)", (long long)M, r);
  LSQ_CHECK(aligned16(X) && aligned16(A) && aligned16(B) && aligned16(Y) && (!U_out || aligned16(U_out)) &&
                (!bias || aligned16(bias)) && (!ws || aligned16(ws)),
            LSQ_ERR_ALIGN, "linear_fwd: unaligned pointer");
  const size_t need = nf4_lora_linear_workspace_size(M, W->n_out, W->n_in, r, dtype);
  LSQ_CHECK(ws && ws_bytes >= need, LSQ_ERR_WORKSPACE, "linear_fwd: workspace too small");
  hipStream_t s = as_stream(stream);
  const WeightRef w = ref_of(W);
  if (M == 0) return LSQ_OK;   // no tokens: nothing to write
  const int Mi = (int)M;
  if (dtype == LSQ_F32) {
    float* U = U_out ? static_cast<float*>(U_out) : static_cast<float*>(ws);
    f32_lora_down_kernel<<<(Mi * r + 255) / 256, 256, 0, s>>>(static_cast<const float*>(X), Mi, w.K,
                                                             static_cast<const float*>(A), r, scale, U);
    const int64_t n = (int64_t)Mi * w.N;
    if (n > 0)
      f32_linear_fwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<const float*>(X), Mi, w, U,
                                                                       static_cast<const float*>(B), r,
                                                                       static_cast<const uint16_t*>(bias),
                                                                       static_cast<float*>(Y));
    LSQ_HIP(hipGetLastError());
    return LSQ_OK;
  }
  const LinWs lw = carve_lin(ws, Mi, w.N, w.K, r, dtype);
  uint16_t* U = U_out ? static_cast<uint16_t*>(U_out) : static_cast<uint16_t*>(lw.U);
  if (int e = zero_counters(lw.cnt, lw.ncnt, s)) return e;
  if (int e = lora_down(static_cast<const uint16_t*>(X), w.K, Mi, w.K, static_cast<const uint16_t*>(A), r, scale, U,
                        r, nullptr, 0, lw.lw, lw.lw_bytes, lw.cnt, s))
    return e;
  FwdParams p{};
  p.X = static_cast<const uint16_t*>(X);
  p.ldx = w.K;
  p.kind = w.kind;
  p.W = w.data;
  p.absmax = w.absmax;
  p.M = Mi;
  p.N = w.N;
  p.K = w.K;
  p.U = U;
  p.ldu = r;
  p.Bl = static_cast<const uint16_t*>(B);
  p.r = r;
  p.nseg = 1;
  p.seg_end[0] = w.N;
  p.seg_ucol[0] = 0;
  p.bias = static_cast<const uint16_t*>(bias);
  p.out = Y;
  p.ldc = w.N;
  return gemm_fwd(p, EPI_BF16, s, lw.part, lw.part_bytes);
}

int nf4_lora_linear_bwd(const lsq_weight* W, const void* X, const void* U_in, int64_t M, const void* A,
                        const void* B, int32_t r, float scale, int32_t dtype, const void* dY, void* dX, float* dA,
                        float* dB, int32_t accumulate, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_weight(W)) return e;
  LSQ_CHECK(dtype == LSQ_F32 || W->n_out % 8 == 0, LSQ_ERR_SHAPE,
            "linear: the bf16 kernels need n_out to be a multiple of 8 (got %lld)", (long long)W->n_out);
  LSQ_CHECK(X && A && B && dY && dX && dA && dB, LSQ_ERR_INVALID, "linear_bwd: null pointer");
  LSQ_CHECK(dtype == LSQ_BF16 || dtype == LSQ_F32, LSQ_ERR_INVALID, "linear_bwd: bad dtype");
  LSQ_CHECK(M >= 0 && M < (1 << 30) && r >= 8 && r <= 64 && r % 8 == 0, LSQ_ERR_SHAPE, "linear_bwd: bad M or r");
  LSQ_CHECK(aligned16(X) && aligned16(A) && aligned16(B) && aligned16(dY) && aligned16(dX) && aligned16(dA) &&
                aligned16(dB) && (!U_in || aligned16(U_in)) && (!ws || aligned16(ws)),
            LSQ_ERR_ALIGN, "linear_bwd: unaligned pointer");
  const size_t need = nf4_lora_linear_workspace_size(M, W->n_out, W->n_in, r, dtype);
  LSQ_CHECK(ws && ws_bytes >= need, LSQ_ERR_WORKSPACE, "linear_bwd: workspace %zu < %zu", ws_bytes, need);
  hipStream_t s = as_stream(stream);
  const WeightRef w = ref_of(W);
  if (M == 0) {   // no tokens: zero adapter gradients, or leave them when accumulating
    if (accumulate) return LSQ_OK;
    if (int e = zero_words(dA, w.K, r, w.K, s)) return e;
    return zero_words(dB, r, w.N, r, s);
  }
  const int Mi = (int)M;
  const LinWs lw = carve_lin(ws, Mi, w.N, w.K, r, dtype);
  void* Uw = lw.U;
  void* Gw = lw.G;
  float* U32 = lw.U32;
  float* G32 = lw.G32;

  if (dtype == LSQ_F32) {
    const float* U = static_cast<const float*>(U_in);
    if (!U) {
      f32_lora_down_kernel<<<(Mi * r + 255) / 256, 256, 0, s>>>(static_cast<const float*>(X), Mi, w.K,
                                                               static_cast<const float*>(A), r, scale,
                                                               static_cast<float*>(Uw));
      U = static_cast<const float*>(Uw);
    }
    float* G = static_cast<float*>(Gw);
    f32_g_kernel<<<(Mi * r + 255) / 256, 256, 0, s>>>(static_cast<const float*>(dY), Mi, w.N,
                                                     static_cast<const float*>(B), r, scale, G);
    const int64_t nx = (int64_t)Mi * w.K;
    if (nx > 0)
      f32_linear_dx_kernel<<<(unsigned)((nx + 255) / 256), 256, 0, s>>>(static_cast<const float*>(dY), Mi, w, G,
                                                                        static_cast<const float*>(A), r,
                                                                        static_cast<float*>(dX));
    f32_tn_kernel<<<(unsigned)((r * w.K + 255) / 256), 256, 0, s>>>(G, r, static_cast<const float*>(X), w.K, Mi, dA,
                                                                    accumulate);
    f32_tn_kernel<<<(unsigned)((w.N * r + 255) / 256), 256, 0, s>>>(static_cast<const float*>(dY), w.N, U, r, Mi, dB,
                                                                    accumulate);
    LSQ_HIP(hipGetLastError());
    return LSQ_OK;
  }
  if (int e = zero_counters(lw.cnt, lw.ncnt, s)) return e;
  {   // B^T [r, N] for the G projection and A^T [K, r] for the LoRA term of dX
    const int64_t nb = (int64_t)w.N * r, na = (int64_t)r * w.K;
    int tok = prof_begin(s);
    transpose_rows_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(B), w.N, r, lw.Bt);
    transpose_rows_kernel<<<(unsigned)((na + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(A), r, w.K, lw.At);
    prof_end(tok, s, PROF_OTHER, 0.0, 4.0 * (nb + na));
  }
  if (U_in) {
    // the caller's bf16 U: its float32 image feeds dB (no unrounded copy exists)
    const int64_t nu = (int64_t)Mi * r;
    if (nu > 0) bf16_to_f32_kernel<<<(unsigned)((nu + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(U_in), nu, U32);
  } else {
    if (int e = lora_down(static_cast<const uint16_t*>(X), w.K, Mi, w.K, static_cast<const uint16_t*>(A), r, scale,
                          static_cast<uint16_t*>(Uw), r, U32, r, lw.lw, lw.lw_bytes, lw.cnt, s))
      return e;
  }
  uint16_t* G = static_cast<uint16_t*>(Gw);
  SegEnds segs{};
  segs.end[0] = w.N;
  if (int e = lora_g(static_cast<const uint16_t*>(dY), w.N, Mi, w.N, lw.Bt, r, 1, segs, scale, G, r, G32, r, lw.lw,
                     lw.lw_bytes, lw.cnt, s))
    return e;
  BwdParams p{};
  p.dY = static_cast<const uint16_t*>(dY);
  p.ldy = w.N;
  p.kind = w.kind;
  p.W = w.data;
  p.absmax = w.absmax;
  p.M = Mi;
  p.N = w.N;
  p.K = w.K;
  p.G = G;
  p.ldg = r;
  p.Al = static_cast<const uint16_t*>(A);
  p.AlT = lw.At;
  p.rr = r;
  p.out = dX;
  p.ldc = w.K;
  if (int e = gemm_bwd(p, EPI_BF16, s, lw.part, lw.part_bytes)) return e;
  GradGroup g{};
  g.G = G32;
  g.ldg = r;
  g.U = U32;
  g.ldu = r;
  g.X = static_cast<const uint16_t*>(X);
  g.ldx = w.K;
  g.dY = static_cast<const uint16_t*>(dY);
  g.ldy = w.N;
  g.Kx = w.K;
  g.r = r;
  g.nseg = 1;
  g.seg_end[0] = w.N;
  g.gA = dA;
  g.gB = dB;
  return lora_grads(g, Mi, accumulate, lw.gw, lw.gw_bytes, lw.cnt, s);
}

// ------------------------------------------------------------ without a workspace
// The scratch of nf4_lora_linear_bwd_noalloc: one static array per GPU (each
// device holds its own copy from module load until the process ends).  In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, taken once per device on the
// first call there (with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[LSQ_NOALLOC_SCRATCH_BYTES];

static int scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;   // per device
  int dev = 0;
  LSQ_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    LSQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    LSQ_CHECK(p, LSQ_ERR_HIP, "nf4_lora_linear_bwd_noalloc: no device address for the scratch array");
    addr[dev] = p;
  }
  *out = addr[dev];
  return LSQ_OK;
}

int nf4_lora_linear_bwd_noalloc(const lsq_weight* W, const void* X, const void* U, int64_t M, const void* A,
                                const void* B, int32_t r, float scale, int32_t dtype, const void* dY, void* dX,
                                float* dA, float* dB, int32_t accumulate, void* stream) {
  if (int e = check_weight(W)) return e;
  LSQ_CHECK(M >= 0 && M < (1 << 30) && r >= 8 && r <= 64 && r % 8 == 0, LSQ_ERR_SHAPE,
            "linear_bwd_noalloc: bad M or r");
  const size_t need = nf4_lora_linear_workspace_size(M, W->n_out, W->n_in, r, dtype);
  LSQ_CHECK(need <= LSQ_NOALLOC_SCRATCH_BYTES, LSQ_ERR_WORKSPACE,
            "linear_bwd_noalloc: this shape needs %zu bytes of scratch, above the static %llu (use "
            "nf4_lora_linear_bwd with a workspace)", need, (unsigned long long)LSQ_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int e = scratch_address(&ws)) return e;
  // the arrival counters in it are zeroed by a kernel inside the call; nothing else must start at zero
  return nf4_lora_linear_bwd(W, X, U, M, A, B, r, scale, dtype, dY, dX, dA, dB, accumulate, ws,
                             LSQ_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
