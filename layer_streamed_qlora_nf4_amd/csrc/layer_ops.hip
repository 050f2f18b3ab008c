// Per-layer kernels around the linears: RMSNorm, rotary embedding, causal
// GQA attention, SwiGLU, embedding gather and the next-token cross-entropy.
//
// The streamed layer is the model family's own decoder layer (LS-docs "How
// it works": transformers' classes); the maths of each piece is the Llama /
// Qwen2 one.  The residual stream is kept in float32 between kernels; the
// GEMM operands are bf16.  Every reduction has a fixed order (no atomics), so
// a resident and a streamed run of the same shapes give identical bits.
#include <math.h>

#include "common.h"
#include "layer_ops.h"

#include <algorithm>
#include <cfloat>
#include <utility>

namespace lsq {
namespace {

// Reductions over the 16 lanes of a DPP row (lanes 16 g .. 16 g + 15): the
// value rotated within the row by 8, 4, 2 and 1 lanes (DPP row_ror, a VALU
// operand modifier, no LDS round trip).  At each step lane i and the lane it
// reads hold the same two partial sums, so every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kRowRor2 = 0x122, kRowRor1 = 0x121;
__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_row<kRowRor8>(v);
  v += dpp_row<kRowRor4>(v);
  v += dpp_row<kRowRor2>(v);
  return v + dpp_row<kRowRor1>(v);
}

// Sum over the wave: within each 16-lane row by DPP, then across the four
// rows by two lane swaps (every lane ends with the same bits).
__device__ __forceinline__ float warp_sum(float v) {
  v = group16_sum(v);
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// ------------------------------------------------------------------ RMSNorm
// One workgroup (4 waves) per row, the row held in registers: each thread
// owns float4 groups tid, tid + 256, ... (up to 8, i.e. H <= 8192), so the row
// is read from HBM once and 256 threads keep loads in flight.  The sums meet
// in a fixed order (wave shuffles, then the 4 wave totals in LDS in wave order).
constexpr int kNormMaxV = 8;
__device__ __forceinline__ float block4_sum(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();   // red is reused by the next call
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// Where a row kernel's float32 input comes from: an array, or the split-K
// partials of the GEMM that produces it, summed in split order (split_sum4,
// the order of the plain reduction) plus an optional float32 residual, the
// summed row also stored when out is set.  Fusing the reduction into its
// consumer this way gives the same bits as the separate reduction kernel.
struct RowSrc {
  const float* x;       // [T][H], or null for partials
  const float* part;    // [splits][T][H]
  int splits;
  const float* resid;   // [T][H] (nullable)
  float* out;           // [T][H] (nullable)
};
__device__ __forceinline__ float4 row_load4(const RowSrc& s, int64_t e, int64_t total) {
  if (s.x) return *reinterpret_cast<const float4*>(s.x + e);
  float4 v = split_sum4(s.part, s.splits, total, e);
  if (s.resid) {
    const float4 r = *reinterpret_cast<const float4*>(s.resid + e);
    v = make_float4(r.x + v.x, r.y + v.y, r.z + v.z, r.w + v.w);
  }
  if (s.out) *reinterpret_cast<float4*>(s.out + e) = v;
  return v;
}

// y = bf16(w * x / sqrt(mean(x^2) + eps)), rows ldy apart; rstd saved.  With
// y_lo, the output is also written as the bf16 rounding of its own remainder
// (y + y_lo carries about 16 bits), for GEMMs run as two bf16 passes.
__global__ void __launch_bounds__(256) rmsnorm_fwd_kernel(RowSrc x, const uint16_t* __restrict__ w, int T, int H,
                                                          float eps, uint16_t* __restrict__ y, int64_t ldy,
                                                          float* __restrict__ rstd, uint16_t* __restrict__ y_lo) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x, n4 = H / 4;
  const int64_t r0 = (int64_t)row * H, total = (int64_t)T * H;
  float4 v[kNormMaxV];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kNormMaxV; ++k) {
    const int i = tid + 256 * k;
    v[k] = i < n4 ? row_load4(x, r0 + 4 * i, total) : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  }
  ss = block4_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (rstd && tid == 0) rstd[row] = r;
  const uint2* wr = reinterpret_cast<const uint2*>(w);
  uint2* yr = reinterpret_cast<uint2*>(y + (int64_t)row * ldy);
  uint2* lr = y_lo ? reinterpret_cast<uint2*>(y_lo + (int64_t)row * ldy) : nullptr;
#pragma unroll
  for (int k = 0; k < kNormMaxV; ++k) {
    const int i = tid + 256 * k;
    if (i >= n4) continue;
    const uint2 ww = wr[i];
    const float o0 = bf_lo(ww.x) * (v[k].x * r), o1 = bf_hi(ww.x) * (v[k].y * r);
    const float o2 = bf_lo(ww.y) * (v[k].z * r), o3 = bf_hi(ww.y) * (v[k].w * r);
    const uint2 hi = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    yr[i] = hi;
    if (lr)
      lr[i] = make_uint2(pack_bf16x2(o0 - bf_lo(hi.x), o1 - bf_hi(hi.x)), pack_bf16x2(o2 - bf_lo(hi.y), o3 - bf_hi(hi.y)));
  }
}

// dx = gres + r (w dy) - x r^3 sum(w dy x) / H ; also a bf16 copy of dx.
__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const float* __restrict__ x, const uint16_t* __restrict__ w,
                                                          RowSrc dy, const float* __restrict__ gres, int T, int H,
                                                          float eps, float* __restrict__ dx,
                                                          uint16_t* __restrict__ dx_b) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x, n4 = H / 4;
  const int64_t r0 = (int64_t)row * H, total = (int64_t)T * H;
  const float4* xr = reinterpret_cast<const float4*>(x + r0);
  const uint2* wr = reinterpret_cast<const uint2*>(w);
  float4 v[kNormMaxV], d[kNormMaxV];
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int k = 0; k < kNormMaxV; ++k) {
    const int i = tid + 256 * k;
    const bool ok = i < n4;
    v[k] = ok ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    d[k] = ok ? row_load4(dy, r0 + 4 * i, total) : make_float4(0.f, 0.f, 0.f, 0.f);
    const uint2 ww = ok ? wr[i] : make_uint2(0u, 0u);
    ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    dot += bf_lo(ww.x) * d[k].x * v[k].x + bf_hi(ww.x) * d[k].y * v[k].y + bf_lo(ww.y) * d[k].z * v[k].z +
           bf_hi(ww.y) * d[k].w * v[k].w;
  }
  ss = block4_sum(ss, red);
  dot = block4_sum(dot, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  const float c = r * r * r * dot / (float)H;
  float4* outr = reinterpret_cast<float4*>(dx + (int64_t)row * H);
  const float4* gr = gres ? reinterpret_cast<const float4*>(gres + (int64_t)row * H) : nullptr;
  uint2* ob = dx_b ? reinterpret_cast<uint2*>(dx_b + (int64_t)row * H) : nullptr;
#pragma unroll
  for (int k = 0; k < kNormMaxV; ++k) {
    const int i = tid + 256 * k;
    if (i >= n4) continue;
    const uint2 ww = wr[i];
    float4 o;
    o.x = r * bf_lo(ww.x) * d[k].x - v[k].x * c;
    o.y = r * bf_hi(ww.x) * d[k].y - v[k].y * c;
    o.z = r * bf_lo(ww.y) * d[k].z - v[k].z * c;
    o.w = r * bf_hi(ww.y) * d[k].w - v[k].w * c;
    if (gr) {
      const float4 g = gr[i];
      o.x += g.x;
      o.y += g.y;
      o.z += g.z;
      o.w += g.w;
    }
    outr[i] = o;
    if (ob) ob[i] = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
  }
}

__global__ void f32_to_bf16_kernel(const float* __restrict__ x, int64_t n, uint16_t* __restrict__ y) {
  int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  float4 v = *reinterpret_cast<const float4*>(x + i);
  *reinterpret_cast<uint2*>(y + i) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

// ------------------------------------------------------------------ rotary
// table[s][i] = (cos, sin) of s * theta^(-2i/d), computed in float64.
__global__ void rope_table_kernel(int S, int half, double theta, float2* __restrict__ table) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= S * half) return;
  int s = e / half, i = e % half;
  double inv = pow(theta, -2.0 * i / (2.0 * half));
  double a = (double)s * inv;
  table[e] = make_float2((float)cos(a), (float)sin(a));
}

// Rotate-half on the q and k heads of a [T, ld] bf16 buffer, in place.
// inverse != 0 applies the transposed rotation (the backward).
__global__ void rope_kernel(uint16_t* __restrict__ buf, int64_t ld, int T, int S, int n_rot_heads, int half,
                            const float2* __restrict__ table, int inverse) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T * n_rot_heads * half;
  if (e >= total) return;
  const int i = e % half;
  const int h = (e / half) % n_rot_heads;
  const int t = e / ((int64_t)half * n_rot_heads);
  const int s = t % S;
  const float2 cs = table[(int64_t)s * half + i];
  const float sn = inverse ? -cs.y : cs.y;
  uint16_t* p = buf + (int64_t)t * ld + (int64_t)h * 2 * half;
  const float x1 = bf16_bits_to_f32(p[i]), x2 = bf16_bits_to_f32(p[i + half]);
  p[i] = f32_to_bf16_bits(x1 * cs.x - x2 * sn);
  p[i + half] = f32_to_bf16_bits(x2 * cs.x + x1 * sn);
}

// ------------------------------------------------------------------ attention
// Causal GQA attention on 64-query x 64-key tiles (one workgroup per (query
// block, head, batch) forward and for dQ, per (key block, head) for dK and dV);
// scores are kept in base 2: s2 = q.k * scale * log2(e), lse2 = max + log2(sum).
constexpr int AT = 64;
// bf16 elements of padding after every row of an attention LDS tile (keeps the
// rows of one 16-lane fragment read in distinct banks)
constexpr int PAD = 8;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------ attention on bf16 MFMA
// The float32 operands (rotated q and k, the probabilities P) enter the bf16
// matrix cores as hi/lo pairs: x = hi + lo with hi = bf16(x), lo = bf16(x - hi),
// which carries 16 of float32's 24 mantissa bits.  Q K^T takes the three
// products hi.hi + hi.lo + lo.hi (the lo.lo term is below 2^-17 of the
// result); P V takes P's two halves against V's exact bf16 values.
// Accumulation is float32 throughout.
__device__ __forceinline__ bf16x8 mfma_a8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 8 floats -> bf16 hi and lo halves, as MFMA operands
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    h[t] = pack_bf16x2(x[2 * t], x[2 * t + 1]);
    l[t] = pack_bf16x2(x[2 * t] - bf_lo(h[t]), x[2 * t + 1] - bf_hi(h[t]));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}
__device__ __forceinline__ void unpack8(uint4 v, float (&x)[8]) {
  x[0] = bf_lo(v.x); x[1] = bf_hi(v.x); x[2] = bf_lo(v.y); x[3] = bf_hi(v.y);
  x[4] = bf_lo(v.z); x[5] = bf_hi(v.z); x[6] = bf_lo(v.w); x[7] = bf_hi(v.w);
}
// 8 consecutive values of a float32 row (zeros when !ok).
__device__ __forceinline__ void load8(const float* p, bool ok, float (&x)[8]) {
  const float4 a = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 b = ok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// 8 consecutive values of a bf16 row, or of a float32 row rounded to bf16, as one uint4 (zeros when !ok).
__device__ __forceinline__ uint4 load8_bf16(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
}
__device__ __forceinline__ uint4 load8_bf16(const float* p, bool ok) {
  float x[8];
  load8(p, ok, x);
  return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7]));
}
// Where the attention preparation reads the float32 q/k/v from: the array
// itself, or (part set) the split-K partials of the q/k/v product, summed in
// split order plus the bias and stored into the array on the way, exactly as
// the plain reduction would write them.
struct QkvSrc {
  float* base;            // the q/k/v array [B*S][ld]
  const float* part;      // [splits][B*S][ld], or null
  int splits;
  int64_t total;          // B*S*ld
  int64_t ld;
  const uint16_t* bias;   // [ld] bf16 (nullable)
};
__device__ __forceinline__ void load8(const QkvSrc& q, const float* p, bool ok, float (&x)[8]) {
  if (!q.part || !ok) {
    load8(p, ok, x);
    return;
  }
  const int64_t e = p - q.base;
  const float4 a = split_sum4(q.part, q.splits, q.total, e), b = split_sum4(q.part, q.splits, q.total, e + 4);
  float r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  if (q.bias) {
    const int64_t col = e % q.ld;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] += bf16_bits_to_f32(q.bias[col + j]);
  }
  *reinterpret_cast<float4*>(q.base + e) = make_float4(r[0], r[1], r[2], r[3]);
  *reinterpret_cast<float4*>(q.base + e + 4) = make_float4(r[4], r[5], r[6], r[7]);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = r[j];
}
__device__ __forceinline__ uint4 load8_bf16(const QkvSrc& q, const float* p, bool ok) {
  float x[8];
  load8(q, p, ok, x);
  return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7]));
}
__device__ __forceinline__ uint4 load8_bf16(const QkvSrc&, const uint16_t* p, bool ok) { return load8_bf16(p, ok); }
// The same for a bf16 operand (the attention output's gradient): the array, or
// (part set) the split-K partials of the product that makes it, summed in
// split order, rounded to bf16 and stored into the array on the way, as the
// plain reduction would store them.
struct Bf16Src {
  uint16_t* base;         // the bf16 array [rows][ld]
  const float* part;      // [splits][rows][ld], or null
  int splits;
  int64_t total;          // rows * ld
};
__device__ __forceinline__ uint4 load8_bf16(const Bf16Src& q, const uint16_t* p, bool ok) {
  if (!q.part || !ok) return load8_bf16(p, ok);
  const int64_t e = p - q.base;
  const float4 a = split_sum4(q.part, q.splits, q.total, e), b = split_sum4(q.part, q.splits, q.total, e + 4);
  auto bits2 = [](float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
  };
  const uint4 v = make_uint4(bits2(a.x, a.y), bits2(a.z, a.w), bits2(b.x, b.y), bits2(b.z, b.w));
  *reinterpret_cast<uint4*>(q.base + e) = v;
  return v;
}
// Rotate-half RoPE of 8 consecutive pair indices i .. i+7 at position pos:
// (x1, x2) -> (x1 c - x2 s, x2 c + x1 s), table[pos][i] = (c, s).
__device__ __forceinline__ void rope8(float (&x1)[8], float (&x2)[8], const float2* __restrict__ tab) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float2 cs = tab[t];
    const float a = x1[t], b = x2[t];
    x1[t] = a * cs.x - b * cs.y;
    x2[t] = b * cs.x + a * cs.y;
  }
}
__device__ __forceinline__ void store_hilo8(uint16_t* hi, uint16_t* lo, const float (&x)[8]) {
  bf16x8 h, l;
  split8(x, h, l);
  *reinterpret_cast<bf16x8*>(hi) = h;
  *reinterpret_cast<bf16x8*>(lo) = l;
}

// ---- backward on bf16 MFMA: staging helpers (64-row blocks, 256 threads)
// Write a 4-row x 8-column bf16 micro-tile transposed: dst[c][r0 .. r0+4] for
// its 8 columns c (two v_perm per column pair).
template <int PITCH>
__device__ __forceinline__ void put_mt_t(uint16_t (*dst)[PITCH], int c0, int r0, const uint4 (&rows)[4]) {
  const uint32_t w[4][4] = {{rows[0].x, rows[0].y, rows[0].z, rows[0].w}, {rows[1].x, rows[1].y, rows[1].z, rows[1].w},
                            {rows[2].x, rows[2].y, rows[2].z, rows[2].w}, {rows[3].x, rows[3].y, rows[3].z, rows[3].w}};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int sel = (c & 1) ? 0x07060302 : 0x05040100;
    const uint32_t lo = __builtin_amdgcn_perm(w[1][c >> 1], w[0][c >> 1], sel);
    const uint32_t hi = __builtin_amdgcn_perm(w[3][c >> 1], w[2][c >> 1], sel);
    *reinterpret_cast<u32x2*>(&dst[c0 + c][r0]) = u32x2{lo, hi};
  }
}
// Rows [row0, row0 + 64) of a bf16 matrix, rotated (RoPE at positions
// row0 + r) and split into hi/lo, row-major.  Rows at or past n read as zero.
template <int HD>
__device__ __forceinline__ void stage_rot(uint16_t (*hi)[HD + PAD], uint16_t (*lo)[HD + PAD], const QkvSrc& qs,
                                          const float* src, int64_t ld, int row0, int n,
                                          const float2* __restrict__ rope) {
  constexpr int HALF = HD / 2, NCH = HALF / 32;
  const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
  const bool ok = r < n;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i0 = (q * NCH + c) * 8;
    float x1[8], x2[8];
    const float* row = src + (int64_t)(row0 + r) * ld;
    load8(qs, row + i0, ok, x1);
    load8(qs, row + HALF + i0, ok, x2);
    if (ok) rope8(x1, x2, rope + (int64_t)(row0 + r) * HALF + i0);
    store_hilo8(&hi[r][i0], &lo[r][i0], x1);
    store_hilo8(&hi[r][HALF + i0], &lo[r][HALF + i0], x2);
  }
}
// Rows [row0, row0 + 64) copied row-major (zero past n).
template <int HD>
__device__ __forceinline__ void stage_rows(uint16_t (*dst)[HD + PAD], const uint16_t* src, int64_t ld, int row0, int n) {
  for (int e = threadIdx.x; e < AT * HD / 8; e += 256) {
    const int r = e / (HD / 8), c = (e % (HD / 8)) * 8;
    *reinterpret_cast<uint4*>(&dst[r][c]) =
        r < n ? *reinterpret_cast<const uint4*>(src + (int64_t)(row0 + r) * ld + c) : make_uint4(0u, 0u, 0u, 0u);
  }
}
// A staged row-major [64][HD] tile transposed into [HD][64] (call after a barrier).
template <int HD>
__device__ __forceinline__ void lds_transpose(uint16_t (*dst)[AT + PAD], const uint16_t (*src)[HD + PAD]) {
  constexpr int NMT = AT / 4 * (HD / 8);
  for (int t = threadIdx.x; t < NMT; t += 256) {
    const int rg = t / (HD / 8), cg = t % (HD / 8);
    uint4 rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rows[i] = *reinterpret_cast<const uint4*>(&src[4 * rg + i][8 * cg]);
    put_mt_t<AT + PAD>(dst, 8 * cg, 4 * rg, rows);
  }
}
// Rows [row0, row0 + 64) of a bf16 matrix straight into [HD][64] (zero past n).
template <int HD, typename SrcT, typename Q>
__device__ __forceinline__ void stage_rows_t(uint16_t (*dst)[AT + PAD], const Q& qs, const SrcT* src, int64_t ld,
                                             int row0, int n) {
  constexpr int NMT = AT / 4 * (HD / 8);
  for (int t = threadIdx.x; t < NMT; t += 256) {
    const int rg = t / (HD / 8), cg = t % (HD / 8);
    uint4 rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * rg + i;
      rows[i] = load8_bf16(qs, src + (int64_t)(row0 + r) * ld + 8 * cg, r < n);
    }
    put_mt_t<AT + PAD>(dst, 8 * cg, 4 * rg, rows);
  }
}
// ---- operands prepared once per attention call
// Every key/query block of 64 rows is staged by many workgroups (one per
// query/key block after it), so the rotation, the hi/lo split and the
// transposes run once per call in the prep kernels below and the attention
// kernels stage plain copies.  Layouts, bf16, rows padded with zeros to Sp, a
// multiple of 64: rows [b][head][Sp][HD], transposed [b][head][HD][Sp].
struct PrepPtrs {
  uint16_t *kh, *kl, *qh, *ql;          // rotated K and Q, bf16 hi/lo rows
  uint16_t* vt;                         // forward: V^T
  uint16_t *kht, *qht, *ot, *vr;   // backward: K^T and Q^T (bf16 of the rotated values), dO^T, V rows
  int Sp;
};
PrepPtrs prep_ptrs(uint16_t* base, int B, int S, int nh, int nkv, int hd, bool bwd) {
  PrepPtrs p{};
  p.Sp = (S + AT - 1) / AT * AT;
  const int64_t ekv = (int64_t)B * nkv * p.Sp * hd, eq = (int64_t)B * nh * p.Sp * hd;
  uint16_t* c = base;
  auto take = [&](int64_t n) {
    uint16_t* r = base ? c : nullptr;
    c += n;
    return r;
  };
  p.kh = take(ekv);
  p.kl = take(ekv);
  p.qh = take(eq);
  p.ql = take(eq);
  if (bwd) {
    p.kht = take(ekv);
    p.vr = take(ekv);
    p.qht = take(eq);
    p.ot = take(eq);
  } else {
    p.vt = take(ekv);
  }
  return p;
}

// One thread's share of a 64 x HD (or HD x 64) bf16 tile: the staging loads of
// a block are all issued into registers before any is stored to LDS, so a
// block costs one memory round trip, and the kernels issue the next block's
// loads before the current block's MFMAs (register prefetch; the last block's
// prefetch is clamped to a block in range and never stored).
template <int HD>
struct Chunks {
  static constexpr int N = AT * HD / 8 / 256;
  uint4 v[N];
};
// f(integral_constant<int, I>) for I = 0 .. N-1, with the index a constant from
// the start (so the register arrays indexed by it never need memory).
template <typename F, int... I>
__device__ __forceinline__ void each_chunk(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void each_chunk(F&& f) {
  each_chunk(f, std::make_integer_sequence<int, N>{});
}
// A tile of ROWS rows x COLS bf16 from rows of pitch ld (rows at or past n read
// as zero) into registers, and out to an LDS tile with rows of COLS + PAD.
template <int ROWS, int COLS>
__device__ __forceinline__ void ld_tile(Chunks<ROWS * COLS / AT>& c, const uint16_t* __restrict__ src, int64_t ld,
                                        int n) {
  each_chunk<Chunks<ROWS * COLS / AT>::N>([&](auto i) __attribute__((always_inline)) {
    const int e = threadIdx.x + 256 * i.value, r = e / (COLS / 8), k = (e % (COLS / 8)) * 8;
    c.v[i.value] = r < n ? *reinterpret_cast<const uint4*>(src + r * ld + k) : make_uint4(0u, 0u, 0u, 0u);
  });
}
template <int ROWS, int COLS>
__device__ __forceinline__ void st_tile(uint16_t (*dst)[COLS + PAD], const Chunks<ROWS * COLS / AT>& c) {
  each_chunk<Chunks<ROWS * COLS / AT>::N>([&](auto i) __attribute__((always_inline)) {
    const int e = threadIdx.x + 256 * i.value, r = e / (COLS / 8), k = (e % (COLS / 8)) * 8;
    *reinterpret_cast<uint4*>(&dst[r][k]) = c.v[i.value];
  });
}
template <int HD>
__device__ __forceinline__ void ld_rows(Chunks<HD>& c, const uint16_t* __restrict__ src, int64_t ld, int n) {
  ld_tile<AT, HD>(c, src, ld, n);
}
template <int HD>
__device__ __forceinline__ void st_rows(uint16_t (*dst)[HD + PAD], const Chunks<HD>& c) {
  st_tile<AT, HD>(dst, c);
}
template <int HD>
__device__ __forceinline__ void ld_cols(Chunks<HD>& c, const uint16_t* __restrict__ src, int Sp) {
  ld_tile<HD, AT>(c, src, Sp, HD);
}
template <int HD>
__device__ __forceinline__ void st_cols(uint16_t (*dst)[AT + PAD], const Chunks<HD>& c) {
  st_tile<HD, AT>(dst, c);
}
// [64][HD] and [HD][64] LDS tiles out to the prepared layouts.
template <int HD>
__device__ __forceinline__ void put_rows(uint16_t* __restrict__ dst, const uint16_t (*src)[HD + PAD]) {
  for (int e = threadIdx.x; e < AT * HD / 8; e += 256) {
    const int r = e / (HD / 8), c = (e % (HD / 8)) * 8;
    *reinterpret_cast<uint4*>(dst + r * HD + c) = *reinterpret_cast<const uint4*>(&src[r][c]);
  }
}
template <int HD>
__device__ __forceinline__ void put_cols(uint16_t* __restrict__ dst, const uint16_t (*src)[AT + PAD], int Sp) {
  for (int e = threadIdx.x; e < HD * AT / 8; e += 256) {
    const int d = e / (AT / 8), c = (e % (AT / 8)) * 8;
    *reinterpret_cast<uint4*>(dst + (int64_t)d * Sp + c) = *reinterpret_cast<const uint4*>(&src[d][c]);
  }
}

template <int HD>
struct PrepRotSmem {
  uint16_t h[AT][HD + PAD], l[AT][HD + PAD];
  uint16_t t[HD][AT + PAD];
};
// Where the rotated rows of one set of heads go (hiT null: no transpose).
struct RotOut {
  uint16_t *hi, *lo, *hiT;
};
// Rows [row0, row0 + 64) of batch b, qkv head column hh (hh < nA: a query
// head, set A; else key head hh - nA, set B), rotated in float32 and split
// into bf16 hi/lo rows, and the hi rows transposed where the set asks for it.
template <int HD>
__device__ __forceinline__ void prep_rot_block(PrepRotSmem<HD>& sm, const QkvSrc& qs, const float* qkv,
                                               int64_t ld, int S, int Sp, int row0, int hh, int b, int nA, int nB,
                                               const float2* __restrict__ rope, const RotOut& A, const RotOut& Bo) {
  const bool in_a = hh < nA;
  const RotOut o = in_a ? A : Bo;
  const int nheads = in_a ? nA : nB, hl = in_a ? hh : hh - nA;
  const float* src = qkv + (int64_t)b * S * ld + (int64_t)hh * HD;
  stage_rot<HD>(sm.h, sm.l, qs, src, ld, row0, S - row0, rope);
  __syncthreads();
  const int64_t hb = (int64_t)b * nheads + hl;
  put_rows<HD>(o.hi + (hb * Sp + row0) * HD, sm.h);
  put_rows<HD>(o.lo + (hb * Sp + row0) * HD, sm.l);
  if (!o.hiT) return;   // uniform over the workgroup
  lds_transpose<HD>(sm.t, sm.h);
  __syncthreads();
  put_cols<HD>(o.hiT + hb * HD * Sp + row0, sm.t, Sp);
}
// The same rows of a plain operand (V from the float32 qkv, dO in bf16) at
// column head `col`, transposed into head hh of dstT, in bf16.
template <int HD, typename SrcT, typename Q>
__device__ __forceinline__ void prep_t_block(uint16_t (*t)[AT + PAD], const Q& qs, const SrcT* src,
                                             int64_t ld, int S, int Sp, int row0, int col, int hh, int b, int nheads,
                                             uint16_t* dstT) {
  stage_rows_t<HD>(t, qs, src + (int64_t)b * S * ld + (int64_t)col * HD, ld, row0, S - row0);
  __syncthreads();
  put_cols<HD>(dstT + ((int64_t)b * nheads + hh) * HD * Sp + row0, t, Sp);
}
// V rows of the float32 qkv rounded to bf16 rows [b][head][Sp][HD] (zero past S).
template <int HD>
__device__ __forceinline__ void prep_rows_block(const float* __restrict__ src, int64_t ld, int S, int Sp, int row0,
                                                int col, int hh, int b, int nheads, uint16_t* dst) {
  const float* base = src + (int64_t)b * S * ld + (int64_t)col * HD;
  uint16_t* out = dst + (((int64_t)b * nheads + hh) * Sp + row0) * HD;
  for (int e = threadIdx.x; e < AT * HD / 8; e += 256) {
    const int r = e / (HD / 8), c = (e % (HD / 8)) * 8;
    *reinterpret_cast<uint4*>(out + r * HD + c) = load8_bf16(base + (int64_t)(row0 + r) * ld + c, row0 + r < S);
  }
}
// D[b*S + t][h] = sum_d dO[t, h, d] * O[t, h, d] for rows [row0, row0 + 64),
// with the float32 O of the forward: D must equal sum_j P_j dP_j, and a
// rounded O breaks that identity exactly where attention is peaked and
// dP_j - D cancels.  Four lanes per row, each a quarter of d in order, then
// summed in a fixed order.
template <int HD>
__device__ __forceinline__ void dot_rows_block(const uint16_t* __restrict__ dO, const float* __restrict__ O,
                                               int64_t ldo, int S, int row0, int h, int b, int nh,
                                               float* __restrict__ D) {
  constexpr int Q = HD / 4;
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int t = row0 + r;
  float acc = 0.f;
  if (t < S) {
    const int64_t off = ((int64_t)b * S + t) * ldo + (int64_t)h * HD + part * Q;
#pragma unroll
    for (int d = 0; d < Q; d += 8) {
      float x[8], y[8];
      load8(O + off + d, true, y);
      const uint4 xb = *reinterpret_cast<const uint4*>(dO + off + d);
      const uint32_t xw[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf_lo(xw[j]);
        x[2 * j + 1] = bf_hi(xw[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += x[j] * y[j];
    }
  }
  const float s1 = acc + __shfl_xor(acc, 1, 64);
  const float s2 = s1 + __shfl_xor(s1, 2, 64);
  if (part == 0 && t < S) D[((int64_t)b * S + t) * nh + h] = s2;
}

// Every operand the forward prepares, one launch: workgroups (row block x,
// y, batch z); y < nh + nkv rotates and splits Q and K, the rest transpose V.
// With qs.part set, every q/k/v value is summed from the product's split-K
// partials (each by the one workgroup that reads it) and stored on the way.
template <int HD>
__global__ void __launch_bounds__(256) attn_prep_fwd_kernel(QkvSrc qs, int64_t ld, int S, int Sp, int nh, int nkv,
                                                           const float2* __restrict__ rope, RotOut Qo, RotOut Ko,
                                                           uint16_t* vt) {
  __shared__ __attribute__((aligned(16))) PrepRotSmem<HD> sm;
  const int row0 = blockIdx.x * AT, y = blockIdx.y, b = blockIdx.z;
  const float* qkv = qs.base;
  if (y < nh + nkv)
    prep_rot_block<HD>(sm, qs, qkv, ld, S, Sp, row0, y, b, nh, nkv, rope, Qo, Ko);
  else
    prep_t_block<HD, float, QkvSrc>(sm.t, qs, qkv, ld, S, Sp, row0, y, y - nh - nkv, b, nkv, vt);
}
// Every operand the backward prepares, one launch: y < nh + nkv rotates and
// splits Q and K (with the transposes of their bf16 values), the next nkv
// round V rows to bf16, the last nh transpose dO and form D for their rows.
template <int HD>
__global__ void __launch_bounds__(256) attn_prep_bwd_kernel(const float* __restrict__ qkv, int64_t ld, int S, int Sp,
                                                           int nh, int nkv, const float2* __restrict__ rope,
                                                           RotOut Qo, RotOut Ko, uint16_t* vr, Bf16Src dos,
                                                           const float* __restrict__ O, int64_t ldo, uint16_t* ot,
                                                           float* __restrict__ D) {
  const uint16_t* dO = dos.base;
  __shared__ __attribute__((aligned(16))) PrepRotSmem<HD> sm;
  const int row0 = blockIdx.x * AT, y = blockIdx.y, b = blockIdx.z;
  if (y < nh + nkv) {
    prep_rot_block<HD>(sm, QkvSrc{const_cast<float*>(qkv), nullptr, 0, 0, ld, nullptr}, qkv, ld, S, Sp, row0, y, b,
                       nh, nkv, rope, Qo, Ko);
  } else if (y < nh + 2 * nkv) {
    prep_rows_block<HD>(qkv, ld, S, Sp, row0, y, y - nh - nkv, b, nkv, vr);
  } else {
    const int h = y - nh - 2 * nkv;
    // dO summed from its product's partials is stored before the barrier
    // inside prep_t_block, so the dot below reads the stored values
    prep_t_block<HD, uint16_t, Bf16Src>(sm.t, dos, dO, ldo, S, Sp, row0, h, h, b, nh, ot);
    dot_rows_block<HD>(dO, O, ldo, S, row0, h, b, nh, D);
  }
}

template <int HD>
__device__ __forceinline__ void load_frags(const uint16_t* row, bool ok, int lg, bf16x8 (&f)[HD / 32]) {
#pragma unroll
  for (int c = 0; c < HD / 32; ++c)
    f[c] = __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const uint4*>(row + 32 * c + 8 * lg)
                                         : make_uint4(0u, 0u, 0u, 0u));
}
// Four consecutive values as bf16 hi/lo quads, one 8-byte store each.
__device__ __forceinline__ void put_hilo4(uint16_t* hi, uint16_t* lo, const float (&x)[4]) {
  const uint32_t h0 = pack_bf16x2(x[0], x[1]), h1 = pack_bf16x2(x[2], x[3]);
  const uint32_t l0 = pack_bf16x2(x[0] - bf_lo(h0), x[1] - bf_hi(h0));
  const uint32_t l1 = pack_bf16x2(x[2] - bf_lo(h1), x[3] - bf_hi(h1));
  *reinterpret_cast<u32x2*>(hi) = u32x2{h0, h1};
  *reinterpret_cast<u32x2*>(lo) = u32x2{l0, l1};
}
// 2^x on the hardware's exponential unit (no denormal-range rescaling; the
// tiny results it would keep only matter far below the softmax's precision).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// Four consecutive values rounded to bf16, one 8-byte store.
__device__ __forceinline__ void put_bf16x4(uint16_t* dst, const float (&x)[4]) {
  *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}
__device__ __forceinline__ void put_hilo(uint16_t* hi, uint16_t* lo, float x) {
  const uint16_t h = f32_to_bf16_bits(x);
  *hi = h;
  *lo = f32_to_bf16_bits(x - bf16_bits_to_f32(h));
}

// XCD-aware order of attention work items (a query or key block of one head
// of one batch row; the grid is (blocks, heads, batch)).  Workgroups reach the
// 8 XCDs round-robin and each XCD has its own L2, while every item of one KV
// head group reads the same K and V.  So, when the item count is a multiple
// of 8, each XCD takes one contiguous run of the item list ordered group by
// group (batch-major), and within a group by block, heaviest first, then
// head: one group's K/V stays in one L2.  Otherwise the plain order: blocks
// along x (heaviest first), heads along y.  desc: the heaviest block is the
// last one (causal queries), else the first (keys).
struct AttnItem {
  int blk, h, b;
};
__device__ __forceinline__ AttnItem attn_item(int nh, int nkv, bool desc) {
  const int nblk = gridDim.x;
  const int total = nblk * nh * gridDim.z;
  if (total & 7) return AttnItem{desc ? nblk - 1 - (int)blockIdx.x : (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
  const int g = blockIdx.x + nblk * (blockIdx.y + nh * blockIdx.z);
  const int v = (g & 7) * (total >> 3) + (g >> 3);
  const int hpg = nh / nkv, per_group = nblk * hpg;
  const int gi = v / per_group, rem = v - gi * per_group;
  const int k = rem / hpg, hh = rem - k * hpg;
  return AttnItem{desc ? nblk - 1 - k : k, (gi % nkv) * hpg + hh, gi / nkv};
}

template <int HD>
struct AttnF16Smem {
  uint16_t kh[AT][HD + PAD];     // rotated K, bf16 hi  [key][d]
  uint16_t kl[AT][HD + PAD];     // rotated K, bf16 lo
  uint16_t vt[HD][AT + PAD];     // V transposed [d][key]
  uint16_t ph[4][16][AT + PAD];  // per-wave P hi [query][key]
  uint16_t pl[4][16][AT + PAD];  // per-wave P lo
  float al[4][16];             // per-wave row factors (rescale, then 1 / sum) by query
};

// Forward: one workgroup per (query block of 64, head, batch), the heaviest
// query blocks first; wave w owns queries 16w .. 16w+15 and keeps its rotated q
// as MFMA operands in registers.
template <int HD>
__global__ void __launch_bounds__(256) attn_fwd_bf16_kernel(AttnArgs a, PrepPtrs pp) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  AttnF16Smem<HD>& sm = *reinterpret_cast<AttnF16Smem<HD>*>(smem_raw);
  constexpr int DC = HD / 32, DT = HD / 16;
  const int nqb = gridDim.x;
  const AttnItem it = attn_item(a.nh, a.nkv, true);
  const int qb = it.blk, h = it.h, b = it.b;
  const int g = h / (a.nh / a.nkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int q0 = qb * AT;
  const int64_t rowbase = (int64_t)b * a.S;
  const int64_t kvh = (int64_t)b * a.nkv + g;
  const uint16_t* Kh = pp.kh + kvh * pp.Sp * HD;
  const uint16_t* Kl = pp.kl + kvh * pp.Sp * HD;
  const uint16_t* Vt = pp.vt + kvh * HD * pp.Sp;
  // this lane's query row (rotated, hi/lo; zero rows past S), its 8-wide d slices 32c + 8 lg .. +8
  bf16x8 qh[DC], ql[DC];
  {
    const int64_t qrow = (((int64_t)b * a.nh + h) * pp.Sp + q0 + 16 * w + lr) * HD;
    load_frags<HD>(pp.qh + qrow, true, lg, qh);
    load_frags<HD>(pp.ql + qrow, true, lg, ql);
  }
  const float sc = a.scale * kLog2e;
  // Scores are formed transposed (S^T = K Q^T): lane (lr, lg) holds keys
  // 16 jt + 4 lg + v of query 16 w + lr, so its P values go to LDS as four
  // 8-byte stores and the softmax state of its query (m_q, l_q) is shared by
  // the four lanes lg.  The output rows (queries 4 lg + v) take their factors
  // from the lanes that own those queries through sm.al.
  const int qi = q0 + 16 * w + lr;
  float m_q = -INFINITY, l_q = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  Chunks<HD> ckh, ckl, cvt;
  ld_rows<HD>(ckh, Kh, HD, AT);
  ld_rows<HD>(ckl, Kl, HD, AT);
  ld_cols<HD>(cvt, Vt, pp.Sp);
  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * AT;
    __syncthreads();   // the previous block's kh/kl/vt reads are done
    st_rows<HD>(sm.kh, ckh);
    st_rows<HD>(sm.kl, ckl);
    st_cols<HD>(sm.vt, cvt);
    __syncthreads();
    {
      const int kn = min(kb + 1, qb) * AT;
      ld_rows<HD>(ckh, Kh + (int64_t)kn * HD, HD, AT);
      ld_rows<HD>(ckl, Kl + (int64_t)kn * HD, HD, AT);
      ld_cols<HD>(cvt, Vt + kn, pp.Sp);
    }
    f32x4 st[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      st[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 kh = mfma_a8(&sm.kh[16 * jt + lr][32 * c + 8 * lg]);
        const bf16x8 kl = mfma_a8(&sm.kl[16 * jt + lr][32 * c + 8 * lg]);
        st[jt] = mfma_bf16(kh, qh[c], st[jt]);
        st[jt] = mfma_bf16(kl, qh[c], st[jt]);
        st[jt] = mfma_bf16(kh, ql[c], st[jt]);
      }
    }
    // Only the diagonal block needs the causal mask: every key of an earlier
    // block precedes every query of this one.  Key and query rows past S are
    // zero (prepared so) and only reach outputs that are never written.
    if (kb == qb) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (16 * jt + 4 * lg + v > 16 * w + lr) st[jt][v] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, st[jt][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // finite: key 0 is in every query's first block
    const float mn = fmaxf(m_q, mx * sc);
    const float alpha = fast_exp2(m_q - mn);
    float rs = 0.f;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      float pv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pv[v] = fast_exp2(fmaf(st[jt][v], sc, -mn));
        rs += pv[v];
      }
      put_hilo4(&sm.ph[w][lr][16 * jt + 4 * lg], &sm.pl[w][lr][16 * jt + 4 * lg], pv);
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l_q = l_q * alpha + rs;
    m_q = mn;
    // sm.al is wave-private: this wave's write lands before its read below
    if (lg == 0) sm.al[w][lr] = alpha;
    {
      const float4 a4 = *reinterpret_cast<const float4*>(&sm.al[w][4 * lg]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt][0] *= a4.x;
        o[dt][1] *= a4.y;
        o[dt][2] *= a4.z;
        o[dt][3] *= a4.w;
      }
    }
    // P is wave-private: this wave's LDS writes are done before its reads below
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x8 pah = mfma_a8(&sm.ph[w][lr][32 * kc + 8 * lg]);
      const bf16x8 pal = mfma_a8(&sm.pl[w][lr][32 * kc + 8 * lg]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 vb = mfma_a8(&sm.vt[16 * dt + lr][32 * kc + 8 * lg]);
        o[dt] = mfma_bf16(pah, vb, o[dt]);
        o[dt] = mfma_bf16(pal, vb, o[dt]);
      }
    }
  }
  if (lg == 0) {
    sm.al[w][lr] = l_q;
    if (qi < a.S) a.lse[((int64_t)b * a.nh + h) * a.S + qi] = m_q + log2f(l_q);
  }
  const float4 l4 = *reinterpret_cast<const float4*>(&sm.al[w][4 * lg]);
  const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int qo = q0 + 16 * w + 4 * lg + v;
    if (qo >= a.S) continue;
    const float inv = 1.f / lv[v];
    uint16_t* out = a.out + (rowbase + qo) * a.ldo + (int64_t)h * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) out[16 * dt + lr] = f32_to_bf16_bits(o[dt][v] * inv);
    if (a.out_f32) {
      float* of = a.out_f32 + (rowbase + qo) * a.ldo + (int64_t)h * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) of[16 * dt + lr] = o[dt][v] * inv;
    }
  }
}

template <int HD>
struct AttnDqSmem {
  uint16_t kh[AT][HD + PAD], kl[AT][HD + PAD];   // rotated K [key][d]
  uint16_t th[HD][AT + PAD];                   // its bf16 value transposed [d][key]
  uint16_t v[AT][HD + PAD];                    // V [key][d]
  uint16_t sh[4][16][AT + PAD], sl[4][16][AT + PAD];   // per-wave dS [query][key]
};

// dQ for one query block of one head; wave w owns queries 16w .. 16w+15.
template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) attn_bwd_dq_bf16_kernel(AttnBwdArgs a, PrepPtrs pp) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  AttnDqSmem<HD>& sm = *reinterpret_cast<AttnDqSmem<HD>*>(smem_raw);
  constexpr int DC = HD / 32, DT = HD / 16;
  const int nqb = gridDim.x;
  const AttnItem it = attn_item(a.nh, a.nkv, true);
  const int qb = it.blk, h = it.h, b = it.b;
  const int g = h / (a.nh / a.nkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int q0 = qb * AT;
  const int64_t rowbase = (int64_t)b * a.S;
  const float sc = a.scale * kLog2e;
  const int64_t kvh = (int64_t)b * a.nkv + g;
  const uint16_t* Vp = pp.vr + kvh * pp.Sp * HD;
  const uint16_t* Kh = pp.kh + kvh * pp.Sp * HD;
  const uint16_t* Kl = pp.kl + kvh * pp.Sp * HD;
  const uint16_t* Kht = pp.kht + kvh * HD * pp.Sp;
  bf16x8 qh[DC], ql[DC], od[DC];
  {
    const int qi = q0 + 16 * w + lr;
    const bool ok = qi < a.S;
    const int64_t qrow = (((int64_t)b * a.nh + h) * pp.Sp + qi) * HD;
    load_frags<HD>(pp.qh + qrow, true, lg, qh);
    load_frags<HD>(pp.ql + qrow, true, lg, ql);
    load_frags<HD>(a.dO + (rowbase + qi) * a.ldo + (int64_t)h * HD, ok, lg, od);
  }
  // this lane's query for the scores (formed transposed: lane = query, its 4 values = 4 keys)
  const int qi = q0 + 16 * w + lr;
  const float lse_q = qi < a.S ? a.lse[((int64_t)b * a.nh + h) * a.S + qi] : 0.f;
  const float dd_q = qi < a.S ? a.D[(rowbase + qi) * a.nh + h] : 0.f;
  f32x4 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // kh, kl and v of the next block are prefetched across this block's MFMAs;
  // the transposed tiles are loaded as a block begins (in flight during its barrier)
  Chunks<HD> ckh, ckl, cv, cth;
  ld_rows<HD>(ckh, Kh, HD, AT);
  ld_rows<HD>(ckl, Kl, HD, AT);
  ld_rows<HD>(cv, Vp, HD, AT);
  ld_cols<HD>(cth, Kht, pp.Sp);
  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * AT;
    __syncthreads();
    st_rows<HD>(sm.kh, ckh);
    st_rows<HD>(sm.kl, ckl);
    st_rows<HD>(sm.v, cv);
    st_cols<HD>(sm.th, cth);
    __syncthreads();
    {
      const int kn = min(kb + 1, qb) * AT;
      ld_rows<HD>(ckh, Kh + (int64_t)kn * HD, HD, AT);
      ld_rows<HD>(ckl, Kl + (int64_t)kn * HD, HD, AT);
      ld_rows<HD>(cv, Vp + (int64_t)kn * HD, HD, AT);
      ld_cols<HD>(cth, Kht + kn, pp.Sp);
    }
    f32x4 st[4], dpt[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      st[jt] = dpt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 kh = mfma_a8(&sm.kh[16 * jt + lr][32 * c + 8 * lg]);
        const bf16x8 kl = mfma_a8(&sm.kl[16 * jt + lr][32 * c + 8 * lg]);
        const bf16x8 vv = mfma_a8(&sm.v[16 * jt + lr][32 * c + 8 * lg]);
        st[jt] = mfma_bf16(kh, qh[c], st[jt]);   // S^T: C[key 16 jt + 4 lg + v][query lr]
        st[jt] = mfma_bf16(kl, qh[c], st[jt]);
        st[jt] = mfma_bf16(kh, ql[c], st[jt]);
        dpt[jt] = mfma_bf16(vv, od[c], dpt[jt]);
      }
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      float ds[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // the causal mask on the diagonal block only (rows past S are zero)
        const bool ok = kb != qb || 16 * jt + 4 * lg + v <= 16 * w + lr;
        const float pv = ok ? fast_exp2(fmaf(st[jt][v], sc, -lse_q)) : 0.f;
        ds[v] = pv * (dpt[jt][v] - dd_q);
      }
      put_hilo4(&sm.sh[w][lr][16 * jt + 4 * lg], &sm.sl[w][lr][16 * jt + 4 * lg], ds);
    }
    // dS is wave-private: this wave's LDS writes are done before its reads below.
    // dQ = dS K takes dS as a hi/lo pair and K as its bf16 value.
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x8 dh = mfma_a8(&sm.sh[w][lr][32 * kc + 8 * lg]);
      const bf16x8 dl = mfma_a8(&sm.sl[w][lr][32 * kc + 8 * lg]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 th = mfma_a8(&sm.th[16 * dt + lr][32 * kc + 8 * lg]);
        dq[dt] = mfma_bf16(dh, th, dq[dt]);
        dq[dt] = mfma_bf16(dl, th, dq[dt]);
      }
    }
  }
  constexpr int HALF_T = DT / 2;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int qi = q0 + 16 * w + 4 * lg + v;
    if (qi >= a.S) continue;
    uint16_t* dqp = a.dqkv + (rowbase + qi) * a.ld + (int64_t)h * HD;
#pragma unroll
    for (int dt = 0; dt < HALF_T; ++dt) {
      const int i = 16 * dt + lr;
      const float2 cs = a.rope[(int64_t)qi * (HD / 2) + i];
      const float g1 = dq[dt][v] * a.scale, g2 = dq[dt + HALF_T][v] * a.scale;
      dqp[i] = f32_to_bf16_bits(g1 * cs.x + g2 * cs.y);
      dqp[i + HD / 2] = f32_to_bf16_bits(g2 * cs.x - g1 * cs.y);
    }
  }
}

template <int HD>
struct AttnDkdvSmem {
  uint16_t qh[AT][HD + PAD], ql[AT][HD + PAD];   // rotated Q [query][d]
  uint16_t th[HD][AT + PAD];                   // its bf16 value transposed [d][query]
  uint16_t o[AT][HD + PAD];                    // dO [query][d]
  uint16_t ot[HD][AT + PAD];                   // dO transposed [d][query]
  uint16_t ph[4][16][AT + PAD], pl[4][16][AT + PAD];   // per-wave P^T [key][query]
  uint16_t sh[4][16][AT + PAD];                      // per-wave dS^T in bf16
  float lse[AT], dd[AT];
};

// One query head's contribution to dK and dV of one key block, over the query
// blocks at or after it, as float32 partials (summed over the group's heads in
// head order by attn_dkdv_reduce_kernel).  Wave w owns keys 16w .. 16w+15;
// scores are formed transposed (S^T = K Q^T) so P^T and dS^T come out key-major.
template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) attn_bwd_dkdv_bf16_kernel(AttnBwdArgs a, PrepPtrs pp) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  AttnDkdvSmem<HD>& sm = *reinterpret_cast<AttnDkdvSmem<HD>*>(smem_raw);
  constexpr int DC = HD / 32, DT = HD / 16;
  const AttnItem it = attn_item(a.nh, a.nkv, false);
  const int kb = it.blk, h = it.h, b = it.b;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int k0 = kb * AT;
  const int g = h / (a.nh / a.nkv);
  const int64_t rowbase = (int64_t)b * a.S;
  const float sc = a.scale * kLog2e;
  bf16x8 kh[DC], kl[DC], vv[DC];
  {   // this lane's key row: rotated K hi/lo and V, prepared rows (zero past S)
    const int64_t krow = (((int64_t)b * a.nkv + g) * pp.Sp + k0 + 16 * w + lr) * HD;
    load_frags<HD>(pp.kh + krow, true, lg, kh);
    load_frags<HD>(pp.kl + krow, true, lg, kl);
    load_frags<HD>(pp.vr + krow, true, lg, vv);
  }
  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nqb = (a.S + AT - 1) / AT;
  const int64_t qh_ = (int64_t)b * a.nh + h;
  const uint16_t* Qh = pp.qh + qh_ * pp.Sp * HD;
  const uint16_t* Ql = pp.ql + qh_ * pp.Sp * HD;
  const uint16_t* Qht = pp.qht + qh_ * HD * pp.Sp;
  const uint16_t* Ot = pp.ot + qh_ * HD * pp.Sp;
  const uint16_t* Op = a.dO + rowbase * a.ldo + (int64_t)h * HD;
  Chunks<HD> cqh, cql, co, cot, cth;
  float clse = 0.f, cdd = 0.f;
  // the blocks' loads, as a macro so that the register arrays stay plain locals
  // qh, ql, dO and the row statistics of the next block are prefetched across
  // this block's MFMAs; the transposed tiles are loaded as a block begins
#define LSQ_DKDV_LOAD(q0)                                                      \
  do {                                                                         \
    ld_rows<HD>(cqh, Qh + (int64_t)(q0) * HD, HD, AT);                         \
    ld_rows<HD>(cql, Ql + (int64_t)(q0) * HD, HD, AT);                         \
    ld_rows<HD>(co, Op + (int64_t)(q0) * a.ldo, a.ldo, a.S - (q0));            \
    ld_cols<HD>(cot, Ot + (q0), pp.Sp);                                        \
    ld_cols<HD>(cth, Qht + (q0), pp.Sp);                                       \
    const bool ok_ = tid < AT && (q0) + tid < a.S;                             \
    clse = ok_ ? a.lse[((int64_t)b * a.nh + h) * a.S + (q0) + tid] : 0.f;      \
    cdd = ok_ ? a.D[(rowbase + (q0) + tid) * a.nh + h] : 0.f;                  \
  } while (0)
  LSQ_DKDV_LOAD(kb * AT);
  for (int qb = kb; qb < nqb; ++qb) {
    const int q0 = qb * AT;
    __syncthreads();
    st_rows<HD>(sm.qh, cqh);
    st_rows<HD>(sm.ql, cql);
    st_rows<HD>(sm.o, co);
    st_cols<HD>(sm.ot, cot);
    st_cols<HD>(sm.th, cth);
    if (tid < AT) {
      sm.lse[tid] = clse;
      sm.dd[tid] = cdd;
    }
    __syncthreads();
    {
      const int qn = min(qb + 1, nqb - 1) * AT;
      LSQ_DKDV_LOAD(qn);
    }
    f32x4 st[4], dpt[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      st[jt] = dpt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 qhf = mfma_a8(&sm.qh[16 * jt + lr][32 * c + 8 * lg]);
        const bf16x8 qlf = mfma_a8(&sm.ql[16 * jt + lr][32 * c + 8 * lg]);
        const bf16x8 of = mfma_a8(&sm.o[16 * jt + lr][32 * c + 8 * lg]);
        st[jt] = mfma_bf16(qhf, kh[c], st[jt]);   // S: C[query 16 jt + 4 lg + v][key lr]
        st[jt] = mfma_bf16(qlf, kh[c], st[jt]);
        st[jt] = mfma_bf16(qhf, kl[c], st[jt]);
        dpt[jt] = mfma_bf16(of, vv[c], dpt[jt]);
      }
    }
    {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        float pv[4], ds[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // the causal mask on the diagonal block only (rows past S are zero)
          const int qr = 16 * jt + 4 * lg + v;
          const bool ok = qb != kb || 16 * w + lr <= qr;
          pv[v] = ok ? fast_exp2(fmaf(st[jt][v], sc, -sm.lse[qr])) : 0.f;
          ds[v] = pv[v] * (dpt[jt][v] - sm.dd[qr]);
        }
        put_hilo4(&sm.ph[w][lr][16 * jt + 4 * lg], &sm.pl[w][lr][16 * jt + 4 * lg], pv);
        put_bf16x4(&sm.sh[w][lr][16 * jt + 4 * lg], ds);
      }
    }
    // P^T and dS^T are wave-private: this wave's LDS writes are done before its
    // reads below.  dV = P^T dO takes P^T as a hi/lo pair; dK = dS^T Q takes
    // both dS and Q as their bf16 values.
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x8 pah = mfma_a8(&sm.ph[w][lr][32 * kc + 8 * lg]);
      const bf16x8 pal = mfma_a8(&sm.pl[w][lr][32 * kc + 8 * lg]);
      const bf16x8 sah = mfma_a8(&sm.sh[w][lr][32 * kc + 8 * lg]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 ob = mfma_a8(&sm.ot[16 * dt + lr][32 * kc + 8 * lg]);
        dv[dt] = mfma_bf16(pah, ob, dv[dt]);
        dv[dt] = mfma_bf16(pal, ob, dv[dt]);
        const bf16x8 th = mfma_a8(&sm.th[16 * dt + lr][32 * kc + 8 * lg]);
        dk[dt] = mfma_bf16(sah, th, dk[dt]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int kj = k0 + 16 * w + 4 * lg + v;
    if (kj >= a.S) continue;
    const int64_t o = (((int64_t)b * a.nh + h) * a.S + kj) * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      a.dk_part[o + 16 * dt + lr] = dk[dt][v];
      a.dv_part[o + 16 * dt + lr] = dv[dt][v];
    }
  }
}
#undef LSQ_DKDV_LOAD

// dK, dV of each KV head = sum of its query heads' partials (head order); dK
// is scaled and taken back through the rotation, both rounded once to bf16.
__global__ void attn_dkdv_reduce_kernel(AttnBwdArgs a, int B) {
  const int half = a.hd / 2;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * a.S * a.nkv * half;
  if (e >= total) return;
  const int i = e % half;
  const int g = (e / half) % a.nkv;
  const int64_t bs = e / ((int64_t)half * a.nkv);   // b * S + s
  const int b = bs / a.S, s = bs % a.S;
  const int group = a.nh / a.nkv;
  float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
  for (int hh = 0; hh < group; ++hh) {
    const int64_t o = (((int64_t)b * a.nh + g * group + hh) * a.S + s) * a.hd;
    k1 += a.dk_part[o + i];
    k2 += a.dk_part[o + i + half];
    v1 += a.dv_part[o + i];
    v2 += a.dv_part[o + i + half];
  }
  k1 *= a.scale;
  k2 *= a.scale;
  const float2 cs = a.rope[(int64_t)s * half + i];
  uint16_t* row = a.dqkv + bs * a.ld;
  row[(int64_t)(a.nh + g) * a.hd + i] = f32_to_bf16_bits(k1 * cs.x + k2 * cs.y);
  row[(int64_t)(a.nh + g) * a.hd + i + half] = f32_to_bf16_bits(k2 * cs.x - k1 * cs.y);
  row[(int64_t)(a.nh + a.nkv + g) * a.hd + i] = f32_to_bf16_bits(v1);
  row[(int64_t)(a.nh + a.nkv + g) * a.hd + i + half] = f32_to_bf16_bits(v2);
}

// ------------------------------------------------------------------ SwiGLU
// gu [T, 2I] (gate | up) -> m [T, I] = bf16(silu(g) * u).
// Rows t = blockIdx.y, + gridDim.y, ...; this thread's 8 intermediate columns start at i.
__global__ void __launch_bounds__(256) swiglu_fwd_kernel(const uint16_t* __restrict__ gu, int T, int I,
                                                         uint16_t* __restrict__ m) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= I) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    const uint4 gv = *reinterpret_cast<const uint4*>(gu + t * 2 * I + i);
    const uint4 uv = *reinterpret_cast<const uint4*>(gu + t * 2 * I + I + i);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float g0 = bf_lo(gw[q]), g1 = bf_hi(gw[q]), u0 = bf_lo(uw[q]), u1 = bf_hi(uw[q]);
      const float s0 = g0 / (1.f + __expf(-g0)), s1 = g1 / (1.f + __expf(-g1));
      o[q] = pack_bf16x2(s0 * u0, s1 * u1);
    }
    *reinterpret_cast<uint4*>(m + t * I + i) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// dgu [T, 2I]: dg = dm u sig(g) (1 + g (1 - sig(g))), du = dm silu(g)
// dm comes from a bf16 array, or (dm null) from the split-K partials of the
// GEMM that produces it, summed in split order and rounded to bf16 as the
// plain reduction would store it.
__global__ void __launch_bounds__(256) swiglu_bwd_kernel(const uint16_t* __restrict__ gu,
                                                         const uint16_t* __restrict__ dm,
                                                         const float* __restrict__ dm_part, int splits, int T, int I,
                                                         uint16_t* __restrict__ dgu) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= I) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    const uint4 gv = *reinterpret_cast<const uint4*>(gu + t * 2 * I + i);
    const uint4 uv = *reinterpret_cast<const uint4*>(gu + t * 2 * I + I + i);
    uint4 dv;
    if (dm) {
      dv = *reinterpret_cast<const uint4*>(dm + t * I + i);
    } else {
      const int64_t total = (int64_t)T * I;
      const float4 a = split_sum4(dm_part, splits, total, t * I + i);
      const float4 b = split_sum4(dm_part, splits, total, t * I + i + 4);
      auto bits2 = [](float lo, float hi) {
        return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
      };
      dv = make_uint4(bits2(a.x, a.y), bits2(a.z, a.w), bits2(b.x, b.y), bits2(b.z, b.w));
    }
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w}, dw[4] = {dv.x, dv.y, dv.z, dv.w};
    uint32_t og[4], ou[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float g[2] = {bf_lo(gw[q]), bf_hi(gw[q])}, u[2] = {bf_lo(uw[q]), bf_hi(uw[q])},
                  d[2] = {bf_lo(dw[q]), bf_hi(dw[q])};
      float dg[2], du[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sg = 1.f / (1.f + __expf(-g[j]));
        dg[j] = d[j] * u[j] * sg * (1.f + g[j] * (1.f - sg));
        du[j] = d[j] * g[j] * sg;
      }
      og[q] = pack_bf16x2(dg[0], dg[1]);
      ou[q] = pack_bf16x2(du[0], du[1]);
    }
    *reinterpret_cast<uint4*>(dgu + t * 2 * I + i) = make_uint4(og[0], og[1], og[2], og[3]);
    *reinterpret_cast<uint4*>(dgu + t * 2 * I + I + i) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
  }
}

// ------------------------------------------------------------------ embedding
__global__ void embed_kernel(const int32_t* __restrict__ ids, const uint16_t* __restrict__ table, int T, int H, int V,
                             float* __restrict__ x, int32_t* __restrict__ bad) {
  int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (e >= (int64_t)T * H) return;
  const int t = e / H, c = e % H;
  int id = ids[t];
  if (id < 0 || id >= V) {
    if (bad && c == 0) atomicOr(bad, 1);
    id = 0;
  }
  const uint2 w = *reinterpret_cast<const uint2*>(table + (int64_t)id * H + c);
  *reinterpret_cast<float4*>(x + e) = make_float4(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y));
}

// ------------------------------------------------------------------ cross-entropy
// One workgroup per row t of logits [T, V] (float32).  Rows whose position is
// the last of its sequence have no target: zero loss, zero gradient.
// loss_rows[t] = lse - logit[target]; dlogits[t] = bf16((softmax - onehot) / count).
// One row of logits per workgroup (V % 4 == 0).  Pass 1 keeps a running
// (max, sum of exp) pair per thread over float4 loads and merges the pairs in
// a fixed order; pass 2 writes dlogits (and its bf16 remainder) four at a time.
constexpr int kCeThreads = 512;
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}
__global__ void __launch_bounds__(kCeThreads) ce_kernel(const float* __restrict__ logits, const int32_t* __restrict__ ids,
                                                        int row0, int S, int V, float inv_count, float* __restrict__ loss_rows,
                                                        uint16_t* __restrict__ dlogits, uint16_t* __restrict__ dlogits_lo) {
  // logits, dlogits: this chunk's rows (chunk-local row blockIdx.x); ids and
  // loss_rows: global token index t = row0 + blockIdx.x
  constexpr int NW = kCeThreads / 64;
  __shared__ float red_m[NW], red_s[NW];
  const int lr = blockIdx.x, t = row0 + lr;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* row = logits + (int64_t)lr * V;
  const float4* row4 = reinterpret_cast<const float4*>(row);
  const int V4 = V / 4;
  // an out-of-range id (flagged by the embedding kernel) contributes no loss
  const int nxt = (t % S) != S - 1 ? ids[t + 1] : -1;
  const bool has_target = nxt >= 0 && nxt < V;
  const int target = has_target ? nxt : -1;
  float m = -FLT_MAX, sum = 0.f;
  for (int i = tid; i < V4; i += kCeThreads) {
    const float4 x = row4[i];
    const float mx4 = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
    if (mx4 > m) {
      sum *= __expf(m - mx4);
      m = mx4;
    }
    sum += ((__expf(x.x - m) + __expf(x.y - m)) + __expf(x.z - m)) + __expf(x.w - m);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(sum, o, 64);
    lse_merge(m, sum, m2, s2);
  }
  if (lane == 0) {
    red_m[w] = m;
    red_s[w] = sum;
  }
  __syncthreads();
  m = red_m[0];
  sum = red_s[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) lse_merge(m, sum, red_m[k], red_s[k]);
  const float lse = m + __logf(sum);
  const float inv_sum = 1.f / sum;
  uint2* drow = reinterpret_cast<uint2*>(dlogits + (int64_t)lr * V);
  uint2* lrow = dlogits_lo ? reinterpret_cast<uint2*>(dlogits_lo + (int64_t)lr * V) : nullptr;
  for (int i = tid; i < V4; i += kCeThreads) {
    const float4 x = row4[i];
    const float xv[4] = {x.x, x.y, x.z, x.w};
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float g = 0.f;
      if (has_target) g = (__expf(xv[c] - m) * inv_sum - (4 * i + c == target ? 1.f : 0.f)) * inv_count;
      hb[c] = f32_to_bf16_bits(g);
      lb[c] = f32_to_bf16_bits(g - bf16_bits_to_f32(hb[c]));
    }
    drow[i] = make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
    if (lrow) lrow[i] = make_uint2(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16));
  }
  if (tid == 0) loss_rows[t] = has_target ? lse - row[target] : 0.f;
}

// loss = sum of loss_rows (fixed order: per-thread strided partials, then a tree) * inv_count
__global__ void __launch_bounds__(256) loss_sum_kernel(const float* __restrict__ loss_rows, int T, float inv_count,
                                                       float* __restrict__ loss) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int i = tid; i < T; i += 256) s += loss_rows[i];
  s = warp_sum(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) *loss = (((red[0] + red[1]) + red[2]) + red[3]) * inv_count;
}

}  // namespace

// ================================================================== launchers
int rmsnorm_fwd(const float* x, const uint16_t* w, int T, int H, float eps, uint16_t* y, int64_t ldy, float* rstd,
                hipStream_t s, uint16_t* y_lo) {
  LSQ_CHECK(H % 4 == 0 && H <= 4 * 256 * kNormMaxV, LSQ_ERR_SHAPE,
            "rmsnorm: hidden %d must be a multiple of 4 and at most %d", H, 4 * 256 * kNormMaxV);
  if (T == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  rmsnorm_fwd_kernel<<<T, 256, 0, s>>>(RowSrc{x, nullptr, 0, nullptr, nullptr}, w, T, H, eps, y, ldy, rstd, y_lo);
  prof_end(tok, s, PROF_ELEM, 0.0, (4.0 + 2.0 + (y_lo ? 2.0 : 0.0)) * T * (double)H + 2.0 * H + (rstd ? 4.0 * T : 0.0));
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int splitk_resid_rmsnorm_fwd(const float* part, int splits, const float* resid, float* h, const uint16_t* w, int T,
                             int H, float eps, uint16_t* y, int64_t ldy, hipStream_t s) {
  LSQ_CHECK(H % 4 == 0 && H <= 4 * 256 * kNormMaxV && splits >= 1, LSQ_ERR_SHAPE,
            "rmsnorm: hidden %d must be a multiple of 4 and at most %d", H, 4 * 256 * kNormMaxV);
  if (T == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  rmsnorm_fwd_kernel<<<T, 256, 0, s>>>(RowSrc{nullptr, part, splits, resid, h}, w, T, H, eps, y, ldy, nullptr,
                                       nullptr);
  prof_end(tok, s, PROF_ELEM, 0.0, (4.0 * splits + (resid ? 4.0 : 0.0) + 4.0 + 2.0) * T * (double)H + 2.0 * H);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int rmsnorm_bwd(const float* x, const uint16_t* w, const float* dy, const float* gres, int T, int H, float eps,
                float* dx, uint16_t* dx_b, hipStream_t s) {
  LSQ_CHECK(H % 4 == 0 && H <= 4 * 256 * kNormMaxV, LSQ_ERR_SHAPE,
            "rmsnorm: hidden %d must be a multiple of 4 and at most %d", H, 4 * 256 * kNormMaxV);
  if (T == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  rmsnorm_bwd_kernel<<<T, 256, 0, s>>>(x, w, RowSrc{dy, nullptr, 0, nullptr, nullptr}, gres, T, H, eps, dx, dx_b);
  prof_end(tok, s, PROF_ELEM, 0.0,
           (4.0 + 4.0 + 4.0 + (gres ? 4.0 : 0.0) + (dx_b ? 2.0 : 0.0)) * T * (double)H + 2.0 * H);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int splitk_rmsnorm_bwd(const float* x, const uint16_t* w, const float* dy_part, int splits, const float* gres, int T,
                       int H, float eps, float* dx, uint16_t* dx_b, hipStream_t s) {
  LSQ_CHECK(H % 4 == 0 && H <= 4 * 256 * kNormMaxV && splits >= 1, LSQ_ERR_SHAPE,
            "rmsnorm: hidden %d must be a multiple of 4 and at most %d", H, 4 * 256 * kNormMaxV);
  if (T == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  rmsnorm_bwd_kernel<<<T, 256, 0, s>>>(x, w, RowSrc{nullptr, dy_part, splits, nullptr, nullptr}, gres, T, H, eps, dx,
                                       dx_b);
  prof_end(tok, s, PROF_ELEM, 0.0,
           (4.0 + 4.0 * splits + 4.0 + (gres ? 4.0 : 0.0) + (dx_b ? 2.0 : 0.0)) * T * (double)H + 2.0 * H);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

// Zero rows x cols 32-bit words at a row pitch of ld words, with a kernel
// rather than hipMemsetAsync so that the clear stays correct inside a captured
// HIP graph replayed several times.
__global__ void zero_words_kernel(uint32_t* __restrict__ dst, int64_t ld, int rows, int cols) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)rows * cols) return;
  dst[(e / cols) * ld + e % cols] = 0u;
}

int zero_words(void* dst, int64_t ld, int rows, int cols, hipStream_t s) {
  const int64_t n = (int64_t)rows * cols;
  if (n == 0) return LSQ_OK;
  zero_words_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<uint32_t*>(dst), ld, rows, cols);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int to_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t s) {
  LSQ_CHECK(n % 4 == 0, LSQ_ERR_SHAPE, "to_bf16: n %% 4 != 0");
  if (n == 0) return LSQ_OK;
  f32_to_bf16_kernel<<<(unsigned)((n / 4 + 255) / 256), 256, 0, s>>>(x, n, y);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int rope_table(int S, int head_dim, float theta, float* table, hipStream_t s) {
  const int half = head_dim / 2;
  if (S == 0) return LSQ_OK;
  rope_table_kernel<<<(S * half + 255) / 256, 256, 0, s>>>(S, half, (double)theta, reinterpret_cast<float2*>(table));
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int rope_apply(uint16_t* buf, int64_t ld, int T, int S, int n_rot_heads, int head_dim, const float* table, int inverse,
               hipStream_t s) {
  const int half = head_dim / 2;
  const int64_t total = (int64_t)T * n_rot_heads * half;
  if (total == 0) return LSQ_OK;
  rope_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(buf, ld, T, S, n_rot_heads, half,
                                                              reinterpret_cast<const float2*>(table), inverse);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

template <typename K>
int allow_smem(K* kernel, size_t bytes) {
  LSQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)bytes));
  return LSQ_OK;
}

size_t attention_prep_bytes(int B, int S, int nh, int nkv, int hd, bool bwd) {
  const PrepPtrs p = prep_ptrs(nullptr, B, S, nh, nkv, hd, bwd);
  const int64_t ekv = (int64_t)B * nkv * p.Sp * hd, eq = (int64_t)B * nh * p.Sp * hd;
  return (size_t)(2 * (bwd ? 4 * ekv + 4 * eq : 3 * ekv + 2 * eq));
}

int attention_fwd(const AttnArgs& a, int B, hipStream_t s) {
  LSQ_CHECK(a.hd == 64 || a.hd == 128, LSQ_ERR_SHAPE, "attention: head_dim %d unsupported (64 or 128)", a.hd);
  LSQ_CHECK(a.nkv > 0 && a.nh % a.nkv == 0, LSQ_ERR_SHAPE, "attention: n_heads %% n_kv_heads != 0");
  if (B == 0 || a.S == 0) return LSQ_OK;
  static int init = [] {
    int e = allow_smem(attn_fwd_bf16_kernel<128>, sizeof(AttnF16Smem<128>));
    return e ? e : allow_smem(attn_fwd_bf16_kernel<64>, sizeof(AttnF16Smem<64>));
  }();
  if (init) return init;
  LSQ_CHECK(a.prep, LSQ_ERR_WORKSPACE, "attention_fwd: prepared-operand workspace missing");
  const PrepPtrs pp = prep_ptrs(a.prep, B, a.S, a.nh, a.nkv, a.hd, false);
  dim3 grid((a.S + AT - 1) / AT, a.nh, B);
  const double flops = 2.0 * 2.0 * B * a.nh * (double)a.S * (a.S + 1) / 2.0 * a.hd;
  int tok = prof_begin(s);
  // Q and K rotated and split into hi/lo rows, and V^T: one launch
  const dim3 gp(pp.Sp / AT, a.nh + 2 * a.nkv, B);
  const RotOut oq{pp.qh, pp.ql, nullptr}, ok{pp.kh, pp.kl, nullptr};
  const QkvSrc qs{const_cast<float*>(a.qkv), a.qkv_part, a.qkv_splits, (int64_t)B * a.S * a.ld, a.ld, a.qkv_bias};
  if (a.hd == 128) {
    attn_prep_fwd_kernel<128><<<gp, 256, 0, s>>>(qs, a.ld, a.S, pp.Sp, a.nh, a.nkv, a.rope, oq, ok, pp.vt);
    attn_fwd_bf16_kernel<128><<<grid, 256, sizeof(AttnF16Smem<128>), s>>>(a, pp);
  } else {
    attn_prep_fwd_kernel<64><<<gp, 256, 0, s>>>(qs, a.ld, a.S, pp.Sp, a.nh, a.nkv, a.rope, oq, ok, pp.vt);
    attn_fwd_bf16_kernel<64><<<grid, 256, sizeof(AttnF16Smem<64>), s>>>(a, pp);
  }
  prof_end(tok, s, PROF_ATTN, flops, 0.0);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int attention_bwd(const AttnBwdArgs& a, int B, float* D, hipStream_t s) {
  LSQ_CHECK(a.hd == 64 || a.hd == 128, LSQ_ERR_SHAPE, "attention: head_dim %d unsupported", a.hd);
  if (B == 0 || a.S == 0) return LSQ_OK;
  static int init = [] {
    int e = allow_smem(attn_bwd_dkdv_bf16_kernel<128>, sizeof(AttnDkdvSmem<128>));
    if (!e) e = allow_smem(attn_bwd_dq_bf16_kernel<128>, sizeof(AttnDqSmem<128>));
    if (!e) e = allow_smem(attn_bwd_dkdv_bf16_kernel<64>, sizeof(AttnDkdvSmem<64>));
    if (!e) e = allow_smem(attn_bwd_dq_bf16_kernel<64>, sizeof(AttnDqSmem<64>));
    return e;
  }();
  if (init) return init;
  const double flops = 2.0 * 5.0 * B * a.nh * (double)a.S * (a.S + 1) / 2.0 * a.hd;
  int tok = prof_begin(s);
  AttnBwdArgs b = a;
  b.D = D;
  LSQ_CHECK(a.dk_part && a.dv_part && a.prep, LSQ_ERR_WORKSPACE, "attention_bwd: workspace buffers missing");
  const PrepPtrs pp = prep_ptrs(a.prep, B, a.S, a.nh, a.nkv, a.hd, true);
  dim3 g1((a.S + AT - 1) / AT, a.nh, B), g2((a.S + AT - 1) / AT, a.nh, B);
  // Q and K rotated, split and transposed, V rows, dO^T and D: one launch
  const dim3 gp(pp.Sp / AT, 2 * a.nh + 2 * a.nkv, B);
  const RotOut oq{pp.qh, pp.ql, pp.qht}, ok{pp.kh, pp.kl, pp.kht};
  const Bf16Src dos{const_cast<uint16_t*>(a.dO), a.dO_part, a.dO_splits, (int64_t)B * a.S * a.ldo};
  if (a.hd == 128) {
    attn_prep_bwd_kernel<128><<<gp, 256, 0, s>>>(a.qkv, a.ld, a.S, pp.Sp, a.nh, a.nkv, a.rope, oq, ok, pp.vr, dos,
                                                 a.O_f32, a.ldo, pp.ot, D);
    attn_bwd_dkdv_bf16_kernel<128><<<g1, 256, sizeof(AttnDkdvSmem<128>), s>>>(b, pp);
    attn_bwd_dq_bf16_kernel<128><<<g2, 256, sizeof(AttnDqSmem<128>), s>>>(b, pp);
  } else {
    attn_prep_bwd_kernel<64><<<gp, 256, 0, s>>>(a.qkv, a.ld, a.S, pp.Sp, a.nh, a.nkv, a.rope, oq, ok, pp.vr, dos,
                                                a.O_f32, a.ldo, pp.ot, D);
    attn_bwd_dkdv_bf16_kernel<64><<<g1, 256, sizeof(AttnDkdvSmem<64>), s>>>(b, pp);
    attn_bwd_dq_bf16_kernel<64><<<g2, 256, sizeof(AttnDqSmem<64>), s>>>(b, pp);
  }
  const int64_t nred = (int64_t)B * a.S * a.nkv * (a.hd / 2);
  attn_dkdv_reduce_kernel<<<(unsigned)((nred + 255) / 256), 256, 0, s>>>(b, B);
  prof_end(tok, s, PROF_ATTN, flops, 0.0);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int swiglu_fwd(const uint16_t* gu, int T, int I, uint16_t* m, hipStream_t s) {
  LSQ_CHECK(I % 8 == 0, LSQ_ERR_SHAPE, "swiglu: intermediate %d must be a multiple of 8", I);
  if ((int64_t)T * I == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  swiglu_fwd_kernel<<<dim3((unsigned)((I / 8 + 255) / 256), (unsigned)std::min(T, 65535)), 256, 0, s>>>(gu, T, I, m);
  prof_end(tok, s, PROF_ELEM, 0.0, 6.0 * T * (double)I);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int swiglu_bwd(const uint16_t* gu, const uint16_t* dm, int T, int I, uint16_t* dgu, hipStream_t s) {
  LSQ_CHECK(I % 8 == 0, LSQ_ERR_SHAPE, "swiglu: intermediate %d must be a multiple of 8", I);
  if ((int64_t)T * I == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  swiglu_bwd_kernel<<<dim3((unsigned)((I / 8 + 255) / 256), (unsigned)std::min(T, 65535)), 256, 0, s>>>(
      gu, dm, nullptr, 0, T, I, dgu);
  prof_end(tok, s, PROF_ELEM, 0.0, 10.0 * T * (double)I);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int splitk_swiglu_bwd(const uint16_t* gu, const float* dm_part, int splits, int T, int I, uint16_t* dgu,
                      hipStream_t s) {
  LSQ_CHECK(I % 8 == 0 && splits >= 1, LSQ_ERR_SHAPE, "swiglu: intermediate %d must be a multiple of 8", I);
  if ((int64_t)T * I == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  swiglu_bwd_kernel<<<dim3((unsigned)((I / 8 + 255) / 256), (unsigned)std::min(T, 65535)), 256, 0, s>>>(
      gu, nullptr, dm_part, splits, T, I, dgu);
  prof_end(tok, s, PROF_ELEM, 0.0, (8.0 + 4.0 * splits) * T * (double)I);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int embed_gather(const int32_t* ids, const uint16_t* table, int T, int H, int V, float* x, int32_t* bad, hipStream_t s) {
  LSQ_CHECK(H % 4 == 0, LSQ_ERR_SHAPE, "embed: hidden %% 4 != 0");
  const int64_t n = (int64_t)T * H / 4;
  if (n == 0) return LSQ_OK;
  const int tok = prof_begin(s);
  embed_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(ids, table, T, H, V, x, bad);
  prof_end(tok, s, PROF_ELEM, 0.0, 6.0 * T * (double)H + 4.0 * T);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int cross_entropy_rows(const float* logits, const int32_t* ids, int B, int S, int V, int row0, int nrows,
                       float* loss_rows, uint16_t* dlogits, uint16_t* dlogits_lo, hipStream_t s) {
  LSQ_CHECK(V % 4 == 0 && row0 >= 0 && nrows >= 0 && row0 + nrows <= B * S, LSQ_ERR_SHAPE, "cross_entropy: bad rows");
  if (nrows == 0) return LSQ_OK;
  const float inv_count = S > 1 ? 1.f / (float)(B * (S - 1)) : 0.f;
  const int tok = prof_begin(s);
  ce_kernel<<<nrows, kCeThreads, 0, s>>>(logits, ids, row0, S, V, inv_count, loss_rows, dlogits, dlogits_lo);
  prof_end(tok, s, PROF_ELEM, 0.0,
           (4.0 + (dlogits ? 2.0 : 0.0) + (dlogits_lo ? 2.0 : 0.0)) * nrows * (double)V + 8.0 * nrows);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int loss_mean(const float* loss_rows, int B, int S, float* loss, hipStream_t s) {
  const float inv_count = S > 1 ? 1.f / (float)(B * (S - 1)) : 0.f;
  loss_sum_kernel<<<1, 256, 0, s>>>(loss_rows, B * S, inv_count, loss);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

int cross_entropy(const float* logits, const int32_t* ids, int B, int S, int V, float* loss_rows, uint16_t* dlogits,
                  uint16_t* dlogits_lo, float* loss, hipStream_t s) {
  if (B * S == 0) return LSQ_OK;
  if (int e = cross_entropy_rows(logits, ids, B, S, V, 0, B * S, loss_rows, dlogits, dlogits_lo, s)) return e;
  return loss_mean(loss_rows, B, S, loss, s);
}

}  // namespace lsq
