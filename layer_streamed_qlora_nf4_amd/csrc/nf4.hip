// NF4 blockwise quantize / dequantize (gfx950).
//
// The shard store is written once, offline, quantising each frozen linear to
// NF4 as it goes (LS-docs "Shard cache"; About).  Format: 64-element blocks
// along a row, one float32 absmax per block, code = nearest NormalFloat-4
// level to fp32(x / absmax), even element in the high nibble.  These kernels
// are HBM-bound: 2 B read + 0.5625 B written per weight (quantize) and the
// reverse (dequantize).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "common.h"
#include "nf4_levels.h"

namespace {

struct Thresholds {
  float t[16];  // t[j] = largest float32 <= midpoint(level j, level j+1); t[15] unused
};

// x / a > t[j]  <=>  x / a lies strictly above the exact midpoint, for every
// float32 quotient: t[j] is the midpoint rounded toward -inf, so no float32
// value lies strictly between t[j] and the midpoint.  An exact tie therefore
// goes to the lower level.
Thresholds make_thresholds() {
  Thresholds th{};
  for (int j = 0; j < 15; ++j) {
    double m = (static_cast<double>(lsq::kNF4Levels[j]) + static_cast<double>(lsq::kNF4Levels[j + 1])) * 0.5;
    float t = static_cast<float>(m);
    if (static_cast<double>(t) > m) t = nextafterf(t, -INFINITY);
    th.t[j] = t;
  }
  th.t[15] = INFINITY;
  return th;
}

__device__ __forceinline__ uint32_t code_of(float n, const Thresholds& th) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (n > th.t[j]) ? 1u : 0u;
  return c;
}

// The 64 elements of block b as float32 (exact for bf16 input).
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ w, int64_t b, float (&x)[64]) {
  const uint4* src = reinterpret_cast<const uint4*>(w + b * 64);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = src[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = bf_lo(u[j]);       // the even element is the low half of its word
      x[8 * i + 2 * j + 1] = bf_hi(u[j]);
    }
  }
}
__device__ __forceinline__ void load_block(const float* __restrict__ w, int64_t b, float (&x)[64]) {
  const float4* src = reinterpret_cast<const float4*>(w + b * 64);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 v = src[i];
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
}

// One thread per 64-element block of bf16 or float32 input.
template <typename T>
__global__ void __launch_bounds__(256) nf4_quantize_kernel(const T* __restrict__ w, int64_t n_blocks,
                                                           uint8_t* __restrict__ packed, float* __restrict__ absmax,
                                                           int32_t* __restrict__ flag, Thresholds th) {
  int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  float x[64];
  load_block(w, b, x);
  float a = 0.f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    finite = finite && isfinite(x[i]);
    a = fmaxf(a, fabsf(x[i]));
  }
  if (!finite && flag) atomicOr(flag, 1);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e0 = x[8 * i + 2 * j], e1 = x[8 * i + 2 * j + 1];   // elements 2(4i+j) and 2(4i+j)+1
      uint32_t c0 = 7, c1 = 7;
      if (a > 0.f) {
        c0 = code_of(e0 / a, th);
        c1 = code_of(e1 / a, th);
      }
      word |= ((c0 << 4) | c1) << (8 * j);
    }
    out[i] = word;
  }
  uint4* dst = reinterpret_cast<uint4*>(packed + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  absmax[b] = a;
}

// Each wave dequantizes one 2048-weight segment in four passes; in pass q,
// lane l takes the 8 weights [512 q + 8 l, + 8) of the segment: one 4-byte
// load of packed codes and its block's absmax, one 16-byte (bf16) or two
// 16-byte (fp32) stores.  Every load and store instruction of a wave covers a
// contiguous range (256 B of codes in, 1 KiB or 2 KiB out).  n_w is a multiple
// of 64, so a lane's 8 weights are all in range or all out.
template <bool OUT_F32>
__global__ void __launch_bounds__(256) nf4_dequant_kernel(const uint8_t* __restrict__ packed,
                                                          const float* __restrict__ absmax, int64_t n_w,
                                                          void* __restrict__ out) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = lsq::kNF4LevelsDev[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t w0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2048 + lane * 8;
  uint32_t word[4];
  float a[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = w0 + q * 512;
    const bool ok = e < n_w;
    word[q] = ok ? *reinterpret_cast<const uint32_t*>(packed + e / 2) : 0u;
    a[q] = ok ? absmax[e >> 6] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = w0 + q * 512;
    if (e >= n_w) break;
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (word[q] >> (8 * j)) & 0xFF;
      v[2 * j] = lut[byte >> 4] * a[q];
      v[2 * j + 1] = lut[byte & 15] * a[q];
    }
    if (OUT_F32) {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + e);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + e) =
          make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
  }
}

// A word of device memory per GPU for the non-finite flag of calls that bring
// none (see nf4_quantize); its address is taken once per device.
__device__ int32_t g_nonfinite;
__global__ void clear_word_kernel(int32_t* w) { *w = 0; }

std::mutex g_flag_mu;   // such calls wait for their stream, so they are serialized
std::vector<int32_t*> g_flag_addr;

int nonfinite_word(int32_t** out) {
  int dev = 0;
  LSQ_HIP(hipGetDevice(&dev));
  if ((int)g_flag_addr.size() <= dev) g_flag_addr.resize(dev + 1, nullptr);
  if (!g_flag_addr[dev]) {
    void* p = nullptr;
    LSQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(g_nonfinite)));
    g_flag_addr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_flag_addr[dev];
  return LSQ_OK;
}

}  // namespace

namespace lsq {
int launch_nf4_quantize(const void* w, int32_t dtype, int64_t n_out, int64_t n_in, void* packed, float* absmax,
                        int32_t* flag, hipStream_t s) {
  static const Thresholds th = make_thresholds();
  int64_t n_blocks = n_out * (n_in / 64);
  if (n_blocks == 0) return LSQ_OK;
  dim3 grid(static_cast<unsigned>((n_blocks + 255) / 256));
  if (dtype == LSQ_F32)
    nf4_quantize_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(w), n_blocks,
                                                    static_cast<uint8_t*>(packed), absmax, flag, th);
  else
    nf4_quantize_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(w), n_blocks,
                                                       static_cast<uint8_t*>(packed), absmax, flag, th);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}
}  // namespace lsq

extern "C" {

void lsq_nf4_codebook(float out[16]) {
  for (int i = 0; i < 16; ++i) out[i] = lsq::kNF4Levels[i];
}

int nf4_quantize(const void* w_dev, int32_t dtype, int64_t n_out, int64_t n_in, int32_t blocksize, void* packed_dev,
                 float* absmax_dev, int32_t* flag_dev, void* stream) {
  LSQ_CHECK(w_dev && packed_dev && absmax_dev, LSQ_ERR_INVALID, "nf4_quantize: null pointer");
  LSQ_CHECK(dtype == LSQ_BF16 || dtype == LSQ_F32, LSQ_ERR_INVALID, "nf4_quantize: input dtype %d unsupported", dtype);
  LSQ_CHECK(blocksize == 64, LSQ_ERR_SHAPE, "nf4_quantize: blocksize %d unsupported (the store format uses 64)",
            blocksize);
  LSQ_CHECK(n_out >= 0 && n_in >= 0 && n_in % 64 == 0, LSQ_ERR_SHAPE,
            "nf4_quantize: n_in must be a multiple of 64 (got %lld x %lld)", (long long)n_out, (long long)n_in);
  LSQ_CHECK(lsq::aligned16(w_dev) && lsq::aligned16(packed_dev) && lsq::aligned16(absmax_dev), LSQ_ERR_ALIGN,
            "nf4_quantize: pointers must be 16-byte aligned");
  hipStream_t s = lsq::as_stream(stream);
  if (flag_dev) return lsq::launch_nf4_quantize(w_dev, dtype, n_out, n_in, packed_dev, absmax_dev, flag_dev, s);
  std::lock_guard<std::mutex> lock(g_flag_mu);
  int32_t* word = nullptr;
  if (int e = nonfinite_word(&word)) return e;
  clear_word_kernel<<<1, 1, 0, s>>>(word);
  LSQ_HIP(hipGetLastError());
  if (int e = lsq::launch_nf4_quantize(w_dev, dtype, n_out, n_in, packed_dev, absmax_dev, word, s)) return e;
  int32_t seen = 0;
  LSQ_HIP(hipMemcpyAsync(&seen, word, sizeof(seen), hipMemcpyDeviceToHost, s));
  LSQ_HIP(hipStreamSynchronize(s));
  LSQ_CHECK(seen == 0, LSQ_ERR_NONFINITE, "nf4_quantize: NaN or Inf in the input");
  return LSQ_OK;
}

int nf4_dequantize(const void* packed_dev, const float* absmax_dev, int64_t n_out, int64_t n_in, int32_t out_dtype,
                   void* w_out_dev, void* stream) {
  LSQ_CHECK(packed_dev && absmax_dev && w_out_dev, LSQ_ERR_INVALID, "nf4_dequantize: null pointer");
  LSQ_CHECK(out_dtype == LSQ_BF16 || out_dtype == LSQ_F32, LSQ_ERR_INVALID, "nf4_dequantize: bad dtype");
  LSQ_CHECK(n_out >= 0 && n_in >= 0 && n_in % 64 == 0, LSQ_ERR_SHAPE,
            "nf4_dequantize: n_in must be a multiple of 64");
  LSQ_CHECK(lsq::aligned16(packed_dev) && lsq::aligned16(absmax_dev) && lsq::aligned16(w_out_dev), LSQ_ERR_ALIGN,
            "nf4_dequantize: pointers must be 16-byte aligned");
  const int64_t n_w = n_out * n_in;
  if (n_w == 0) return LSQ_OK;
  dim3 grid(static_cast<unsigned>((n_w + 8191) / 8192));   // 4 waves x 2048 weights per block
  hipStream_t s = lsq::as_stream(stream);
  if (out_dtype == LSQ_F32)
    nf4_dequant_kernel<true><<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(packed_dev), absmax_dev, n_w, w_out_dev);
  else
    nf4_dequant_kernel<false><<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(packed_dev), absmax_dev, n_w, w_out_dev);
  LSQ_HIP(hipGetLastError());
  return LSQ_OK;
}

}  // extern "C"
