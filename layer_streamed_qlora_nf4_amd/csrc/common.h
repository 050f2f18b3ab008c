// Internal helpers shared by the liblsq translation units (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string>

#include "../../include/lsq.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ errors
namespace lsq {
void set_error(const char* fmt, ...);
int fail(int code, const char* fmt, ...);
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
}  // namespace lsq

#define LSQ_HIP(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return lsq::fail(LSQ_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), \
                       __FILE__, __LINE__);                                            \
  } while (0)

#define LSQ_CHECK(cond, code, ...)              \
  do {                                          \
    if (!(cond)) return lsq::fail(code, __VA_ARGS__); \
  } while (0)

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// Two float32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}

// Sum over splits of a split-K launch's float32 partials part[s][e .. e + 3]
// (total elements per split apart), in split order; the loads go out four
// splits at a time.  Every kernel that consumes split-K partials sums them
// through this, so a fused consumer gives the same bits as the plain
// reduction.
__device__ __forceinline__ float4 split_sum4(const float* __restrict__ part, int splits, int64_t total, int64_t e) {
  float4 v = *reinterpret_cast<const float4*>(part + e);
  for (int sb = 1; sb < splits; sb += 4) {
    float4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (sb + j < splits) ? *reinterpret_cast<const float4*>(part + (int64_t)(sb + j) * total + e)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sb + j < splits) {
        v.x += w[j].x;
        v.y += w[j].y;
        v.z += w[j].z;
        v.w += w[j].w;
      }
  }
  return v;
}

// ------------------------------------------------------------------ timing hooks
namespace lsq {
// Kernel families credited by the profiler (lsq_prof_*).
enum ProfKind {
  PROF_GEMM_FWD = 0,   // NF4-weight tile kernels
  PROF_GEMM_BWD = 1,
  PROF_LORA = 2,
  PROF_ATTN = 3,
  PROF_OTHER = 4,
  PROF_GEMM_BF16 = 5,  // bf16-weight tile kernels (bf16 base, the head), both directions
  PROF_ELEM = 6,       // HBM-bound row and elementwise kernels (norms, SwiGLU, gather, cross-entropy)
  PROF_N = 7
};
bool prof_on();
// Returns an opaque token; prof_end credits flops/bytes to the family.
int prof_begin(hipStream_t s);
void prof_end(int token, hipStream_t s, ProfKind kind, double flops, double bytes);
// For one kernel launched with hipExtLaunchKernelGGL: the pair's events are
// handed out unrecorded (null when timing is off) and the launch attaches them
// to its dispatch, so they time the kernel's own execution.
int prof_begin_kernel(hipEvent_t* start, hipEvent_t* stop);
void prof_end_kernel(int token, ProfKind kind, double flops, double bytes);
}  // namespace lsq
