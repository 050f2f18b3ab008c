// Internal interface of the NF4-LoRA GEMM kernels (see gemm.hip).
#pragma once
#include "common.h"

namespace lsq {

enum Epi { EPI_BF16 = 0, EPI_F32 = 1, EPI_F32_RESID = 2 };

struct WeightRef {
  int kind;              // LSQ_W_NF4 / LSQ_W_BF16
  const void* data;      // packed [N, K/2] or bf16 [N, K]
  const float* absmax;   // [N, K/64]
  int N, K;
};

struct SegEnds {
  int end[4];
};

// Forward: out[M, N] = X[M, K] W^T + U[:, seg] Bl^T (+ bias) (+ resid).
// Columns [seg_end[s-1], seg_end[s]) use U columns [seg_ucol[s], seg_ucol[s] + r).
struct FwdParams {
  const uint16_t* X;
  int64_t ldx;
  int kind;
  const void* W;
  const float* absmax;
  int M, N, K;           // K: the reduction length over X's columns
  int Kw;                // the weight's columns: K, or K / 2 for X = [X_hi | X_lo], whose
                         // reduction steps past Kw read the weight again from column 0
                         // (Y = X_hi W^T + X_lo W^T); 0 means K
  const uint16_t* U;     // scaled down-projection, bf16 [M, ldu]; unused when r == 0
  int ldu;
  const uint16_t* Bl;    // [N, r]
  int r;
  int nseg;
  int seg_end[4];
  int seg_ucol[4];
  const uint16_t* bias;  // [N] or null
  const float* resid;    // [M, ldc] float32 (EPI_F32_RESID)
  void* out;
  int64_t ldc;
  float* part;           // split-K partials [splits, M, N] (workspace); set by gemm_fwd
  int splits;
  int bn;                // tile width in output columns; set by gemm_fwd
};

// Backward: out[M, K] = dY[M, N] W + G[M, rr] Al[rr, K] (+ resid).
struct BwdParams {
  const uint16_t* dY;
  int64_t ldy;
  int kind;
  const void* W;
  const float* absmax;
  int M, N, K;
  const uint16_t* G;     // scaled, bf16 [M, ldg]
  int64_t ldg;
  const uint16_t* Al;    // stacked A, bf16 [rr, K]
  int rr;
  const uint16_t* AlT;   // Al transposed [K, rr]: the LoRA term's operand (required when rr > 0)
  const float* resid;
  void* out;
  int64_t ldc;
  float* part;           // split-K partials [splits, M, K] (workspace); set by gemm_bwd
  int splits;
  int bo;                // tile width in output columns; set by gemm_bwd
};

// Split-K: a launch with fewer tiles than the chip has CUs splits its
// reduction into a fixed number of ranges (a pure function of the shape),
// writes float32 partials and sums them in split order in a second kernel.
// Forward plan: tile width (256, or 224 or 192 for the NF4 DMA kernels when
// that fills the rounds of workgroups better) and split count.  narrow: the
// launch can take a narrower tile (NF4 weights, operands within 32-bit
// offsets).  The workspace sizes cover the plans with and without narrow.
struct GemmPlan {
  int bn, splits;
};
GemmPlan gemm_fwd_plan(int M, int N, int K, bool narrow);
// Backward plan: output tile width (256, or 224 for the NF4 DMA kernel) and
// split count of the reduction over N.
GemmPlan gemm_bwd_plan(int M, int N, int K, bool narrow);
size_t gemm_fwd_ws_bytes(int M, int N, int K);
size_t gemm_bwd_ws_bytes(int M, int N, int K, int rr);

// ws: split-K partial buffer (>= the *_ws_bytes query), may be null when that is 0.
// With deferred_splits, a split-K launch leaves its float32 partials at the
// start of ws ([splits][M][out width]) for the caller to reduce (split_sum4
// order) and stores the split count there; 1 means the tile kernel wrote the
// output itself.
int gemm_fwd(const FwdParams& p, int epi, hipStream_t s, void* ws = nullptr, size_t ws_bytes = 0,
             int* deferred_splits = nullptr);
int gemm_bwd(const BwdParams& p, int epi, hipStream_t s, void* ws = nullptr, size_t ws_bytes = 0,
             int* deferred_splits = nullptr);
// ------------------------------------------------------------ rank-r kernels (lora.hip)
// Each product is one launch; where its reduction is split over workgroups,
// the last workgroup of a group to arrive sums the group's float32 partials
// in a fixed order.  cnt: that launch's arrival counters, which must be zero
// when it starts and are zero again when it ends (zero_counters once per
// workspace use; every launch leaves them as it found them).
size_t counters_bytes(int n);
int zero_counters(int* cnt, int n, hipStream_t s);

// U[M, rr] = bf16(s X A^T), A = stacked [rr, K]; U32 (nullable, ld ldu32)
// receives the same values before the bf16 rounding.
int lora_down_counters(int M);
size_t lora_down_ws_bytes(int M, int K, int rr);
int lora_down(const uint16_t* X, int64_t ldx, int M, int K, const uint16_t* A, int rr, float s, uint16_t* U,
              int64_t ldu, float* U32, int64_t ldu32, float* ws, size_t ws_bytes, int* cnt, hipStream_t st);
// G[M, s*r .. s*r + r) = bf16(s dY[:, seg s] B[seg s rows]) from Bt = B^T [r, N];
// G32 (nullable, ld ldg32) receives the unrounded values.
int lora_g_counters(int M, int nseg);
size_t lora_g_ws_bytes(int M, int N, int r);
int lora_g(const uint16_t* dY, int64_t ldy, int M, int N, const uint16_t* Bt, int r, int nseg, const SegEnds& segs,
           float s, uint16_t* G, int64_t ldg, float* G32, int64_t ldg32, float* ws, size_t ws_bytes, int* cnt,
           hipStream_t st);
// The adapter gradients of one linear group over the token dimension, from
// the unrounded float32 G and U: dA [nseg r, Kx] = G^T X (rows of the stacked
// group) and, per segment s of dY's columns, dB[seg rows] = dY_seg^T U_seg.
struct GradGroup {
  const float* G;
  int64_t ldg;
  const float* U;
  int64_t ldu;
  const uint16_t* X;
  int64_t ldx;
  const uint16_t* dY;
  int64_t ldy;
  int Kx, r, nseg;
  int seg_end[3];
  float* gA;
  float* gB;
};
int lora_grads_counters(int Kx, int r, int nseg, const int* seg_end);
size_t lora_grads_ws_bytes(int Kx, int r, int nseg, const int* seg_end, int M);
int lora_grads(const GradGroup& g, int M, int accumulate, float* ws, size_t ws_bytes, int* cnt, hipStream_t st);
// The adapters of n_layers consecutive layers transposed block by block
// (A [rr, K] -> [K, rr], B [N, r] -> [r, N]) into the same offsets of lora_t.
int adapter_transpose(const lsq_model_cfg* c, const uint16_t* lora, uint16_t* lora_t, int n_layers, hipStream_t st);

}  // namespace lsq
