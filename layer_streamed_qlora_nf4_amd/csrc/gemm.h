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
  int M, N, K;
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
  const uint16_t* AlT;   // Al transposed [K, rr] (workspace; set by gemm_bwd)
  const float* resid;
  void* out;
  int64_t ldc;
  float* part;           // split-K partials [splits, M, K] (workspace); set by gemm_bwd
  int splits;
};

// Split-K: a launch with fewer tiles than the chip has CUs splits its
// reduction into a fixed number of ranges (a pure function of the shape),
// writes float32 partials and sums them in split order in a second kernel.
// Forward plan: tile width (256, or 192 for the NF4 DMA kernels when 256-wide
// tiles would leave a quarter of the CUs idle) and split count.  narrow: the
// launch can take the narrower tile (NF4 weights, operands within 32-bit
// offsets).  The split count does not depend on narrow.
struct GemmPlan {
  int bn, splits;
};
GemmPlan gemm_fwd_plan(int M, int N, int K, bool narrow);
int gemm_bwd_splits(int M, int N, int K, int rr);
size_t gemm_fwd_ws_bytes(int M, int N, int K);
size_t gemm_bwd_ws_bytes(int M, int N, int K, int rr);

// ws: split-K partial buffer (>= the *_ws_bytes query), may be null when that is 0.
int gemm_fwd(const FwdParams& p, int epi, hipStream_t s, void* ws = nullptr, size_t ws_bytes = 0);
int gemm_bwd(const BwdParams& p, int epi, hipStream_t s, void* ws = nullptr, size_t ws_bytes = 0);
// Reduction chunks of lora_g, each inside one segment.
struct GChunks {
  int begin[128], end[128];
  int n;
};

// U[M, rr] = bf16(s X A^T), A = stacked [rr, K]; ws holds the chunk partials.
// U32 (nullable, ld ldu32) receives the same values before the bf16 rounding.
size_t lora_down_ws_bytes(int M, int K, int rr);
int lora_down(const uint16_t* X, int64_t ldx, int M, int K, const uint16_t* A, int rr, float s, uint16_t* U,
              int64_t ldu, float* U32, int64_t ldu32, float* ws, size_t ws_bytes, hipStream_t st);
// G[M, s*r .. s*r + r) = bf16(s dY[:, seg s] B[seg s rows]); ws holds B transposed and partials.
// G32 (nullable, ld ldg32) receives the unrounded values.
size_t lora_g_ws_bytes(int M, int N, int r);
int lora_g(const uint16_t* dY, int64_t ldy, int M, int N, const uint16_t* B, int r, int nseg, const SegEnds& segs,
           float s, uint16_t* G, int64_t ldg, float* G32, int64_t ldg32, float* ws, size_t ws_bytes, hipStream_t st);
// One reduction over the token dimension, C = S^T L: S [M, ns] float32 (ns <=
// 64, a multiple of 8), L [M, nl] bf16; small_rows: out [ns, nl] (dA); else
// out [nl, ns] (dB).  The small side is the unrounded U or G.
struct TnTask {
  const float* S;
  int64_t lds;
  int ns;
  const uint16_t* L;
  int64_t ldl;
  int nl;
  float* out;
  int64_t ldo;
  int small_rows;
  int tile0;          // set by lora_grads
  int64_t part_off;   // set by lora_grads: this task's float32 partials in the workspace
};
struct TnBatch {
  TnTask t[8];
  int ntasks, M, accumulate;
  int splits, per;    // token ranges of `per` tokens (a multiple of 64); splits > 1 writes partials
  float* part;
};
struct SegFinish {
  int c0[4], c1[4], col[4];
  int n;
};
// Every task of one group in one launch.  Launches with few column tiles
// split the tokens into ranges whose float32 partials are summed in range
// order by a second kernel (a pure function of the shapes; fixed order).
size_t lora_grads_ws_bytes(const TnTask* tasks, int ntasks, int M);
int lora_grads(const TnTask* tasks, int ntasks, int M, int accumulate, float* ws, size_t ws_bytes, hipStream_t st);

// Token-dimension reduction C = S^T L (small_rows: [ns, nl]; else [nl, ns]).
size_t lora_tn_ws_bytes(int M, int ns, int nl);
int lora_tn(const float* S, int64_t lds_, int ns, const uint16_t* L, int64_t ldl, int nl, int M, bool small_rows,
            float* out, int64_t ldo, int accumulate, float* ws, size_t ws_bytes, hipStream_t st);

}  // namespace lsq
