// Internal interface of the per-layer kernels (see layer_ops.hip).
#pragma once
#include "common.h"

namespace lsq {

// qkv: float32 [B*S, ld] with q heads | k heads | v heads per token row (q
// and k are rotated and split into bf16 hi/lo pairs once, by the prep
// kernels; v enters its products rounded to bf16).
struct AttnArgs {
  const float* qkv;
  int64_t ld;
  int S, nh, nkv, hd;
  float scale;
  uint16_t* out;    // [B*S, ldo], head h at column h*hd
  int64_t ldo;
  float* lse;       // [B, nh, S], base-2 log-sum-exp of the scaled scores
  const float2* rope;  // [S, hd/2] (cos, sin); q and k are rotated on load
  float* out_f32;      // nullable: the same output in float32 (kept for the backward)
  uint16_t* prep;      // attention_prep_bytes(.., false) of workspace
  // Optional: q/k/v not yet reduced.  With qkv_part set, the preparation sums
  // the q/k/v product's split-K partials [qkv_splits][B*S][ld] in split order,
  // adds qkv_bias (bf16, nullable) and stores the result into qkv, as the
  // plain reduction would, before using it.
  const float* qkv_part = nullptr;
  int qkv_splits = 0;
  const uint16_t* qkv_bias = nullptr;
};

struct AttnBwdArgs {
  const float* qkv;
  int64_t ld;
  int S, nh, nkv, hd;
  float scale;
  const uint16_t* O;    // forward output [B*S, ldo]
  const float* O_f32;   // the same in float32
  const uint16_t* dO;   // its gradient   [B*S, ldo]
  int64_t ldo;
  const float* lse;
  const float* D;       // [B*S, nh] rowsum(dO * O) (filled by attention_bwd)
  uint16_t* dqkv;       // [B*S, ld], same layout as qkv; dq, dk w.r.t. the unrotated q, k
  const float2* rope;
  float* dk_part;       // [B, nh, S, hd] per-query-head partials (workspace)
  float* dv_part;
  uint16_t* prep;       // attention_prep_bytes(.., true) of workspace
  // Optional: dO not yet reduced.  With dO_part set, the preparation sums the
  // split-K partials [dO_splits][B*S][ldo] of the product that makes dO in
  // split order, rounds them to bf16 and stores them into dO, as the plain
  // reduction would, before anything reads dO.
  const float* dO_part = nullptr;
  int dO_splits = 0;
};

// Workspace of the operands each attention call prepares once (rotated and
// split into bf16 hi/lo, or transposed, rows padded with zeros to a multiple
// of 64): Q, K and V^T for the forward; Q, K, the transposes of their bf16
// values, V and dO^T for the backward.
size_t attention_prep_bytes(int B, int S, int nh, int nkv, int hd, bool bwd);

// y [T, ldy] bf16 (and, with y_lo, the bf16 remainder at the same row pitch).
int rmsnorm_fwd(const float* x, const uint16_t* w, int T, int H, float eps, uint16_t* y, int64_t ldy, float* rstd,
                hipStream_t s, uint16_t* y_lo = nullptr);
int rmsnorm_bwd(const float* x, const uint16_t* w, const float* dy, const float* gres, int T, int H, float eps,
                float* dx, uint16_t* dx_b, hipStream_t s);
// The same row kernels fed by a GEMM's deferred split-K partials ([splits][T][H],
// summed in split order): h = resid + sum (stored), then y = rmsnorm(h); and
// the backward with dy = sum.  Bit-identical to the reduction followed by the
// plain kernel.
int splitk_resid_rmsnorm_fwd(const float* part, int splits, const float* resid, float* h, const uint16_t* w, int T,
                             int H, float eps, uint16_t* y, int64_t ldy, hipStream_t s);
int splitk_rmsnorm_bwd(const float* x, const uint16_t* w, const float* dy_part, int splits, const float* gres, int T,
                       int H, float eps, float* dx, uint16_t* dx_b, hipStream_t s);
int to_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t s);
// Zero rows x cols 32-bit words, row pitch ld words (a kernel, safe under graph capture).
int zero_words(void* dst, int64_t ld, int rows, int cols, hipStream_t s);
int rope_table(int S, int head_dim, float theta, float* table, hipStream_t s);
int rope_apply(uint16_t* buf, int64_t ld, int T, int S, int n_rot_heads, int head_dim, const float* table, int inverse,
               hipStream_t s);
int attention_fwd(const AttnArgs& a, int B, hipStream_t s);
int attention_bwd(const AttnBwdArgs& a, int B, float* D, hipStream_t s);
int swiglu_fwd(const uint16_t* gu, int T, int I, uint16_t* m, hipStream_t s);
int swiglu_bwd(const uint16_t* gu, const uint16_t* dm, int T, int I, uint16_t* dgu, hipStream_t s);
// dm = bf16(sum of a GEMM's deferred split-K partials [splits][T][I]).
int splitk_swiglu_bwd(const uint16_t* gu, const float* dm_part, int splits, int T, int I, uint16_t* dgu,
                      hipStream_t s);
int embed_gather(const int32_t* ids, const uint16_t* table, int T, int H, int V, float* x, int32_t* bad, hipStream_t s);
// dlogits (and, if non-null, dlogits_lo = bf16 of the remainder) for the head backward.
int cross_entropy(const float* logits, const int32_t* ids, int B, int S, int V, float* loss_rows, uint16_t* dlogits,
                  uint16_t* dlogits_lo, float* loss, hipStream_t s);
// One chunk of rows [row0, row0 + nrows): logits and dlogits hold just those
// rows; ids and loss_rows are indexed by the global token.
int cross_entropy_rows(const float* logits, const int32_t* ids, int B, int S, int V, int row0, int nrows,
                       float* loss_rows, uint16_t* dlogits, uint16_t* dlogits_lo, hipStream_t s);
// loss = mean of loss_rows over the B*(S-1) positions that have a target.
int loss_mean(const float* loss_rows, int B, int S, float* loss, hipStream_t s);

}  // namespace lsq
