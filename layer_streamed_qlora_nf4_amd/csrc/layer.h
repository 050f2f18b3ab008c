// Internal interface of the decoder layer (see layer.hip).
#pragma once
#include "common.h"

namespace lsq {

constexpr uint64_t kBlobHeader = 4096;   // bytes reserved at the start of every blob

struct Dims {
  int H, nh, nkv, hd, I, Nq, Nkv, Nqkv, r;
  int gN[4], gK[4];   // stacked linear groups: qkv, o, gate|up, down
};

int check_cfg(const lsq_model_cfg* c);
Dims dims_of(const lsq_model_cfg* c);
void blob_layout(const lsq_model_cfg* c, lsq_blob_layout* L);
void lora_layout(const lsq_model_cfg* c, lsq_lora_layout* L);
// keep: the forward activations live in a separate per-layer region of
// layer_acts_bytes (no recompute), so the workspace itself is smaller.
size_t layer_ws_bytes(const lsq_model_cfg* c, int B, int S, bool keep);
size_t layer_acts_bytes(const lsq_model_cfg* c, int B, int S);

// Called between the recompute (or, with kept activations, the start) and
// the backward proper of layer_bwd.
struct LayerHook {
  int (*after_recompute)(void* ctx);
  void* ctx;
};

// acts (nullable): this layer's kept-activation region.  layer_fwd fills it;
// layer_bwd then reads it instead of recomputing the forward.
int layer_fwd(const lsq_model_cfg* c, const void* blob, const void* lora, const float* x_in, int B, int S,
              float* x_out, void* ws, hipStream_t s, void* acts);
int layer_bwd(const lsq_model_cfg* c, const void* blob, const void* lora, const float* x_in, const float* dx_out,
              int B, int S, float* dx_in, float* grad, int accumulate, void* ws, hipStream_t s,
              const LayerHook* hook, void* acts);

}  // namespace lsq
