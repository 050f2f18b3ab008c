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
// A layer's rank-r store: its down projections U (bf16) and U32 (float32)
// from the forward, for the backward's recompute to reuse instead of
// recomputing them.
size_t layer_ustore_bytes(const lsq_model_cfg* c, int B, int S);

// Called between the recompute (or, with kept activations, the start) and
// the backward proper of layer_bwd.
struct LayerHook {
  int (*after_recompute)(void* ctx);
  void* ctx;
};

// Once per workspace use, before the first layer pass on it: the rotary
// table and the rank-r launches' arrival counters (zeroed).
int layer_prepare(const lsq_model_cfg* c, int B, int S, void* ws, hipStream_t s);
// acts (nullable): this layer's kept-activation region.  layer_fwd fills it;
// layer_bwd then reads it instead of recomputing the forward.  lora_t
// (nullable): the layer's adapters transposed block by block
// (adapter_transpose); null transposes them into the workspace first.
// ustore (nullable): the layer's rank-r store; layer_fwd fills it and a
// layer_bwd given the same store skips the recompute's down projections.
int layer_fwd(const lsq_model_cfg* c, const void* blob, const void* lora, const float* x_in, int B, int S,
              float* x_out, void* ws, hipStream_t s, void* acts, void* ustore = nullptr);
// Every layer_bwd leaves bf16(dx_in) in the workspace's bf16 gradient buffer
// (layer_bwd_dy_b: the same address in every backward carve of one
// workspace), which is the bf16 copy of dx_out the layer below starts from:
// with dy_b_ready, layer_bwd takes it as bf16(dx_out) instead of converting.
int layer_bwd(const lsq_model_cfg* c, const void* blob, const void* lora, const void* lora_t, const float* x_in,
              const float* dx_out, int B, int S, float* dx_in, float* grad, int accumulate, void* ws, hipStream_t s,
              const LayerHook* hook, void* acts, bool dy_b_ready = false, void* ustore = nullptr);
uint16_t* layer_bwd_dy_b(const lsq_model_cfg* c, int B, int S, void* ws);

}  // namespace lsq
