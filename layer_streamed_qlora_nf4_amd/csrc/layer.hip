// One decoder layer over a shard ("blob") in device memory: layouts,
// forward, and backward with recompute.
//
// The pooled buffer is substituted into the unmodified layer, so the same
// kernels run on the same weight bytes whether the blob sits in a streaming
// slot or in a resident arena (LS-docs "How it works").  The backward
// recomputes the layer from its saved input (LS-docs "How it works": each
// layer is read twice per step) and reads the blob until its last GEMM.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "layer.h"
#include "layer_ops.h"

namespace lsq {

static uint64_t up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int check_cfg(const lsq_model_cfg* c) {
  LSQ_CHECK(c, LSQ_ERR_INVALID, "model cfg: null");
  LSQ_CHECK(c->hidden > 0 && c->hidden % 64 == 0 && c->n_heads > 0 && c->n_kv_heads > 0 &&
                c->n_heads % c->n_kv_heads == 0 && (c->head_dim == 64 || c->head_dim == 128) &&
                c->intermediate > 0 && c->intermediate % 64 == 0 && c->vocab > 0 && c->vocab % 8 == 0 &&
                c->n_layers > 0,
            LSQ_ERR_SHAPE,
            "model cfg: need hidden, intermediate multiples of 64, head_dim 64/128, heads divisible, vocab %% 8 == 0");
  LSQ_CHECK((c->n_heads * c->head_dim) % 64 == 0, LSQ_ERR_SHAPE, "model cfg: n_heads*head_dim %% 64 != 0");
  LSQ_CHECK(c->hidden <= 8192, LSQ_ERR_SHAPE, "model cfg: hidden %d above 8192 (RMSNorm keeps a row in registers)",
            c->hidden);
  LSQ_CHECK(c->weight_kind == LSQ_W_NF4 || c->weight_kind == LSQ_W_BF16, LSQ_ERR_INVALID, "model cfg: weight_kind");
  LSQ_CHECK(c->lora_r >= 8 && c->lora_r <= 64 && c->lora_r % 8 == 0, LSQ_ERR_SHAPE,
            "model cfg: lora_r must be 8..64 and a multiple of 8 (got %d)", c->lora_r);
  LSQ_CHECK(c->rms_eps > 0 && c->rope_theta > 0, LSQ_ERR_INVALID, "model cfg: eps / theta");
  LSQ_CHECK(c->loss_chunk >= 0, LSQ_ERR_INVALID, "model cfg: loss_chunk must be >= 0 (0 = all tokens)");
  return LSQ_OK;
}

Dims dims_of(const lsq_model_cfg* c) {
  Dims d;
  d.H = c->hidden;
  d.nh = c->n_heads;
  d.nkv = c->n_kv_heads;
  d.hd = c->head_dim;
  d.I = c->intermediate;
  d.Nq = d.nh * d.hd;
  d.Nkv = d.nkv * d.hd;
  d.Nqkv = d.Nq + 2 * d.Nkv;
  d.r = c->lora_r;
  d.gN[0] = d.Nqkv;
  d.gK[0] = d.H;
  d.gN[1] = d.H;
  d.gK[1] = d.Nq;
  d.gN[2] = 2 * d.I;
  d.gK[2] = d.H;
  d.gN[3] = d.H;
  d.gK[3] = d.I;
  return d;
}

void blob_layout(const lsq_model_cfg* c, lsq_blob_layout* L) {
  const Dims d = dims_of(c);
  uint64_t off = kBlobHeader;
  for (int g = 0; g < 4; ++g) {
    const uint64_t n = (uint64_t)d.gN[g] * d.gK[g];
    L->w_off[g] = off;
    off = up(off + (c->weight_kind == LSQ_W_NF4 ? n / 2 : n * 2), 4096);
  }
  for (int g = 0; g < 4; ++g) {
    if (c->weight_kind == LSQ_W_NF4) {
      L->absmax_off[g] = off;
      off = up(off + (uint64_t)d.gN[g] * (d.gK[g] / 64) * 4, 4096);
    } else {
      L->absmax_off[g] = 0;
    }
  }
  L->norm1_off = off;
  off = up(off + 2ull * d.H, 256);
  L->norm2_off = off;
  off = up(off + 2ull * d.H, 256);
  if (c->qkv_bias) {
    L->bias_off = off;
    off = up(off + 2ull * d.Nqkv, 256);
  } else {
    L->bias_off = 0;
  }
  L->total_bytes = up(off, 4096);
}

void lora_layout(const lsq_model_cfg* c, lsq_lora_layout* L) {
  const Dims d = dims_of(c);
  const uint64_t r = d.r;
  const uint64_t a_rows[4] = {3 * r, r, 2 * r, r};
  uint64_t off = 0;
  for (int g = 0; g < 4; ++g) {
    L->a_off[g] = off;
    off = up(off + a_rows[g] * d.gK[g], 128);
  }
  for (int g = 0; g < 4; ++g) {
    L->b_off[g] = off;
    off = up(off + (uint64_t)d.gN[g] * r, 128);
  }
  L->layer_elems = off;
}

// ------------------------------------------------------------------ workspace
// Buffers of one layer pass, carved from the caller's workspace in a fixed order.
struct LayerWs {
  float* rope;        // [S, hd/2] (cos, sin)
  uint16_t* xn1;      // [T, 2H]: the normed input as bf16 (columns [0, H)) and the
                      // bf16 rounding of its remainder (columns [H, 2H))
  uint16_t* U_qkv;    // [T, 3r]
  float* qkv;         // [T, Nqkv] float32
  uint16_t* attn;     // [T, Nq]
  float* lse;         // [B, nh, S]
  uint16_t* U_o;      // [T, r]
  float* h;           // [T, H]
  uint16_t* xn2;      // [T, H]
  uint16_t* U_gu;     // [T, 2r]
  uint16_t* gu;       // [T, 2I]
  uint16_t* m;        // [T, I]
  uint16_t* U_d;      // [T, r]
  // backward only
  float* U32[4];      // unrounded U of each group (adapter-gradient inputs)
  float* G32;         // [T, 3r] unrounded G
  float* attn_f32;    // [T, Nq] attention output in float32 (recompute pass)
  uint16_t* dy_b;     // [T, H] bf16 copy of an upstream residual gradient
  uint16_t* G;        // [T, 3r]
  uint16_t* dm;       // [T, I]
  uint16_t* dgu;      // [T, 2I]
  float* dxn;         // [T, H]
  float* dh;          // [T, H]
  uint16_t* dattn;    // [T, Nq]
  float* D;           // [T, nh]
  uint16_t* dqkv;     // [T, Nqkv]
  float* dk_part;     // [T, nh, hd] per-query-head dK, dV partials
  float* dv_part;
  uint16_t* aprep;    // attention operands prepared once per call
  float* lws;         // partials of the LoRA down / G projections
  size_t lws_bytes;
  float* tn;          // partials of the adapter-gradient token reduction
  size_t tn_bytes;
  int* cnt;           // arrival counters of the rank-r launches
  int ncnt;
  uint16_t* lora_t;   // backward: this layer's adapters transposed (when the caller has none)
  void* gemm;         // split-K partials of the layer's GEMMs
  size_t gemm_bytes;
  size_t total;
};

static size_t gemm_need(const Dims& d, int T) {
  size_t m = 0;
  for (int g = 0; g < 4; ++g) {
    const int rr = (g == 0 ? 3 : g == 2 ? 2 : 1) * d.r;
    // the q/k/v group reduces over its input's bf16 hi and lo halves (2H)
    m = std::max(m, gemm_fwd_ws_bytes(T, d.gN[g], g == 0 ? 2 * d.gK[g] : d.gK[g]));
    m = std::max(m, gemm_bwd_ws_bytes(T, d.gN[g], d.gK[g], rr));
  }
  return m;
}

// The four groups' adapter-gradient reductions: (stacked rank segments, input
// width, segment ends of the output columns).
struct GroupShape {
  int nseg, Kx;
  int seg_end[3];
};
static void group_shapes(const Dims& d, GroupShape (&g)[4]) {
  g[0] = GroupShape{3, d.H, {d.Nq, d.Nq + d.Nkv, d.Nqkv}};
  g[1] = GroupShape{1, d.Nq, {d.H, 0, 0}};
  g[2] = GroupShape{2, d.H, {d.I, 2 * d.I, 0}};
  g[3] = GroupShape{1, d.I, {d.H, 0, 0}};
}

static size_t tn_need(const Dims& d, int T) {
  GroupShape g[4];
  group_shapes(d, g);
  size_t m = 0;
  for (const auto& x : g) m = std::max(m, lora_grads_ws_bytes(x.Kx, d.r, x.nseg, x.seg_end, T));
  return m;
}

// Arrival counters: the most any one rank-r launch of the layer uses.
static int counters_need(const Dims& d, int T) {
  GroupShape g[4];
  group_shapes(d, g);
  int n = std::max(lora_down_counters(T), lora_g_counters(T, 3));
  for (const auto& x : g) n = std::max(n, lora_grads_counters(x.Kx, d.r, x.nseg, x.seg_end));
  return n;
}

static size_t lws_need(const Dims& d, int T) {
  size_t m = 0;
  for (int g = 0; g < 4; ++g) {
    const int rr = (g == 0 ? 3 : g == 2 ? 2 : 1) * d.r;
    m = std::max(m, lora_down_ws_bytes(T, d.gK[g], rr));
    m = std::max(m, lora_g_ws_bytes(T, d.gN[g], d.r));
  }
  return m;
}

// The forward activations the backward reads (xn1 .. U_d, the unrounded U and
// the float32 attention output) come from `acts` when the caller keeps them
// per layer (no recompute), else from the workspace itself.  keep: a region
// size query for that split (base and acts may both be null).
// ustore (nullable): the layer's rank-r inputs U (bf16) and U32 (float32),
// kept from its forward for the backward's recompute, which then skips the
// down projections (layer_ustore_bytes).
static LayerWs carve(const lsq_model_cfg* c, int B, int S, void* base, bool bwd, void* acts = nullptr,
                     bool keep = false, uint64_t* acts_total = nullptr, void* ustore = nullptr,
                     uint64_t* ustore_total = nullptr) {
  const Dims d = dims_of(c);
  const uint64_t T = (uint64_t)B * S;
  keep = keep || acts != nullptr;
  LayerWs w{};
  char* p = static_cast<char*>(base);
  char* pa = static_cast<char*>(acts);
  uint64_t off = 0, aoff = 0;
  auto take = [&](uint64_t bytes) -> void* {
    void* r = base ? p + off : nullptr;
    off = up(off + std::max<uint64_t>(bytes, 1), 256);
    return r;
  };
  auto take_act = [&](uint64_t bytes) -> void* {
    if (!keep) return take(bytes);
    void* r = acts ? pa + aoff : nullptr;
    aoff = up(aoff + std::max<uint64_t>(bytes, 1), 256);
    return r;
  };
  char* pu = static_cast<char*>(ustore);
  uint64_t uoff = 0;
  auto take_u = [&](uint64_t bytes) -> void* {
    if (!ustore) return take_act(bytes);
    void* r = pu + uoff;
    uoff = up(uoff + std::max<uint64_t>(bytes, 1), 256);
    return r;
  };
  // rope and the counters first: the same addresses in every carve of one
  // workspace (forward or backward, kept activations or not), so one
  // layer_prepare serves every pass
  w.rope = static_cast<float*>(take(8ull * S * (d.hd / 2)));
  w.ncnt = counters_need(d, (int)T);
  w.cnt = static_cast<int*>(take(counters_bytes(w.ncnt)));
  // the backward's bf16 upstream gradient next, so that it too has one
  // address in every backward carve and one layer can hand it to the next
  if (bwd) w.dy_b = static_cast<uint16_t*>(take(2 * T * d.H));
  w.xn1 = static_cast<uint16_t*>(take_act(2 * T * 2 * d.H));
  w.U_qkv = static_cast<uint16_t*>(take_u(2 * T * 3 * d.r));
  w.qkv = static_cast<float*>(take_act(4 * T * d.Nqkv));
  w.attn = static_cast<uint16_t*>(take_act(2 * T * d.Nq));
  w.lse = static_cast<float*>(take_act(4ull * B * d.nh * S));
  w.U_o = static_cast<uint16_t*>(take_u(2 * T * d.r));
  w.h = static_cast<float*>(take_act(4 * T * d.H));
  w.xn2 = static_cast<uint16_t*>(take_act(2 * T * d.H));
  w.U_gu = static_cast<uint16_t*>(take_u(2 * T * 2 * d.r));
  w.gu = static_cast<uint16_t*>(take_act(2 * T * 2 * d.I));
  w.m = static_cast<uint16_t*>(take_act(2 * T * d.I));
  w.U_d = static_cast<uint16_t*>(take_u(2 * T * d.r));
  if (bwd || keep || ustore) {
    const int ur[4] = {3, 1, 2, 1};
    for (int g = 0; g < 4; ++g) w.U32[g] = static_cast<float*>(take_u(4 * T * ur[g] * d.r));
  }
  if (bwd || keep) w.attn_f32 = static_cast<float*>(take_act(4 * T * d.Nq));
  if (acts_total) *acts_total = aoff;
  if (ustore_total) *ustore_total = uoff;
  w.gemm_bytes = gemm_need(d, (int)T);
  w.gemm = take(w.gemm_bytes);
  w.lws_bytes = lws_need(d, (int)T);
  w.lws = static_cast<float*>(take(w.lws_bytes));
  w.aprep = static_cast<uint16_t*>(take(attention_prep_bytes(B, S, d.nh, d.nkv, d.hd, bwd)));
  if (bwd) {
    w.G32 = static_cast<float*>(take(4 * T * 3 * d.r));
    w.G = static_cast<uint16_t*>(take(2 * T * 3 * d.r));
    w.dm = static_cast<uint16_t*>(take(2 * T * d.I));
    w.dgu = static_cast<uint16_t*>(take(2 * T * 2 * d.I));
    w.dxn = static_cast<float*>(take(4 * T * d.H));
    w.dh = static_cast<float*>(take(4 * T * d.H));
    w.dattn = static_cast<uint16_t*>(take(2 * T * d.Nq));
    w.D = static_cast<float*>(take(4 * T * d.nh));
    w.dqkv = static_cast<uint16_t*>(take(2 * T * d.Nqkv));
    w.dk_part = static_cast<float*>(take(4 * T * d.nh * d.hd));
    w.dv_part = static_cast<float*>(take(4 * T * d.nh * d.hd));
    w.tn_bytes = tn_need(d, (int)T);
    w.tn = static_cast<float*>(take(w.tn_bytes));
    lsq_lora_layout LL;
    lora_layout(c, &LL);
    w.lora_t = static_cast<uint16_t*>(take(2 * LL.layer_elems));
  }
  w.total = off;
  return w;
}

size_t layer_ws_bytes(const lsq_model_cfg* c, int B, int S, bool keep) {
  return carve(c, B, S, nullptr, true, nullptr, keep).total;
}
size_t layer_acts_bytes(const lsq_model_cfg* c, int B, int S) {
  uint64_t a = 0;
  carve(c, B, S, nullptr, true, nullptr, true, &a);
  return a;
}
size_t layer_ustore_bytes(const lsq_model_cfg* c, int B, int S) {
  uint64_t u = 0;
  char probe;   // any non-null address: only the offsets are used
  carve(c, B, S, nullptr, true, nullptr, false, nullptr, &probe, &u);
  return u;
}

struct BlobView {
  WeightRef w[4];
  const uint16_t* norm1;
  const uint16_t* norm2;
  const uint16_t* bias;
};

static BlobView view_blob(const lsq_model_cfg* c, const void* blob) {
  lsq_blob_layout L;
  blob_layout(c, &L);
  const Dims d = dims_of(c);
  const char* b = static_cast<const char*>(blob);
  BlobView v;
  for (int g = 0; g < 4; ++g)
    v.w[g] = WeightRef{c->weight_kind, b + L.w_off[g],
                       c->weight_kind == LSQ_W_NF4 ? reinterpret_cast<const float*>(b + L.absmax_off[g]) : nullptr,
                       d.gN[g], d.gK[g]};
  v.norm1 = reinterpret_cast<const uint16_t*>(b + L.norm1_off);
  v.norm2 = reinterpret_cast<const uint16_t*>(b + L.norm2_off);
  v.bias = c->qkv_bias ? reinterpret_cast<const uint16_t*>(b + L.bias_off) : nullptr;
  return v;
}

// A layer's adapters (A [rr, K], B [N, r] per group) and, for the backward,
// their transposed copies (A^T [K, rr], B^T [r, N]) at the same offsets.
struct LoraView {
  const uint16_t* A[4];
  const uint16_t* B[4];
  const uint16_t* AT[4];
  const uint16_t* BT[4];
};
static LoraView view_lora(const lsq_model_cfg* c, const void* lora, const void* lora_t = nullptr) {
  lsq_lora_layout L;
  lora_layout(c, &L);
  const uint16_t* p = static_cast<const uint16_t*>(lora);
  const uint16_t* t = static_cast<const uint16_t*>(lora_t);
  LoraView v{};
  for (int g = 0; g < 4; ++g) {
    v.A[g] = p + L.a_off[g];
    v.B[g] = p + L.b_off[g];
    if (t) {
      v.AT[g] = t + L.a_off[g];
      v.BT[g] = t + L.b_off[g];
    }
  }
  return v;
}

static FwdParams fwd_params(const uint16_t* X, int T, const WeightRef& w, const uint16_t* U, int ldu,
                            const uint16_t* Bl, int r) {
  FwdParams p{};
  p.X = X;
  p.ldx = w.K;
  p.kind = w.kind;
  p.W = w.data;
  p.absmax = w.absmax;
  p.M = T;
  p.N = w.N;
  p.K = w.K;
  p.U = U;
  p.ldu = ldu;
  p.Bl = Bl;
  p.r = r;
  p.nseg = 1;
  p.seg_end[0] = w.N;
  p.seg_ucol[0] = 0;
  p.ldc = w.N;
  return p;
}

static BwdParams bwd_params(const uint16_t* dY, int T, const WeightRef& w, const uint16_t* G, int ldg,
                            const uint16_t* Al, const uint16_t* AlT, int rr) {
  BwdParams p{};
  p.dY = dY;
  p.ldy = w.N;
  p.kind = w.kind;
  p.W = w.data;
  p.absmax = w.absmax;
  p.M = T;
  p.N = w.N;
  p.K = w.K;
  p.G = G;
  p.ldg = ldg;
  p.Al = Al;
  p.AlT = AlT;
  p.rr = rr;
  p.ldc = w.K;
  return p;
}

#define TRY(x)                 \
  do {                         \
    if (int e_ = (x)) return e_; \
  } while (0)

// Forward through the layer.  x_out == nullptr stops after the MLP activation
// and its down-projection input U_d (the part of the forward the backward reads).
// u_ready: U and U32 already hold this layer's down projections (kept from
// its forward in the layer's rank-r store), so the recompute skips them; the
// kernels are deterministic, so the values are the ones it would recompute.
static int forward_impl(const lsq_model_cfg* c, const BlobView& bv, const LoraView& lv, const float* x_in, int B,
                        int S, float* x_out, const LayerWs& w, hipStream_t s, bool u_ready = false) {
  const Dims d = dims_of(c);
  const int T = B * S, r = d.r;
  const float sc = c->lora_scale;
  // attention block.  q and k decide the attention weights, whose error grows
  // with the scores' magnitude: the q/k/v product takes the normed input as a
  // bf16 hi/lo pair (two passes over one weight) and keeps its output in
  // float32.  The adapters' down-projection and gradient read the hi half.
  TRY(rmsnorm_fwd(x_in, bv.norm1, T, d.H, c->rms_eps, w.xn1, 2 * d.H, nullptr, s, w.xn1 + d.H));
  if (!u_ready)
    TRY(lora_down(w.xn1, 2 * d.H, T, d.H, lv.A[0], 3 * r, sc, w.U_qkv, 3 * r, w.U32[0], 3 * r, w.lws, w.lws_bytes,
                  w.cnt, s));
  {
    FwdParams p = fwd_params(w.xn1, T, bv.w[0], w.U_qkv, 3 * r, lv.B[0], r);
    p.ldx = 2 * d.H;
    p.K = 2 * d.H;
    p.Kw = d.H;
    p.nseg = 3;
    p.seg_end[0] = d.Nq;
    p.seg_end[1] = d.Nq + d.Nkv;
    p.seg_end[2] = d.Nqkv;
    p.seg_ucol[0] = 0;
    p.seg_ucol[1] = r;
    p.seg_ucol[2] = 2 * r;
    p.bias = bv.bias;
    p.out = w.qkv;
    // a split-K launch leaves its partials to the attention's operand
    // preparation, which sums them (plus the bias) and writes q/k/v on the way
    int sp = 1;
    TRY(gemm_fwd(p, EPI_F32, s, w.gemm, w.gemm_bytes, &sp));
    AttnArgs a{w.qkv, d.Nqkv, S, d.nh, d.nkv, d.hd, 1.0f / sqrtf((float)d.hd), w.attn, d.Nq, w.lse,
               reinterpret_cast<const float2*>(w.rope), w.attn_f32, w.aprep};
    if (sp > 1) {
      a.qkv_part = static_cast<const float*>(w.gemm);
      a.qkv_splits = sp;
      a.qkv_bias = bv.bias;
    }
    TRY(attention_fwd(a, B, s));
  }
  if (!u_ready)
    TRY(lora_down(w.attn, d.Nq, T, d.Nq, lv.A[1], r, sc, w.U_o, r, w.U32[1], r, w.lws, w.lws_bytes, w.cnt, s));
  // h = x + o(attn) and the MLP's RMSNorm; a split-K o projection leaves its
  // partials to the norm kernel, which sums them (and writes h) on the way in
  {
    FwdParams p = fwd_params(w.attn, T, bv.w[1], w.U_o, r, lv.B[1], r);
    p.resid = x_in;
    p.out = w.h;
    int sp = 1;
    TRY(gemm_fwd(p, EPI_F32_RESID, s, w.gemm, w.gemm_bytes, &sp));
    if (sp > 1)
      TRY(splitk_resid_rmsnorm_fwd(static_cast<const float*>(w.gemm), sp, x_in, w.h, bv.norm2, T, d.H, c->rms_eps,
                                   w.xn2, d.H, s));
    else
      TRY(rmsnorm_fwd(w.h, bv.norm2, T, d.H, c->rms_eps, w.xn2, d.H, nullptr, s));
  }
  // MLP block
  if (!u_ready)
    TRY(lora_down(w.xn2, d.H, T, d.H, lv.A[2], 2 * r, sc, w.U_gu, 2 * r, w.U32[2], 2 * r, w.lws, w.lws_bytes, w.cnt,
                  s));
  {
    FwdParams p = fwd_params(w.xn2, T, bv.w[2], w.U_gu, 2 * r, lv.B[2], r);
    p.nseg = 2;
    p.seg_end[0] = d.I;
    p.seg_end[1] = 2 * d.I;
    p.seg_ucol[0] = 0;
    p.seg_ucol[1] = r;
    p.out = w.gu;
    TRY(gemm_fwd(p, EPI_BF16, s, w.gemm, w.gemm_bytes));
  }
  TRY(swiglu_fwd(w.gu, T, d.I, w.m, s));
  if (!u_ready)
    TRY(lora_down(w.m, d.I, T, d.I, lv.A[3], r, sc, w.U_d, r, w.U32[3], r, w.lws, w.lws_bytes, w.cnt, s));
  if (x_out) {
    FwdParams p = fwd_params(w.m, T, bv.w[3], w.U_d, r, lv.B[3], r);
    p.resid = w.h;
    p.out = x_out;
    TRY(gemm_fwd(p, EPI_F32_RESID, s, w.gemm, w.gemm_bytes));
  }
  return LSQ_OK;
}

// dA of the stacked group (G^T X) and dB of each segment (dY_seg^T U_seg), in
// one launch, from the unrounded float32 G and U.
static int adapter_grads(const Dims& d, int T, const float* G, int ldg, const float* U, int ldu,
                         const uint16_t* X, int64_t ldx, int Kx, const uint16_t* dY, int ldy, int nseg,
                         const int* seg_end, float* gA, float* gB, int accumulate, const LayerWs& w, hipStream_t s) {
  GradGroup g{};
  g.G = G;
  g.ldg = ldg;
  g.U = U;
  g.ldu = ldu;
  g.X = X;
  g.ldx = ldx;
  g.dY = dY;
  g.ldy = ldy;
  g.Kx = Kx;
  g.r = d.r;
  g.nseg = nseg;
  for (int i = 0; i < nseg; ++i) g.seg_end[i] = seg_end[i];
  g.gA = gA;
  g.gB = gB;
  return lora_grads(g, T, accumulate, w.tn, w.tn_bytes, w.cnt, s);
}

static int backward_impl(const lsq_model_cfg* c, const BlobView& bv, const LoraView& lv, const float* x_in,
                         const float* dx_out, int B, int S, float* dx_in, float* grad, int accumulate,
                         const LayerWs& w, hipStream_t s, bool dy_b_ready) {
  const Dims d = dims_of(c);
  const int T = B * S, r = d.r;
  const float sc = c->lora_scale;
  lsq_lora_layout L;
  lora_layout(c, &L);
  float* gA[4];
  float* gB[4];
  for (int g = 0; g < 4; ++g) {
    gA[g] = grad + L.a_off[g];
    gB[g] = grad + L.b_off[g];
  }
  SegEnds one{};
  // ---- down projection: out = h + down(m)
  if (!dy_b_ready) TRY(to_bf16(dx_out, (int64_t)T * d.H, w.dy_b, s));
  one.end[0] = d.H;
  TRY(lora_g(w.dy_b, d.H, T, d.H, lv.BT[3], r, 1, one, sc, w.G, r, w.G32, r, w.lws, w.lws_bytes, w.cnt, s));
  // dm, and through SwiGLU dgu; a split-K launch leaves dm's partials to the
  // SwiGLU kernel
  {
    BwdParams p = bwd_params(w.dy_b, T, bv.w[3], w.G, r, lv.A[3], lv.AT[3], r);
    p.out = w.dm;
    int sp = 1;
    TRY(gemm_bwd(p, EPI_BF16, s, w.gemm, w.gemm_bytes, &sp));
    if (sp > 1)
      TRY(splitk_swiglu_bwd(w.gu, static_cast<const float*>(w.gemm), sp, T, d.I, w.dgu, s));
    else
      TRY(swiglu_bwd(w.gu, w.dm, T, d.I, w.dgu, s));
  }
  {
    const int se[1] = {d.H};
    TRY(adapter_grads(d, T, w.G32, r, w.U32[3], r, w.m, d.I, d.I, w.dy_b, d.H, 1, se, gA[3], gB[3], accumulate, w, s));
  }
  // ---- gate/up
  SegEnds two{};
  two.end[0] = d.I;
  two.end[1] = 2 * d.I;
  TRY(lora_g(w.dgu, 2 * d.I, T, 2 * d.I, lv.BT[2], r, 2, two, sc, w.G, 2 * r, w.G32, 2 * r, w.lws, w.lws_bytes,
             w.cnt, s));
  // dxn2, then dh = dout + rmsnorm2'(dxn2) (from the partials of a split-K launch)
  {
    BwdParams p = bwd_params(w.dgu, T, bv.w[2], w.G, 2 * r, lv.A[2], lv.AT[2], 2 * r);
    p.out = w.dxn;
    int sp = 1;
    TRY(gemm_bwd(p, EPI_F32, s, w.gemm, w.gemm_bytes, &sp));
    if (sp > 1)
      TRY(splitk_rmsnorm_bwd(w.h, bv.norm2, static_cast<const float*>(w.gemm), sp, dx_out, T, d.H, c->rms_eps, w.dh,
                             w.dy_b, s));
    else
      TRY(rmsnorm_bwd(w.h, bv.norm2, w.dxn, dx_out, T, d.H, c->rms_eps, w.dh, w.dy_b, s));
  }
  {
    const int se[2] = {d.I, 2 * d.I};
    TRY(adapter_grads(d, T, w.G32, 2 * r, w.U32[2], 2 * r, w.xn2, d.H, d.H, w.dgu, 2 * d.I, 2, se, gA[2], gB[2], accumulate,
                      w, s));
  }
  // ---- o projection
  one.end[0] = d.H;
  TRY(lora_g(w.dy_b, d.H, T, d.H, lv.BT[1], r, 1, one, sc, w.G, r, w.G32, r, w.lws, w.lws_bytes, w.cnt, s));
  // d_attn; a split-K launch leaves its partials to the attention backward's
  // operand preparation, which sums and stores them on the way
  int sp_o = 1;
  {
    BwdParams p = bwd_params(w.dy_b, T, bv.w[1], w.G, r, lv.A[1], lv.AT[1], r);
    p.out = w.dattn;
    TRY(gemm_bwd(p, EPI_BF16, s, w.gemm, w.gemm_bytes, &sp_o));
  }
  {
    const int se[1] = {d.H};
    TRY(adapter_grads(d, T, w.G32, r, w.U32[1], r, w.attn, d.Nq, d.Nq, w.dy_b, d.H, 1, se, gA[1], gB[1], accumulate, w, s));
  }
  // ---- attention (rotary applied inside, in float32)
  {
    AttnBwdArgs a{w.qkv, d.Nqkv, S, d.nh, d.nkv, d.hd, 1.0f / sqrtf((float)d.hd), w.attn, w.attn_f32, w.dattn, d.Nq,
                  w.lse, nullptr, w.dqkv, reinterpret_cast<const float2*>(w.rope), w.dk_part, w.dv_part, w.aprep};
    if (sp_o > 1) {
      a.dO_part = static_cast<const float*>(w.gemm);
      a.dO_splits = sp_o;
    }
    TRY(attention_bwd(a, B, w.D, s));
  }
  // ---- q, k, v projections
  SegEnds three{};
  three.end[0] = d.Nq;
  three.end[1] = d.Nq + d.Nkv;
  three.end[2] = d.Nqkv;
  TRY(lora_g(w.dqkv, d.Nqkv, T, d.Nqkv, lv.BT[0], r, 3, three, sc, w.G, 3 * r, w.G32, 3 * r, w.lws,
             w.lws_bytes, w.cnt, s));
  // dxn1, then dx = dh + rmsnorm1'(dxn1) (from the partials of a split-K
  // launch), with its bf16 copy in dy_b for the layer below (layer_bwd_dy_b)
  {
    BwdParams p = bwd_params(w.dqkv, T, bv.w[0], w.G, 3 * r, lv.A[0], lv.AT[0], 3 * r);
    p.out = w.dxn;
    int sp = 1;
    TRY(gemm_bwd(p, EPI_F32, s, w.gemm, w.gemm_bytes, &sp));
    if (sp > 1)
      TRY(splitk_rmsnorm_bwd(x_in, bv.norm1, static_cast<const float*>(w.gemm), sp, w.dh, T, d.H, c->rms_eps, dx_in,
                             w.dy_b, s));
    else
      TRY(rmsnorm_bwd(x_in, bv.norm1, w.dxn, w.dh, T, d.H, c->rms_eps, dx_in, w.dy_b, s));
  }
  {
    const int se[3] = {d.Nq, d.Nq + d.Nkv, d.Nqkv};
    TRY(adapter_grads(d, T, w.G32, 3 * r, w.U32[0], 3 * r, w.xn1, 2 * d.H, d.H, w.dqkv, d.Nqkv, 3, se, gA[0], gB[0], accumulate,
                      w, s));
  }
  return LSQ_OK;
}

// The per-call preparation a layer pass needs: the rotary table, and zeroed
// arrival counters.  A step does it once for all of its layer passes (they
// share one workspace and every rank-r launch leaves the counters at zero).
int layer_prepare(const lsq_model_cfg* c, int B, int S, void* ws, hipStream_t s) {
  const LayerWs w = carve(c, B, S, ws, true);
  TRY(rope_table(S, dims_of(c).hd, c->rope_theta, w.rope, s));
  return zero_counters(w.cnt, w.ncnt, s);
}

int layer_fwd(const lsq_model_cfg* c, const void* blob, const void* lora, const float* x_in, int B, int S,
              float* x_out, void* ws, hipStream_t s, void* acts, void* ustore) {
  LayerWs w = carve(c, B, S, ws, false, acts, false, nullptr, ustore);
  return forward_impl(c, view_blob(c, blob), view_lora(c, lora), x_in, B, S, x_out, w, s);
}

uint16_t* layer_bwd_dy_b(const lsq_model_cfg* c, int B, int S, void* ws) { return carve(c, B, S, ws, true).dy_b; }

int layer_bwd(const lsq_model_cfg* c, const void* blob, const void* lora, const void* lora_t, const float* x_in,
              const float* dx_out, int B, int S, float* dx_in, float* grad, int accumulate, void* ws, hipStream_t s,
              const LayerHook* hook, void* acts, bool dy_b_ready, void* ustore) {
  LayerWs w = carve(c, B, S, ws, true, acts, false, nullptr, ustore);
  if (!lora_t) {
    TRY(adapter_transpose(c, static_cast<const uint16_t*>(lora), w.lora_t, 1, s));
    lora_t = w.lora_t;
  }
  const BlobView bv = view_blob(c, blob);
  const LoraView lv = view_lora(c, lora, lora_t);
  if (!acts) TRY(forward_impl(c, bv, lv, x_in, B, S, nullptr, w, s, ustore != nullptr));
  if (hook && hook->after_recompute) TRY(hook->after_recompute(hook->ctx));
  return backward_impl(c, bv, lv, x_in, dx_out, B, S, dx_in, grad, accumulate, w, s, dy_b_ready);
}

}  // namespace lsq

// ================================================================== C ABI
using namespace lsq;

extern "C" {

int lsq_blob_layout_get(const lsq_model_cfg* cfg, lsq_blob_layout* out) {
  if (int e = check_cfg(cfg)) return e;
  LSQ_CHECK(out, LSQ_ERR_INVALID, "lsq_blob_layout_get: null out");
  blob_layout(cfg, out);
  return LSQ_OK;
}

int lsq_lora_layout_get(const lsq_model_cfg* cfg, lsq_lora_layout* out) {
  if (int e = check_cfg(cfg)) return e;
  LSQ_CHECK(out, LSQ_ERR_INVALID, "lsq_lora_layout_get: null out");
  lora_layout(cfg, out);
  return LSQ_OK;
}

size_t decoder_layer_workspace_size(const lsq_model_cfg* cfg, int32_t batch, int32_t seq) {
  if (check_cfg(cfg) || batch < 0 || seq < 0) return 0;
  return layer_ws_bytes(cfg, batch, seq, false);
}

static int check_layer_args(const lsq_model_cfg* cfg, const void* blob, const void* lora, const void* x, int B,
                            int S, const void* ws, size_t ws_bytes) {
  if (int e = check_cfg(cfg)) return e;
  LSQ_CHECK(blob && lora && x && ws, LSQ_ERR_INVALID, "decoder_layer: null pointer");
  LSQ_CHECK(B >= 1 && S >= 1 && (int64_t)B * S < (1 << 24), LSQ_ERR_SHAPE, "decoder_layer: bad batch/seq");
  LSQ_CHECK(aligned16(blob) && aligned16(lora) && aligned16(x) && aligned16(ws), LSQ_ERR_ALIGN,
            "decoder_layer: unaligned pointer");
  LSQ_CHECK(ws_bytes >= layer_ws_bytes(cfg, B, S, false), LSQ_ERR_WORKSPACE, "decoder_layer: workspace %zu < %zu",
            ws_bytes, layer_ws_bytes(cfg, B, S, false));
  return LSQ_OK;
}

int decoder_layer_fwd(const lsq_model_cfg* cfg, const void* blob, const void* lora, const float* x_in, int32_t batch,
                      int32_t seq, float* x_out, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_layer_args(cfg, blob, lora, x_in, batch, seq, ws, ws_bytes)) return e;
  LSQ_CHECK(x_out && aligned16(x_out) && x_out != x_in, LSQ_ERR_INVALID, "decoder_layer_fwd: bad x_out");
  if (int e = layer_prepare(cfg, batch, seq, ws, as_stream(stream))) return e;
  return layer_fwd(cfg, blob, lora, x_in, batch, seq, x_out, ws, as_stream(stream), nullptr);
}

int decoder_layer_bwd(const lsq_model_cfg* cfg, const void* blob, const void* lora, const float* x_in_saved,
                      const float* dx_out, int32_t batch, int32_t seq, float* dx_in, float* lora_grad,
                      int32_t accumulate, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_layer_args(cfg, blob, lora, x_in_saved, batch, seq, ws, ws_bytes)) return e;
  LSQ_CHECK(dx_out && dx_in && lora_grad && aligned16(dx_out) && aligned16(dx_in) && aligned16(lora_grad),
            LSQ_ERR_INVALID, "decoder_layer_bwd: bad gradient pointers");
  if (int e = layer_prepare(cfg, batch, seq, ws, as_stream(stream))) return e;
  return layer_bwd(cfg, blob, lora, nullptr, x_in_saved, dx_out, batch, seq, dx_in, lora_grad, accumulate, ws,
                   as_stream(stream), nullptr, nullptr);
}

}  // extern "C"
