/*
 * lsq.h -- C ABI of liblsq: layer-streamed LoRA fine-tuning over a frozen NF4
 * (or bf16) base on one AMD Instinct MI355X (gfx950).
 *
 * Citations name a page and a section heading on it:
 *   LS-docs = "Layer streaming: fine-tune a model that does not fit in your
 *             card" (trysoup.dev/docs/layer-streaming)
 *   About   = "About Soup" (trysoup.dev/about)
 *
 * Conventions for every call
 * --------------------------
 * - Return value: LSQ_OK (0) or a negative lsq_status.  On error nothing has
 *   been enqueued: all argument, shape and alignment checks run before the
 *   first launch.  lsq_last_error() returns a thread-local message.
 * - Pointers named *_dev, and every tensor argument of a compute call, are
 *   device pointers; the caller owns them and keeps them alive until the work
 *   enqueued on `stream` has completed.  The library never frees them.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   compute calls are asynchronous with respect to the host and ordered on
 *   that stream, unless stated otherwise.
 * - Tensors are row-major and contiguous.  Device tensor pointers must be
 *   16-byte aligned (LSQ_ERR_ALIGN otherwise).
 * - dtype LSQ_BF16 tensors hold bfloat16 bit patterns; LSQ_F32 hold float32.
 * - Kernel choice is a pure function of (M, N, K, r, dtype): a resident run
 *   and a streamed run of the same shapes execute the same kernels on the
 *   same bytes (LS-docs "How it works"; "Bit-exact is two claims, not one").
 * - No call on the training path allocates device memory; workspaces are
 *   passed in, sized by the *_workspace_size queries.
 */
#ifndef LSQ_H
#define LSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
typedef enum {
  LSQ_OK = 0,
  LSQ_ERR_INVALID = -1,   /* null pointer, bad enum, bad flag            */
  LSQ_ERR_SHAPE = -2,     /* e.g. n_in % 64 != 0, r < 1, batch < 1       */
  LSQ_ERR_ALIGN = -3,     /* device pointer not 16-byte aligned          */
  LSQ_ERR_NONFINITE = -4, /* NaN or Inf in a quantize input              */
  LSQ_ERR_OOM = -5,       /* host allocation failed                      */
  LSQ_ERR_HIP = -6,       /* a HIP runtime call failed (message says which) */
  LSQ_ERR_STATE = -7,     /* pool misuse: acquire of a layer never fetched, ... */
  LSQ_ERR_REFUSED = -8,   /* pre-flight: predicted peak exceeds free VRAM */
  LSQ_ERR_WORKSPACE = -9, /* workspace smaller than the size query returns */
  LSQ_ERR_IO = -10        /* a store file could not be written or read, is not a store,
                             or fails its checksums                        */
} lsq_status;

const char* lsq_last_error(void);
int32_t lsq_version(void);

/* The 16 NF4 levels the kernels decode with, ascending (host query, no GPU). */
void lsq_nf4_codebook(float out[16]);

enum { LSQ_BF16 = 0, LSQ_F32 = 1 };       /* activation / adapter dtypes */
enum { LSQ_W_NF4 = 0, LSQ_W_BF16 = 1 };   /* streamed base weight kinds  */

/* ---------------------------------------------------------------- NF4 (a0)
 * Blockwise NF4 quantization of a frozen bf16 weight, done once offline when
 * the shard store is written (LS-docs "Shard cache"; About: the store is about
 * four times smaller in NF4).  The pages do not give the format; this library
 * uses: 64-element blocks along each row (n_in % 64 == 0), one float32 absmax
 * per block, code = index of the NormalFloat-4 level nearest to
 * fp32(x / absmax) (IEEE division; an all-zero block gets code 7, the zero
 * level), and two codes per byte with the even element in the high nibble.
 */

/* w_dev [n_out, n_in] of dtype LSQ_BF16 or LSQ_F32 -> packed_dev uint8
 * [n_out, n_in/2] and absmax_dev float32 [n_out, n_in/64].  blocksize must be
 * 64 (the store format; others are LSQ_ERR_SHAPE).  A NaN or Inf input leaves
 * its block's outputs unspecified and is reported in one of two ways:
 * flag_dev (device int32, nullable) non-null: the call is stream-ordered and
 * sets *flag_dev to 1 (never clears it);
 * flag_dev null: the call waits for the stream and returns LSQ_ERR_NONFINITE
 * (such calls use one library-owned device word per GPU and are serialized by
 * the library). */
int nf4_quantize(const void* w_dev, int32_t dtype, int64_t n_out, int64_t n_in, int32_t blocksize,
                 void* packed_dev, float* absmax_dev, int32_t* flag_dev, void* stream);

/* Inverse map: w = bf16(fp32(level[code] * absmax)) (out_dtype LSQ_BF16) or the
 * float32 product itself (LSQ_F32), written to w_out_dev [n_out, n_in]. */
int nf4_dequantize(const void* packed_dev, const float* absmax_dev, int64_t n_out, int64_t n_in,
                   int32_t out_dtype, void* w_out_dev, void* stream);

/* ------------------------------------------------------ LoRA linear (a4, a8, a9)
 * One frozen-base linear with a plain LoRA adapter (LS-docs "Honest scope":
 * plain LoRA only; About: only the adapters train).  PEFT naming: A [r, K],
 * B [N, r], scale s = alpha / r.  For X [M, K]:
 *     U = s X A^T              (saved for the backward)
 *     Y = X W^T + U B^T (+ bias)
 * and for dY [M, N], with G = s dY B:
 *     dX = dY W + G A,  dA = G^T X,  dB = dY^T U
 * which is PEFT's dX = dY W + s (dY B) A, dA = s (dY B)^T X, dB = s dY^T (X A^T).
 * No gradient for W or the bias: the base is frozen, yet the backward still
 * needs W to push the gradient to X (LS-docs "How it works").
 * Precision: LSQ_BF16 runs bf16 MFMA with float32 accumulation; U and G are
 * rounded to bf16 once where they enter an MFMA (Y and dX), while dA and dB
 * are reduced in float32 from their unrounded values.  LSQ_F32 runs float32
 * end to end (dequantized weights are the exact float32 products).
 */
typedef struct {
  int32_t kind;          /* LSQ_W_NF4 or LSQ_W_BF16                          */
  int32_t reserved;
  const void* data;      /* NF4: uint8 [n_out, n_in/2]; BF16: bf16 [n_out, n_in] */
  const float* absmax;   /* NF4: float32 [n_out, n_in/64]; BF16: NULL          */
  int64_t n_out, n_in;   /* N, K                                               */
} lsq_weight;

size_t nf4_lora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dtype);

/* X [M, K], A [r, K], B [N, r], bias [N] (nullable, bf16) in `dtype`;
 * Y [M, N] in `dtype`; U_out [M, r] in `dtype` (nullable).
 * Shapes: K % 64 == 0, r in {8, 16, ..., 64}, and N % 8 == 0 for LSQ_BF16
 * (LSQ_ERR_SHAPE otherwise, checked before anything is enqueued). */
int nf4_lora_linear_fwd(const lsq_weight* W, const void* bias, const void* X, int64_t M,
                        const void* A, const void* B, int32_t r, float scale, int32_t dtype,
                        void* Y, void* U_out, void* ws, size_t ws_bytes, void* stream);

/* U [M, r] as written by the forward (nullable: recomputed into ws).
 * dX [M, K] in `dtype`; dA [r, K] and dB [N, r] float32; accumulate != 0 adds
 * into dA and dB instead of overwriting.  Reductions over M run in a fixed
 * order: results are bitwise reproducible run to run. */
int nf4_lora_linear_bwd(const lsq_weight* W, const void* X, const void* U, int64_t M,
                        const void* A, const void* B, int32_t r, float scale, int32_t dtype,
                        const void* dY, void* dX, float* dA, float* dB, int32_t accumulate,
                        void* ws, size_t ws_bytes, void* stream);

/* nf4_lora_linear_bwd with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Its scratch is a static device array of
 * LSQ_NOALLOC_SCRATCH_BYTES per GPU, created with the library's code on each
 * device and held until the process ends; the call itself allocates nothing.
 * A shape whose nf4_lora_linear_workspace_size exceeds that size is refused
 * with LSQ_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialized by the caller.  The arguments and
 * results are those of nf4_lora_linear_bwd, bit for bit. */
#define LSQ_NOALLOC_SCRATCH_BYTES (128ull << 20)
int nf4_lora_linear_bwd_noalloc(const lsq_weight* W, const void* X, const void* U, int64_t M,
                                const void* A, const void* B, int32_t r, float scale, int32_t dtype,
                                const void* dY, void* dX, float* dA, float* dB, int32_t accumulate,
                                void* stream);

/* ---------------------------------------------------------------- model shape
 * A Llama / Qwen2 decoder stack (LS-docs "How it works": transformers' own
 * classes).  weight_kind selects the streamed base format (LS-docs "Turn it
 * on": quantization none or 4bit). */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, n_layers;
  int32_t qkv_bias;      /* Qwen2: frozen bf16 bias on q, k, v              */
  int32_t tied;          /* head == embedding                               */
  int32_t weight_kind;   /* LSQ_W_NF4 or LSQ_W_BF16                         */
  int32_t lora_r;
  float rms_eps, rope_theta, lora_scale;
  int32_t loss_chunk;    /* stream_loss_chunk (LS-docs "Scaling a streaming run",
                            "Troubleshooting": the logits are usually the whole
                            story): tokens per head/cross-entropy chunk, which
                            bounds the logits buffers at loss_chunk x vocab;
                            0 = all tokens at once                             */
} lsq_model_cfg;

/* One layer's shard ("blob"): one contiguous, 4 KiB-aligned byte range, so a
 * layer moves in one copy (LS-docs "How it works": one shard per decoder
 * layer, one pooled buffer per layer).  Groups: 0 = q,k,v rows stacked,
 * 1 = o, 2 = gate,up rows stacked, 3 = down.  Offsets in bytes. */
typedef struct {
  uint64_t total_bytes;
  uint64_t w_off[4];       /* NF4 packed codes or bf16 weights of each group */
  uint64_t absmax_off[4];  /* NF4 only                                       */
  uint64_t norm1_off, norm2_off;  /* bf16 [hidden]                           */
  uint64_t bias_off;       /* bf16 [(n_heads + 2 n_kv_heads) head_dim]; 0 if none */
} lsq_blob_layout;
int lsq_blob_layout_get(const lsq_model_cfg* cfg, lsq_blob_layout* out);

/* One layer's adapters in one block, groups stacked like the blob:
 * A_qkv [3r, H], A_o [r, n_heads*head_dim], A_gu [2r, H], A_down [r, I],
 * B_qkv [Nqkv, r], B_o [H, r], B_gu [2I, r], B_down [H, r].  Offsets and
 * sizes count elements (bf16 for parameters, float32 for gradients). */
typedef struct {
  uint64_t a_off[4], b_off[4];
  uint64_t layer_elems;
} lsq_lora_layout;
int lsq_lora_layout_get(const lsq_model_cfg* cfg, lsq_lora_layout* out);

/* ----------------------------------------------------- decoder layer (a3, a7)
 * x_in / x_out / dx: float32 [batch*seq, hidden] residual stream.  blob: the
 * layer's shard in device memory (a pool slot or a resident arena).  lora:
 * bf16 adapter block; lora_grad: float32 block of the same layout.
 * decoder_layer_bwd recomputes the forward from the saved x_in (the layer is
 * read twice per step: LS-docs "How it works") and then backpropagates dx_out;
 * it reads the blob until its last kernel, so the caller may release the slot
 * only after the call's work (LS-docs "If you streamed a 32B or larger model
 * in NF4": the backward must never read a refilled slot). */
size_t decoder_layer_workspace_size(const lsq_model_cfg* cfg, int32_t batch, int32_t seq);
int decoder_layer_fwd(const lsq_model_cfg* cfg, const void* blob, const void* lora,
                      const float* x_in, int32_t batch, int32_t seq, float* x_out,
                      void* ws, size_t ws_bytes, void* stream);
int decoder_layer_bwd(const lsq_model_cfg* cfg, const void* blob, const void* lora,
                      const float* x_in_saved, const float* dx_out, int32_t batch, int32_t seq,
                      float* dx_in, float* lora_grad, int32_t accumulate,
                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ shard store (a0, a1)
 * Host store of every layer blob, rewritten once and held in page-locked
 * memory when possible, because pinned copies run asynchronously and overlap
 * compute while pageable ones do not (LS-docs "How it works"; "Why NF4 also
 * made the 3B row faster").  One hipHostMalloc arena holds all layers. */
typedef struct lsq_store lsq_store;
enum {
  LSQ_STORE_ALLOW_PAGEABLE = 1,  /* fall back to pageable memory, with a printed notice */
  LSQ_STORE_FORCE_PAGEABLE = 2,  /* measure the pageable path on purpose          */
  LSQ_STORE_FAIL_PIN = 4         /* test hook: behave as if page-locking failed   */
};
int shard_store_create(const lsq_model_cfg* cfg, int32_t flags, lsq_store** out);
void shard_store_destroy(lsq_store* store);
int32_t shard_store_is_pinned(const lsq_store* store);
uint64_t shard_store_layer_bytes(const lsq_store* store);
/* Host pointer to layer i's blob (read-only view for tests and copies). */
const void* shard_store_layer_host(const lsq_store* store, int32_t layer);

/* The frozen tensors of one layer as bf16 device tensors (biases nullable
 * unless cfg.qkv_bias): w[0..6] = q, k, v, o, gate, up, down [out, in]. */
typedef struct {
  const void* w[7];
  const void* norm1;
  const void* norm2;
  const void* bias[3];
} lsq_layer_src;
/* Quantize (NF4) or copy (bf16) one layer into a device staging blob
 * (staging_dev, shard_store_layer_bytes() bytes, plus 256 bytes for a flag),
 * then copy it into the host store.  Synchronous: returns after the copy.
 * LSQ_ERR_NONFINITE if any weight is NaN/Inf. */
int shard_store_write_layer(lsq_store* store, int32_t layer, const lsq_layer_src* src,
                            void* staging_dev, size_t staging_bytes, void* stream);

/* Shard cache on disk (LS-docs "Shard cache": the rewrite happens once,
 * offline, and a cache whose quantisation or shapes differ is re-sharded, not
 * streamed).  File layout: a 4 KiB header (magic "LSQSTORE", format version,
 * the blob-shaping fields of the config, blob bytes, layer count), a table of
 * one 64-bit checksum per layer padded to 4 KiB, then the blobs back to back.
 * shard_store_save writes path + ".tmp" and renames it over path, so an
 * interrupted save never leaves a file that loads.  Host-only calls (no GPU
 * work); LSQ_ERR_IO on any file error. */
int shard_store_save(const lsq_store* store, const char* path);
/* Reads a saved store into a new host arena (page-locked per `flags`, as in
 * shard_store_create).  expect (nullable): the config the caller will stream
 * with; a file whose hidden, heads, kv heads, head_dim, intermediate, layers,
 * qkv_bias or weight_kind differ is refused with LSQ_ERR_STATE and a message
 * naming the first differing field.  A short file, a bad magic, a blob header
 * that names another layer or a checksum mismatch is LSQ_ERR_IO. */
int shard_store_load(const char* path, const lsq_model_cfg* expect, int32_t flags, lsq_store** out);

/* ------------------------------------------------------ layer pool (a2, a5)
 * N pre-allocated VRAM slots (2..8, default 2) and a dedicated copy stream:
 * layer i+1 is copied while layer i computes (LS-docs "Turn it on":
 * stream_buffers; "How it works").  Handoff is by hipEvent: a copy into a slot
 * is issued once that slot's free event, recorded on the compute stream after
 * the last kernel that read the slot's previous layer, has completed (the host
 * waits for it in stream_layer_prefetch; a copy stream waiting on the compute
 * stream's event instead slowed the copies and the kernels beside them); the
 * compute stream waits on the slot's ready event before reading it.  A layer still in a slot is not
 * copied again (LS-docs "Roadmap": layer 0 at the step boundary; this pool
 * applies the same rule to every layer, e.g. at the forward/backward turn).
 * Resident mode (flags LSQ_POOL_RESIDENT, n_buffers == n_layers) copies every
 * layer once at create and never again: the acceptance partner of a streamed
 * run, same kernels, same bytes (LS-docs "Bit-exact is two claims, not one").
 * dev_slots: n_buffers * slot_stride bytes of device memory owned by the
 * caller; slot_stride >= shard_store_layer_bytes() and a multiple of 4096.
 * copy_stream: the caller's stream for the layer copies, or NULL.  The overlap
 * needs the copy stream to run while the compute stream is busy, which HIP
 * does not promise: streams share a few hardware queues (GPU_MAX_HW_QUEUES),
 * and two streams on one queue run in submission order.  So a streaming pool
 * checks at create (a kernel on the compute stream waits, at most 20 ms, for a
 * flag set by a kernel on the copy stream, using slot 0's first bytes) and, if
 * the copy stream is NULL, the compute stream itself, or fails the check,
 * copies on a stream of its own that passes it (destroyed with the pool; a
 * message on stderr if none does).  layer_pool_copy_stream names the stream in
 * use.  A resident pool copies once, on copy_stream or else compute_stream. */
typedef struct lsq_pool lsq_pool;
enum {
  LSQ_POOL_RESIDENT = 1,
  LSQ_POOL_POISON = 2          /* debug: fill a slot with 0xFF bytes before each refill */
};
int layer_pool_create(const lsq_store* store, int32_t n_buffers, void* dev_slots, uint64_t slot_stride,
                      void* compute_stream, void* copy_stream, int32_t flags, lsq_pool** out);
void layer_pool_destroy(lsq_pool* pool);
/* The stream the pool's layer copies run on (*stream; the pool's own when it
 * replaced or was not given one). */
int layer_pool_copy_stream(const lsq_pool* pool, void** stream);
/* Enqueue the copy of `layer` into a free slot on the copy stream; no-op if it
 * is already in a slot.  Blocks the calling thread until the chosen slot's
 * free event has completed (its work is already enqueued, so the wait ends):
 * enqueue the current layer's kernels before prefetching the next.
 * LSQ_ERR_STATE if every slot is held. */
int stream_layer_prefetch(lsq_pool* pool, int32_t layer);
/* Make the compute stream wait until `layer` is in its slot; returns the slot's
 * device address.  LSQ_ERR_STATE if the layer was never prefetched. */
int layer_pool_acquire(lsq_pool* pool, int32_t layer, const void** blob_dev);
/* Record the slot's free event on the compute stream: call after enqueuing the
 * last kernel that reads the layer. */
int layer_pool_release(lsq_pool* pool, int32_t layer);
typedef struct {
  uint64_t copies, copy_bytes, hits;
  double copy_ms;      /* summed durations of the timed copies (events on the copy stream) */
  uint64_t large_copies, large_bytes;   /* head copies of LSQ_STEP_STREAM_LARGE steps */
  uint64_t timed_copies, timed_bytes;   /* the copies copy_ms covers: at most 1024 between two
                                           layer_pool_stats calls carry events */
} lsq_pool_stats;
int layer_pool_stats(lsq_pool* pool, int32_t reset, lsq_pool_stats* out);

/* Copy/compute timeline of the steps run on a pool (the evidence for the
 * pages' overlap claim, LS-docs "How it works": layer i+1's bytes arrive while
 * layer i computes).  With capacity > 0, every layer copy on the copy stream
 * and every layer pass on the compute stream (forward, backward, and the head
 * with its loss) is bracketed by a pair of timing events; capacity 0 turns it
 * off.  Events are recorded only while enabled and cost a few microseconds per
 * record, so a timed measurement runs with the timeline off.  Records past the
 * capacity are dropped (counted in `dropped`).  lsq_timeline_read waits for
 * the recorded work, writes at most `max` entries in recording order with
 * times in ms relative to the first entry's start, and clears the timeline. */
enum { LSQ_TL_COPY = 0, LSQ_TL_FWD = 1, LSQ_TL_BWD = 2, LSQ_TL_HEAD = 3, LSQ_TL_LARGE_COPY = 4 };
typedef struct {
  int32_t kind;        /* LSQ_TL_* */
  int32_t layer;       /* layer index (-1 for the head and its copy) */
  double start_ms, end_ms;
} lsq_timeline_entry;
int lsq_timeline_enable(lsq_pool* pool, int32_t capacity);
int lsq_timeline_read(lsq_pool* pool, lsq_timeline_entry* out, int32_t max, int32_t* n, int32_t* dropped);

/* --------------------------------------------------- training step (a0..a9)
 * One streamed fwd+bwd step: embedding gather, L layers forward (prefetch one
 * ahead, acquire, layer forward, release), final RMSNorm, head GEMM, mean
 * next-token cross-entropy and its gradient, then L layers backward in reverse
 * with per-layer recompute (or kept activations), writing every adapter
 * gradient.  Embedding, final
 * norm and head stay resident and get no gradient (LS-docs "How it works").
 * Runs on the pool's compute stream. */
typedef struct {
  const void* embed;       /* bf16 [vocab, hidden]                     */
  const void* head;        /* bf16 [vocab, hidden]; == embed if tied   */
  const void* final_norm;  /* bf16 [hidden]                            */
  const void* lora;        /* bf16 [n_layers, lora layer_elems]        */
  float* lora_grad;        /* float32 [n_layers, lora layer_elems]     */
} lsq_resident;
enum {
  LSQ_STEP_FORWARD_ONLY = 1,        /* loss and logits only                      */
  LSQ_STEP_DEBUG_EARLY_RELEASE = 2, /* control: release each layer's slot after
                                       its backward recompute and let the next
                                       copy land before its backward GEMMs, the
                                       aliasing defect the pages describe; must
                                       make gradients differ                    */
  LSQ_STEP_KEEP_ACTIVATIONS = 4,     /* stream_recompute off (LS-docs "How it
                                       works"): keep each layer's forward
                                       activations and skip the backward's
                                       recompute; the backward still re-reads
                                       every layer's weights.  Needs the larger
                                       workspace the size query returns for it. */
  LSQ_STEP_STREAM_LARGE = 16,        /* large-layer streaming of an untied
                                       embedding and head (LS-docs "Measured
                                       numbers": they move into the store and
                                       share one vocabulary-sized buffer):
                                       res->embed and res->head are then
                                       page-locked HOST pointers.  The gather
                                       reads only the batch's embedding rows
                                       over the link; the head is copied once
                                       per step into the workspace's head buffer
                                       on the pool's copy stream, after the last
                                       layer copy of the forward.  Refused for
                                       tied models.                              */
  LSQ_STEP_RECOMPUTE_ALL = 32,       /* recompute every layer in the backward.
                                       Without it (and without
                                       LSQ_STEP_KEEP_ACTIVATIONS) a step keeps
                                       the forward activations of layers L-1, 1
                                       and 0: their backward passes run while
                                       both slots hold layers still needed and
                                       the copy stream has nothing to do (the
                                       forward/backward turn and the step's
                                       tail), so their recompute would sit on
                                       the step's critical path.  Every other
                                       layer is recomputed under its copy.
                                       Results are bit-identical either way. */
  LSQ_STEP_REFERENCE_FORWARD = 8     /* preference losses (LS-docs "Preference
                                       losses over streaming"; Editorial "The
                                       Honest Cost"): also run the reference
                                       model, the same streamed base with its
                                       adapters off, and return its per-token
                                       negative log-likelihood.  Both forwards
                                       run on each layer while it is in its
                                       slot, so the stack is still read twice
                                       per step.  Needs lsq_step_extra outputs. */
};
/* Workspace of a step run with `flags` (LSQ_STEP_KEEP_ACTIVATIONS adds
 * n_layers kept-activation regions, the default min(n_layers, 3), and
 * LSQ_STEP_RECOMPUTE_ALL none). */
size_t lsq_step_workspace_size(const lsq_model_cfg* cfg, int32_t batch, int32_t seq, int32_t flags);
/* ids_dev int32 [batch, seq]; loss_dev float32 [1]; logits_out float32
 * [batch*seq, vocab] (nullable). */
int lsq_train_step(const lsq_model_cfg* cfg, lsq_pool* pool, const lsq_resident* res,
                   const int32_t* ids_dev, int32_t batch, int32_t seq, float* loss_dev,
                   float* logits_out, int32_t flags, void* ws, size_t ws_bytes);
/* The same step, also copying (both nullable, float32, [n_layers + 1, batch*seq,
 * hidden]) every layer's input x_i (x_trace[n_layers] = the final residual) and
 * the gradient arriving at every layer's output (dx_trace[i] = dL/dx_i), so a
 * checker can recompute each layer from the exact inputs this run used. */
int lsq_train_step_traced(const lsq_model_cfg* cfg, lsq_pool* pool, const lsq_resident* res,
                          const int32_t* ids_dev, int32_t batch, int32_t seq, float* loss_dev,
                          float* logits_out, int32_t flags, void* ws, size_t ws_bytes,
                          float* x_trace, float* dx_trace);
/* Optional step outputs (every pointer nullable, device memory). */
typedef struct {
  float* x_trace;       /* as lsq_train_step_traced                               */
  float* dx_trace;
  float* ref_nll_rows;  /* LSQ_STEP_REFERENCE_FORWARD: float32 [batch*seq], the
                           reference model's -log p(next token); 0 at the last
                           position of each sequence                              */
  float* ref_loss;      /* float32 [1]: their mean over the batch*(seq-1) targets */
} lsq_step_extra;
int lsq_train_step_ex(const lsq_model_cfg* cfg, lsq_pool* pool, const lsq_resident* res,
                      const int32_t* ids_dev, int32_t batch, int32_t seq, float* loss_dev,
                      float* logits_out, int32_t flags, void* ws, size_t ws_bytes,
                      const lsq_step_extra* extra);

/* ------------------------------------------------------ VRAM pre-flight
 * Predict the peak device memory of a streamed step for this exact batch and
 * sequence length and refuse before any GPU work if it does not fit (LS-docs
 * "Turn it on"; "Troubleshooting": the terms streaming does not bound are the
 * activations and logits).  The prediction is the sum of the buffers this
 * library asks the caller to allocate (the pool's slots at their 4 KiB stride,
 * the resident tensors, adapters and their gradients, the step workspace), the
 * caller's own step tensors, and a margin, so that it errs high like the
 * pages' pre-flight (LS-docs "Run it yourself on a free Colab T4": 3.02 GB
 * predicted against 2.91 GB measured). */
typedef struct {
  uint64_t slots, resident, adapters, checkpoints, saved_activations, step_workspace;
  uint64_t caller;   /* the token ids and the loss scalar, plus up to 511 bytes of
                        allocator rounding for each of the step's 16 buffers     */
  uint64_t margin;   /* 1% of the sum above (at least 1 MiB): allocator slack     */
  uint64_t total;
} lsq_vram_breakdown;
/* step_flags: the flags the step will run with (kept activations are a term
 * of their own). */
int vram_predict_peak(const lsq_model_cfg* cfg, int32_t batch, int32_t seq, int32_t n_buffers,
                      int32_t step_flags, lsq_vram_breakdown* out);
/* LSQ_ERR_REFUSED when the prediction exceeds free VRAM.  free_override_bytes
 * > 0 replaces the device's free memory (a capped process cannot see its cap:
 * LS-docs "Run it yourself on a free Colab T4"). */
int lsq_preflight(const lsq_model_cfg* cfg, int32_t batch, int32_t seq, int32_t n_buffers,
                  int32_t step_flags, uint64_t free_override_bytes, lsq_vram_breakdown* out);

/* ------------------------------------------------------ kernel timing
 * When enabled, every launch of the timed kernel families is bracketed by
 * hipEvents on its own stream (library-owned event pool) and credited with its
 * algorithmic flops and bytes.  lsq_prof_read synchronizes the events and
 * fills one entry per family (it needs at least 7 entries):
 *   gemm_fwd_nf4_lora, gemm_bwd_nf4_lora  the NF4-weight tile kernels alone
 *   lora_skinny        rank-r down-projection, G and adapter-gradient kernels
 *   attention          attention forward and backward kernels
 *   other              split-K reductions, transposes of the adapters
 *   gemm_bf16_weights  tile kernels over bf16 weights (bf16 base, the head)
 *   elementwise        RMSNorm forward and backward, SwiGLU forward and
 *                      backward, the embedding gather and the cross-entropy
 *                      rows: bytes = each operand read once and written once
 * Enabling resets the counts. */
typedef struct {
  char name[48];
  uint64_t launches;
  double ms;        /* summed event durations */
  double flops;     /* algorithmic flops      */
  double bytes;     /* algorithmic HBM bytes  */
} lsq_prof_entry;
int lsq_prof_enable(int32_t on);
int lsq_prof_read(lsq_prof_entry* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif
#endif /* LSQ_H */
