// Streaming runtime: shard store, VRAM layer pool, training step, pre-flight.
//
// What the pages describe and this file implements (LS-docs "How it works";
// "Turn it on"; About): the frozen base is rewritten once into one shard per
// decoder layer, held in page-locked host memory; a small pool of N
// pre-allocated VRAM buffers (2..8) receives one layer at a time on a
// dedicated copy stream, layer i+1 while layer i computes; only the
// embedding, final norm, head and the adapters (with their gradients) stay
// resident.  The backward re-reads every layer (recompute) and must never read
// a slot that has been refilled (LS-docs "If you streamed a 32B or larger
// model in NF4"): a slot's free event is recorded after the last kernel that
// reads it and every refill waits on it.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "common.h"
#include "gemm.h"
#include "layer.h"
#include "layer_ops.h"

using namespace lsq;

namespace {
uint64_t up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

struct BlobHeader {
  char magic[8];  // "LSQBLOB1"
  int32_t layer, weight_kind, hidden, n_heads, n_kv_heads, head_dim, intermediate, lora_r, qkv_bias;
  uint64_t total_bytes;
};
}  // namespace

// ================================================================== store
struct lsq_store {
  lsq_model_cfg cfg;
  uint64_t layer_bytes;
  char* host;
  bool pinned;
};

extern "C" {

int shard_store_create(const lsq_model_cfg* cfg, int32_t flags, lsq_store** out) {
  if (int e = check_cfg(cfg)) return e;
  LSQ_CHECK(out, LSQ_ERR_INVALID, "shard_store_create: null out");
  lsq_blob_layout L;
  blob_layout(cfg, &L);
  const uint64_t total = L.total_bytes * (uint64_t)cfg->n_layers;
  lsq_store* st = new (std::nothrow) lsq_store{*cfg, L.total_bytes, nullptr, false};
  LSQ_CHECK(st, LSQ_ERR_OOM, "shard_store_create: out of host memory");
  bool want_pin = !(flags & LSQ_STORE_FORCE_PAGEABLE);
  if (want_pin) {
    void* p = nullptr;
    hipError_t e = (flags & LSQ_STORE_FAIL_PIN) ? hipErrorOutOfMemory : hipHostMalloc(&p, total, hipHostMallocDefault);
    if (e == hipSuccess) {
      st->host = static_cast<char*>(p);
      st->pinned = true;
    } else {
      (void)hipGetLastError();  // clear the failed page-lock before anything else runs
      if (!(flags & LSQ_STORE_ALLOW_PAGEABLE)) {
        delete st;
        return fail(LSQ_ERR_OOM, "could not page-lock the %.2f GB shard store (%s); refusing (pass "
                    "LSQ_STORE_ALLOW_PAGEABLE to fall back to a pageable store)", total / 1e9, hipGetErrorString(e));
      }
      fprintf(stderr, "[lsq] could not page-lock the %.2f GB shard store; falling back to a PAGEABLE store: "
              "host-to-device copies become synchronous and stop overlapping compute\n", total / 1e9);
    }
  }
  if (!st->host) {
    st->host = static_cast<char*>(aligned_alloc(4096, up(total, 4096)));
    if (!st->host) {
      delete st;
      return fail(LSQ_ERR_OOM, "shard_store_create: cannot allocate %.2f GB of host memory", total / 1e9);
    }
  }
  *out = st;
  return LSQ_OK;
}

void shard_store_destroy(lsq_store* st) {
  if (!st) return;
  if (st->pinned)
    (void)hipHostFree(st->host);
  else
    free(st->host);
  delete st;
}

// ------------------------------------------------------------------ shard cache file
namespace {
constexpr int32_t kStoreFileVersion = 1;
struct StoreFileHeader {
  char magic[8];  // "LSQSTORE"
  int32_t version;
  int32_t hidden, n_heads, n_kv_heads, head_dim, intermediate, n_layers, qkv_bias, weight_kind;
  uint64_t layer_bytes;
};
static_assert(sizeof(StoreFileHeader) <= 4096, "store header fits its page");

// 64-bit checksum of a blob: a multiply-xorshift mix over 8-byte words (blob
// sizes are multiples of 4 KiB), seeded with the layer index.
uint64_t blob_checksum(const char* p, uint64_t n, int layer) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)layer;
  const uint64_t* w = reinterpret_cast<const uint64_t*>(p);
  for (uint64_t i = 0; i < n / 8; ++i) {
    h ^= w[i] + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    h *= 0xBF58476D1CE4E5B9ull;
  }
  h ^= h >> 31;
  return h;
}

uint64_t table_bytes(int n_layers) { return up(8ull * n_layers, 4096); }

int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n ? 0 : -1; }
int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : -1; }
}  // namespace

int shard_store_save(const lsq_store* st, const char* path) {
  LSQ_CHECK(st && path, LSQ_ERR_INVALID, "shard_store_save: null pointer");
  const lsq_model_cfg& c = st->cfg;
  std::vector<char> page(4096, 0);
  StoreFileHeader hdr{};
  memcpy(hdr.magic, "LSQSTORE", 8);
  hdr.version = kStoreFileVersion;
  hdr.hidden = c.hidden;
  hdr.n_heads = c.n_heads;
  hdr.n_kv_heads = c.n_kv_heads;
  hdr.head_dim = c.head_dim;
  hdr.intermediate = c.intermediate;
  hdr.n_layers = c.n_layers;
  hdr.qkv_bias = c.qkv_bias;
  hdr.weight_kind = c.weight_kind;
  hdr.layer_bytes = st->layer_bytes;
  memcpy(page.data(), &hdr, sizeof(hdr));
  std::vector<char> table(table_bytes(c.n_layers), 0);
  for (int l = 0; l < c.n_layers; ++l) {
    const uint64_t sum = blob_checksum(st->host + (uint64_t)l * st->layer_bytes, st->layer_bytes, l);
    memcpy(table.data() + 8ull * l, &sum, 8);
  }
  std::string tmp = std::string(path) + ".tmp";
  FILE* f = fopen(tmp.c_str(), "wb");
  LSQ_CHECK(f, LSQ_ERR_IO, "shard_store_save: cannot create %s", tmp.c_str());
  bool ok = write_all(f, page.data(), page.size()) == 0 && write_all(f, table.data(), table.size()) == 0 &&
            write_all(f, st->host, st->layer_bytes * (uint64_t)c.n_layers) == 0;
  ok = (fclose(f) == 0) && ok;
  if (!ok) {
    remove(tmp.c_str());
    return fail(LSQ_ERR_IO, "shard_store_save: writing %s failed", tmp.c_str());
  }
  if (rename(tmp.c_str(), path) != 0) {
    remove(tmp.c_str());
    return fail(LSQ_ERR_IO, "shard_store_save: cannot rename %s to %s", tmp.c_str(), path);
  }
  return LSQ_OK;
}

int shard_store_load(const char* path, const lsq_model_cfg* expect, int32_t flags, lsq_store** out) {
  LSQ_CHECK(path && out, LSQ_ERR_INVALID, "shard_store_load: null pointer");
  FILE* f = fopen(path, "rb");
  LSQ_CHECK(f, LSQ_ERR_IO, "shard_store_load: cannot open %s", path);
  std::vector<char> page(4096);
  StoreFileHeader hdr{};
  if (read_all(f, page.data(), page.size()) != 0) {
    fclose(f);
    return fail(LSQ_ERR_IO, "shard_store_load: %s is shorter than a store header", path);
  }
  memcpy(&hdr, page.data(), sizeof(hdr));
  if (memcmp(hdr.magic, "LSQSTORE", 8) != 0 || hdr.version != kStoreFileVersion) {
    fclose(f);
    return fail(LSQ_ERR_IO, "shard_store_load: %s is not a version-%d shard store", path, kStoreFileVersion);
  }
  lsq_model_cfg c{};
  if (expect) c = *expect;
  const struct {
    const char* name;
    int32_t file, want;
  } fields[] = {{"hidden", hdr.hidden, c.hidden},           {"n_heads", hdr.n_heads, c.n_heads},
                {"n_kv_heads", hdr.n_kv_heads, c.n_kv_heads}, {"head_dim", hdr.head_dim, c.head_dim},
                {"intermediate", hdr.intermediate, c.intermediate}, {"n_layers", hdr.n_layers, c.n_layers},
                {"qkv_bias", hdr.qkv_bias, c.qkv_bias},     {"weight_kind", hdr.weight_kind, c.weight_kind}};
  if (expect) {
    for (const auto& fd : fields) {
      if (fd.file != fd.want) {
        fclose(f);
        return fail(LSQ_ERR_STATE, "shard_store_load: %s was written for %s=%d but the run asks for %d; re-shard",
                    path, fd.name, fd.file, fd.want);
      }
    }
  } else {
    // no expectation: take the shape from the file and plausible defaults for the rest
    c.hidden = hdr.hidden;
    c.n_heads = hdr.n_heads;
    c.n_kv_heads = hdr.n_kv_heads;
    c.head_dim = hdr.head_dim;
    c.intermediate = hdr.intermediate;
    c.n_layers = hdr.n_layers;
    c.qkv_bias = hdr.qkv_bias;
    c.weight_kind = hdr.weight_kind;
    c.vocab = 8;
    c.lora_r = 8;
    c.rms_eps = 1e-5f;
    c.rope_theta = 1e4f;
    c.lora_scale = 1.f;
  }
  lsq_store* st = nullptr;
  if (int e = shard_store_create(&c, flags, &st)) {
    fclose(f);
    return e;
  }
  auto bad = [&](const char* why, int layer) {
    fclose(f);
    shard_store_destroy(st);
    return fail(LSQ_ERR_IO, "shard_store_load: %s: %s (layer %d)", path, why, layer);
  };
  if (hdr.layer_bytes != st->layer_bytes) return bad("blob size differs from this library's layout", -1);
  std::vector<char> table(table_bytes(c.n_layers));
  if (read_all(f, table.data(), table.size()) != 0) return bad("truncated checksum table", -1);
  for (int l = 0; l < c.n_layers; ++l) {
    char* blob = st->host + (uint64_t)l * st->layer_bytes;
    if (read_all(f, blob, st->layer_bytes) != 0) return bad("truncated", l);
    uint64_t want = 0;
    memcpy(&want, table.data() + 8ull * l, 8);
    if (blob_checksum(blob, st->layer_bytes, l) != want) return bad("checksum mismatch", l);
    BlobHeader bh{};
    memcpy(&bh, blob, sizeof(bh));
    if (memcmp(bh.magic, "LSQBLOB1", 8) != 0 || bh.layer != l) return bad("blob header names another layer", l);
  }
  char extra;
  if (fread(&extra, 1, 1, f) != 0) return bad("trailing bytes after the last blob", c.n_layers - 1);
  fclose(f);
  *out = st;
  return LSQ_OK;
}

int32_t shard_store_is_pinned(const lsq_store* st) { return st && st->pinned ? 1 : 0; }
uint64_t shard_store_layer_bytes(const lsq_store* st) { return st ? st->layer_bytes : 0; }
const void* shard_store_layer_host(const lsq_store* st, int32_t layer) {
  if (!st || layer < 0 || layer >= st->cfg.n_layers) return nullptr;
  return st->host + (uint64_t)layer * st->layer_bytes;
}

int shard_store_write_layer(lsq_store* st, int32_t layer, const lsq_layer_src* src, void* staging, size_t staging_bytes,
                            void* stream) {
  LSQ_CHECK(st && src && staging, LSQ_ERR_INVALID, "shard_store_write_layer: null pointer");
  LSQ_CHECK(layer >= 0 && layer < st->cfg.n_layers, LSQ_ERR_INVALID, "shard_store_write_layer: layer %d", layer);
  LSQ_CHECK(staging_bytes >= st->layer_bytes + 256, LSQ_ERR_WORKSPACE, "shard_store_write_layer: staging too small");
  LSQ_CHECK(aligned16(staging), LSQ_ERR_ALIGN, "shard_store_write_layer: unaligned staging");
  const lsq_model_cfg* c = &st->cfg;
  for (int i = 0; i < 7; ++i) LSQ_CHECK(src->w[i] && aligned16(src->w[i]), LSQ_ERR_INVALID, "layer src: weight %d", i);
  LSQ_CHECK(src->norm1 && src->norm2, LSQ_ERR_INVALID, "layer src: norms");
  if (c->qkv_bias) LSQ_CHECK(src->bias[0] && src->bias[1] && src->bias[2], LSQ_ERR_INVALID, "layer src: biases");
  hipStream_t s = as_stream(stream);
  lsq_blob_layout L;
  blob_layout(c, &L);
  const Dims d = dims_of(c);
  char* blob = static_cast<char*>(staging);
  int32_t* flag = reinterpret_cast<int32_t*>(blob + st->layer_bytes);
  LSQ_HIP(hipMemsetAsync(blob, 0, st->layer_bytes + 256, s));
  BlobHeader hdr{};
  memcpy(hdr.magic, "LSQBLOB1", 8);
  hdr.layer = layer;
  hdr.weight_kind = c->weight_kind;
  hdr.hidden = c->hidden;
  hdr.n_heads = c->n_heads;
  hdr.n_kv_heads = c->n_kv_heads;
  hdr.head_dim = c->head_dim;
  hdr.intermediate = c->intermediate;
  hdr.lora_r = c->lora_r;
  hdr.qkv_bias = c->qkv_bias;
  hdr.total_bytes = st->layer_bytes;
  LSQ_HIP(hipMemcpyAsync(blob, &hdr, sizeof(hdr), hipMemcpyHostToDevice, s));
  // projections in group order: qkv = q,k,v ; o ; gate|up = gate,up ; down
  const int group_of[7] = {0, 0, 0, 1, 2, 2, 3};
  const int rows_of[7] = {d.Nq, d.Nkv, d.Nkv, d.H, d.I, d.I, d.H};
  int row_off[7];
  for (int i = 0, g = -1, acc = 0; i < 7; ++i) {
    if (group_of[i] != g) {
      g = group_of[i];
      acc = 0;
    }
    row_off[i] = acc;
    acc += rows_of[i];
  }
  for (int i = 0; i < 7; ++i) {
    const int g = group_of[i];
    const int64_t K = d.gK[g];
    if (c->weight_kind == LSQ_W_NF4) {
      void* packed = blob + L.w_off[g] + (uint64_t)row_off[i] * (K / 2);
      float* absmax = reinterpret_cast<float*>(blob + L.absmax_off[g] + (uint64_t)row_off[i] * (K / 64) * 4);
      if (int e = nf4_quantize(src->w[i], LSQ_BF16, rows_of[i], K, 64, packed, absmax, flag, stream)) return e;
    } else {
      LSQ_HIP(hipMemcpyAsync(blob + L.w_off[g] + (uint64_t)row_off[i] * K * 2, src->w[i], (size_t)rows_of[i] * K * 2,
                             hipMemcpyDeviceToDevice, s));
    }
  }
  LSQ_HIP(hipMemcpyAsync(blob + L.norm1_off, src->norm1, 2ull * d.H, hipMemcpyDeviceToDevice, s));
  LSQ_HIP(hipMemcpyAsync(blob + L.norm2_off, src->norm2, 2ull * d.H, hipMemcpyDeviceToDevice, s));
  if (c->qkv_bias) {
    LSQ_HIP(hipMemcpyAsync(blob + L.bias_off, src->bias[0], 2ull * d.Nq, hipMemcpyDeviceToDevice, s));
    LSQ_HIP(hipMemcpyAsync(blob + L.bias_off + 2ull * d.Nq, src->bias[1], 2ull * d.Nkv, hipMemcpyDeviceToDevice, s));
    LSQ_HIP(hipMemcpyAsync(blob + L.bias_off + 2ull * (d.Nq + d.Nkv), src->bias[2], 2ull * d.Nkv,
                           hipMemcpyDeviceToDevice, s));
  }
  int32_t host_flag = 0;
  LSQ_HIP(hipMemcpyAsync(st->host + (uint64_t)layer * st->layer_bytes, blob, st->layer_bytes, hipMemcpyDeviceToHost,
                         s));
  LSQ_HIP(hipMemcpyAsync(&host_flag, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s));
  LSQ_HIP(hipStreamSynchronize(s));
  LSQ_CHECK(host_flag == 0, LSQ_ERR_NONFINITE, "shard_store_write_layer: layer %d has a NaN or Inf weight", layer);
  return LSQ_OK;
}

}  // extern "C"

// ================================================================== pool
namespace {
struct Slot {
  int layer = -1;
  bool held = false;
  bool ready_recorded = false;
  bool free_recorded = false;
  uint64_t last_use = 0;
  hipEvent_t ready = nullptr, free_ev = nullptr;
};
constexpr int kCopyTimers = 1024;
}  // namespace

struct lsq_pool {
  const lsq_store* store;
  int n;
  char* dev;
  uint64_t stride;
  hipStream_t compute, copy;
  hipStream_t own_copy = nullptr;   // a copy stream the pool created (see copy_stream_runs_beside)
  int flags;
  bool resident;
  std::vector<Slot> slots;
  uint64_t tick = 0;
  lsq_pool_stats stats{};
  std::vector<hipEvent_t> tev;  // copy timing pairs (ring)
  int tev_used = 0;
  hipEvent_t large_ready = nullptr, large_free = nullptr;  // the step's head buffer (LSQ_STEP_STREAM_LARGE)
  bool large_free_recorded = false;
  // timeline (lsq_timeline_enable): event pairs and what each one brackets
  std::vector<hipEvent_t> tl_ev;
  std::vector<int32_t> tl_kind, tl_layer;
  int tl_cap = 0, tl_used = 0, tl_dropped = 0;
};

namespace {
// Open a timeline record on stream st; returns its index, or -1 when off or full.
int tl_begin(lsq_pool* p, int kind, int layer, hipStream_t st) {
  if (p->tl_cap == 0) return -1;
  if (p->tl_used >= p->tl_cap) {
    ++p->tl_dropped;
    return -1;
  }
  const int i = p->tl_used++;
  p->tl_kind[i] = kind;
  p->tl_layer[i] = layer;
  if (hipEventRecord(p->tl_ev[2 * i], st) != hipSuccess) return -1;
  return i;
}
int tl_end(lsq_pool* p, int i, hipStream_t st) {
  if (i >= 0) LSQ_HIP(hipEventRecord(p->tl_ev[2 * i + 1], st));
  return LSQ_OK;
}

int find_slot(lsq_pool* p, int layer) {
  for (int i = 0; i < p->n; ++i)
    if (p->slots[i].layer == layer) return i;
  return -1;
}

int copy_into(lsq_pool* p, int si, int layer) {
  Slot& sl = p->slots[si];
  char* dst = p->dev + (uint64_t)si * p->stride;
  // The slot's last reader must be done before the copy lands.  The host waits
  // for that (the event's work is already enqueued, so the wait ends) and then
  // issues the copy: with the wait on the copy stream instead (a queue waiting
  // on the compute stream's event), copies ran at 52 rather than 56 GB/s and
  // every kernel beside them about 15% slower on the 8B-shaped stack.  The
  // step therefore issues each prefetch after enqueuing the current layer's
  // pass, so the compute stream has work queued while the host waits.
  if (sl.free_recorded) LSQ_HIP(hipEventSynchronize(sl.free_ev));
  if (p->flags & LSQ_POOL_POISON) LSQ_HIP(hipMemsetAsync(dst, 0xFF, p->store->layer_bytes, p->copy));
  const bool timed = p->tev_used < kCopyTimers;
  if (timed) LSQ_HIP(hipEventRecord(p->tev[2 * p->tev_used], p->copy));
  const int tl = p->resident ? -1 : tl_begin(p, LSQ_TL_COPY, layer, p->copy);
  LSQ_HIP(hipMemcpyAsync(dst, shard_store_layer_host(p->store, layer), p->store->layer_bytes, hipMemcpyHostToDevice,
                         p->copy));
  if (int e = tl_end(p, tl, p->copy)) return e;
  if (timed) {
    LSQ_HIP(hipEventRecord(p->tev[2 * p->tev_used + 1], p->copy));
    ++p->tev_used;
    p->stats.timed_copies += 1;
    p->stats.timed_bytes += p->store->layer_bytes;
  }
  LSQ_HIP(hipEventRecord(sl.ready, p->copy));
  sl.ready_recorded = true;
  sl.layer = layer;
  sl.last_use = ++p->tick;
  p->stats.copies += 1;
  p->stats.copy_bytes += p->store->layer_bytes;
  return LSQ_OK;
}
// ---- can the copy stream run while the compute stream is busy?
// HIP places streams on a few hardware queues (GPU_MAX_HW_QUEUES, 4 by
// default); once there are more streams than queues, a new stream shares the
// queue of an existing one, and work on two streams of one queue runs in
// submission order.  A copy stream on the compute stream's queue waits behind
// every kernel enqueued before each copy, so the copies stop overlapping
// compute (a step of the 8B-shaped stack went from 142 to 197 ms when the
// caller had created two other streams first).  The check: a kernel on the
// compute stream waits, for at most kProbeMs, for a flag that a kernel on the
// copy stream sets.  Both loops end on their own: the wait by time and by an
// iteration cap, whatever the other stream does.
constexpr int kProbeMs = 20;
__global__ void pool_probe_clear_kernel(int* w) {
  if (threadIdx.x < 2) w[threadIdx.x] = 0;
}
__global__ void pool_probe_set_kernel(int* w) { __hip_atomic_store(w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__global__ void pool_probe_wait_kernel(int* w, long long ticks, int max_iter) {
  const long long t0 = wall_clock64();
  int seen = 0;
  for (int i = 0; i < max_iter; ++i) {
    seen = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (seen || wall_clock64() - t0 > ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
  w[1] = seen;
}

// *ok: a kernel on `copy` ran while the compute stream was busy.  Uses the
// first 8 bytes of slot 0, which holds nothing before the first copy.
int copy_stream_runs_beside(lsq_pool* p, hipStream_t copy, bool* ok) {
  int dev = 0, khz = 0;
  LSQ_HIP(hipGetDevice(&dev));
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
  int* w = reinterpret_cast<int*>(p->dev);
  hipEvent_t cleared;
  LSQ_HIP(hipEventCreateWithFlags(&cleared, hipEventDisableTiming));
  pool_probe_clear_kernel<<<1, 64, 0, p->compute>>>(w);
  LSQ_HIP(hipEventRecord(cleared, p->compute));
  pool_probe_wait_kernel<<<1, 64, 0, p->compute>>>(w, (long long)khz * kProbeMs, 1 << 20);
  LSQ_HIP(hipStreamWaitEvent(copy, cleared, 0));
  pool_probe_set_kernel<<<1, 64, 0, copy>>>(w);
  int res[2] = {0, 0};
  LSQ_HIP(hipMemcpyAsync(res, w, sizeof(res), hipMemcpyDeviceToHost, p->compute));
  LSQ_HIP(hipStreamSynchronize(copy));
  LSQ_HIP(hipStreamSynchronize(p->compute));
  LSQ_HIP(hipGetLastError());
  LSQ_HIP(hipEventDestroy(cleared));
  *ok = res[1] != 0;
  return LSQ_OK;
}

// Keep the caller's copy stream if it runs beside the compute stream, else
// create streams until one does (each new stream goes to the least used
// queue, so a few tries reach a queue of its own).
int choose_copy_stream(lsq_pool* p) {
  bool ok = false;
  if (p->copy && p->copy != p->compute)
    if (int e = copy_stream_runs_beside(p, p->copy, &ok)) return e;
  std::vector<hipStream_t> tried;
  for (int t = 0; !ok && t < 4; ++t) {
    hipStream_t s = nullptr;
    LSQ_HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    tried.push_back(s);
    if (int e = copy_stream_runs_beside(p, s, &ok)) return e;
    if (ok) {
      p->own_copy = s;
      p->copy = s;
      tried.pop_back();
    }
  }
  for (hipStream_t s : tried) LSQ_HIP(hipStreamDestroy(s));
  if (!ok && !p->copy) {
    LSQ_HIP(hipStreamCreateWithFlags(&p->own_copy, hipStreamNonBlocking));
    p->copy = p->own_copy;
  }
  if (!ok)
    fprintf(stderr, "layer_pool_create: no copy stream found that runs beside the compute stream; layer copies "
                    "will serialize with compute\n");
  return LSQ_OK;
}
}  // namespace

extern "C" {

int layer_pool_create(const lsq_store* store, int32_t n_buffers, void* dev_slots, uint64_t slot_stride,
                      void* compute_stream, void* copy_stream, int32_t flags, lsq_pool** out) {
  LSQ_CHECK(store && dev_slots && out, LSQ_ERR_INVALID, "layer_pool_create: null pointer");
  const bool resident = flags & LSQ_POOL_RESIDENT;
  if (resident)
    LSQ_CHECK(n_buffers == store->cfg.n_layers, LSQ_ERR_INVALID, "resident pool needs n_buffers == n_layers");
  else
    LSQ_CHECK(n_buffers >= 2 && n_buffers <= 8, LSQ_ERR_INVALID,
              "stream_buffers must be in [2, 8] (got %d): a refusal, not a clamp", n_buffers);
  LSQ_CHECK(slot_stride >= store->layer_bytes && slot_stride % 4096 == 0 && aligned16(dev_slots), LSQ_ERR_ALIGN,
            "layer_pool_create: slot stride must cover a blob and be a multiple of 4096");
  lsq_pool* p = new (std::nothrow) lsq_pool();
  LSQ_CHECK(p, LSQ_ERR_OOM, "layer_pool_create: out of memory");
  p->store = store;
  p->n = n_buffers;
  p->dev = static_cast<char*>(dev_slots);
  p->stride = slot_stride;
  p->compute = as_stream(compute_stream);
  p->copy = as_stream(copy_stream);
  p->flags = flags;
  p->resident = resident;
  p->slots.resize(n_buffers);
  p->tev.resize(2 * kCopyTimers);
  for (auto& e : p->tev) LSQ_HIP(hipEventCreate(&e));
  for (auto& s : p->slots) {
    LSQ_HIP(hipEventCreateWithFlags(&s.ready, hipEventDisableTiming));
    LSQ_HIP(hipEventCreateWithFlags(&s.free_ev, hipEventDisableTiming));
  }
  LSQ_HIP(hipEventCreateWithFlags(&p->large_ready, hipEventDisableTiming));
  LSQ_HIP(hipEventCreateWithFlags(&p->large_free, hipEventDisableTiming));
  if (resident) {
    if (!p->copy) p->copy = p->compute;   // copies once, at create
    for (int i = 0; i < n_buffers; ++i)
      if (int e = copy_into(p, i, i)) return e;
    LSQ_HIP(hipStreamSynchronize(p->copy));
  } else if (int e = choose_copy_stream(p)) {
    layer_pool_destroy(p);
    return e;
  }
  *out = p;
  return LSQ_OK;
}

void layer_pool_destroy(lsq_pool* p) {
  if (!p) return;
  (void)hipStreamSynchronize(p->copy);
  (void)hipStreamSynchronize(p->compute);
  for (auto& e : p->tev) (void)hipEventDestroy(e);
  for (auto& e : p->tl_ev) (void)hipEventDestroy(e);
  for (auto& s : p->slots) {
    (void)hipEventDestroy(s.ready);
    (void)hipEventDestroy(s.free_ev);
  }
  if (p->large_ready) (void)hipEventDestroy(p->large_ready);
  if (p->large_free) (void)hipEventDestroy(p->large_free);
  if (p->own_copy) (void)hipStreamDestroy(p->own_copy);
  delete p;
}

int layer_pool_copy_stream(const lsq_pool* p, void** stream) {
  LSQ_CHECK(p && stream, LSQ_ERR_INVALID, "layer_pool_copy_stream: null pointer");
  *stream = p->copy;
  return LSQ_OK;
}

int stream_layer_prefetch(lsq_pool* p, int32_t layer) {
  LSQ_CHECK(p && layer >= 0 && layer < p->store->cfg.n_layers, LSQ_ERR_INVALID, "prefetch: bad layer %d", layer);
  int si = find_slot(p, layer);
  if (si >= 0) {
    p->stats.hits += 1;
    p->slots[si].last_use = ++p->tick;
    return LSQ_OK;
  }
  LSQ_CHECK(!p->resident, LSQ_ERR_STATE, "prefetch: resident pool lost layer %d", layer);
  int victim = -1;
  for (int i = 0; i < p->n; ++i) {
    if (p->slots[i].held) continue;
    if (victim < 0 || p->slots[i].last_use < p->slots[victim].last_use) victim = i;
  }
  LSQ_CHECK(victim >= 0, LSQ_ERR_STATE, "prefetch: every slot is held (release a layer first)");
  return copy_into(p, victim, layer);
}

int layer_pool_acquire(lsq_pool* p, int32_t layer, const void** blob_dev) {
  LSQ_CHECK(p && blob_dev, LSQ_ERR_INVALID, "acquire: null pointer");
  int si = find_slot(p, layer);
  LSQ_CHECK(si >= 0, LSQ_ERR_STATE, "acquire: layer %d was never prefetched", layer);
  Slot& sl = p->slots[si];
  if (sl.ready_recorded && !p->resident) LSQ_HIP(hipStreamWaitEvent(p->compute, sl.ready, 0));
  sl.held = true;
  sl.last_use = ++p->tick;
  *blob_dev = p->dev + (uint64_t)si * p->stride;
  return LSQ_OK;
}

int layer_pool_release(lsq_pool* p, int32_t layer) {
  LSQ_CHECK(p, LSQ_ERR_INVALID, "release: null pool");
  int si = find_slot(p, layer);
  LSQ_CHECK(si >= 0 && p->slots[si].held, LSQ_ERR_STATE, "release: layer %d is not held", layer);
  Slot& sl = p->slots[si];
  LSQ_HIP(hipEventRecord(sl.free_ev, p->compute));
  sl.free_recorded = true;
  sl.held = false;
  return LSQ_OK;
}

int lsq_timeline_enable(lsq_pool* p, int32_t capacity) {
  LSQ_CHECK(p && capacity >= 0 && capacity <= (1 << 20), LSQ_ERR_INVALID, "lsq_timeline_enable: bad capacity %d",
            capacity);
  LSQ_HIP(hipStreamSynchronize(p->copy));
  LSQ_HIP(hipStreamSynchronize(p->compute));
  for (auto& e : p->tl_ev) LSQ_HIP(hipEventDestroy(e));
  p->tl_ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& e : p->tl_ev) LSQ_HIP(hipEventCreate(&e));
  p->tl_kind.assign(capacity, 0);
  p->tl_layer.assign(capacity, 0);
  p->tl_cap = capacity;
  p->tl_used = p->tl_dropped = 0;
  return LSQ_OK;
}

int lsq_timeline_read(lsq_pool* p, lsq_timeline_entry* out, int32_t max, int32_t* n, int32_t* dropped) {
  LSQ_CHECK(p && n && (out || max == 0) && max >= 0, LSQ_ERR_INVALID, "lsq_timeline_read: null pointer");
  const int cnt = std::min(p->tl_used, (int)max);
  for (int i = 0; i < cnt; ++i) {
    LSQ_HIP(hipEventSynchronize(p->tl_ev[2 * i + 1]));
    float a = 0.f, b = 0.f;
    LSQ_HIP(hipEventElapsedTime(&a, p->tl_ev[0], p->tl_ev[2 * i]));
    LSQ_HIP(hipEventElapsedTime(&b, p->tl_ev[0], p->tl_ev[2 * i + 1]));
    out[i] = lsq_timeline_entry{p->tl_kind[i], p->tl_layer[i], (double)a, (double)b};
  }
  *n = cnt;
  if (dropped) *dropped = p->tl_dropped + (p->tl_used - cnt);
  p->tl_used = p->tl_dropped = 0;
  return LSQ_OK;
}

int layer_pool_stats(lsq_pool* p, int32_t reset, lsq_pool_stats* out) {
  LSQ_CHECK(p && out, LSQ_ERR_INVALID, "layer_pool_stats: null pointer");
  double ms = 0.0;
  for (int t = 0; t < p->tev_used; ++t) {
    LSQ_HIP(hipEventSynchronize(p->tev[2 * t + 1]));
    float e = 0.f;
    LSQ_HIP(hipEventElapsedTime(&e, p->tev[2 * t], p->tev[2 * t + 1]));
    ms += e;
  }
  p->stats.copy_ms += ms;
  p->tev_used = 0;
  *out = p->stats;
  if (reset) p->stats = lsq_pool_stats{};
  return LSQ_OK;
}

}  // extern "C"

// ================================================================== step
namespace {
struct StepWs {
  float* xs;         // (L+1) x [T, H] layer inputs (checkpoints)
  float* dxa;        // [T, H]
  float* dxb;        // [T, H]
  uint16_t* xf;      // [T, H]  final-norm output, bf16
  int chunk;         // tokens per head / cross-entropy chunk
  float* logits;     // [chunk, V]
  uint16_t* dlogits; // [chunk, V]
  uint16_t* head;    // LSQ_STEP_STREAM_LARGE: the head, copied in each step [V, H]
  float* loss_rows;  // [T]
  float* dxf;        // [T, H]
  int32_t* bad;      // [1]
  void* gemm;        // split-K partials of the head GEMMs
  size_t gemm_bytes;
  void* layer;       // layer workspace
  size_t layer_bytes;
  char* acts;        // n_kept x acts_bytes of kept forward activations
  size_t acts_bytes;
  int n_kept;
  char* ustore;      // n_layers x ustore_bytes: each layer's rank-r store (U, U32) for its recompute
  size_t ustore_bytes;
  uint16_t* lora_t;  // every layer's adapters transposed block by block, once per step
  float* xr[2];      // reference mode: the adapters-off residual stream, ping-pong [T, H]
  float* ref_loss_tmp;  // reference mode: its mean loss when the caller wants rows only
  size_t total;
};

// Layers whose forward activations a step keeps: all of them under
// LSQ_STEP_KEEP_ACTIVATIONS, none under LSQ_STEP_RECOMPUTE_ALL, else the ones
// whose backward runs while the copy stream idles (L-1 at the turn, 1 and 0 at
// the tail).  Returns the count; slot[i] = the layer's region index or -1.
int kept_layers(const lsq_model_cfg* c, int32_t flags, std::vector<int>* slot_out) {
  const int L = c->n_layers;
  std::vector<int> slot(L, -1);
  int n = 0;
  if (flags & LSQ_STEP_KEEP_ACTIVATIONS) {
    for (int i = 0; i < L; ++i) slot[i] = n++;
  } else if (!(flags & (LSQ_STEP_RECOMPUTE_ALL | LSQ_STEP_FORWARD_ONLY))) {
    for (int i : {L - 1, 1, 0})
      if (i >= 0 && i < L && slot[i] < 0) slot[i] = n++;
  }
  if (slot_out) *slot_out = std::move(slot);
  return n;
}

StepWs carve_step(const lsq_model_cfg* c, int B, int S, void* base, int32_t flags) {
  const bool keep = flags & LSQ_STEP_KEEP_ACTIVATIONS;
  const int n_kept = kept_layers(c, flags, nullptr);
  const uint64_t T = (uint64_t)B * S, H = c->hidden, V = c->vocab;
  StepWs w{};
  uint64_t off = 0;
  char* p = static_cast<char*>(base);
  auto take = [&](uint64_t bytes) -> void* {
    void* r = base ? p + off : nullptr;
    off = up(off + std::max<uint64_t>(bytes, 1), 256);
    return r;
  };
  w.xs = static_cast<float*>(take(4 * T * H * (c->n_layers + 1)));
  w.dxa = static_cast<float*>(take(4 * T * H));
  w.dxb = static_cast<float*>(take(4 * T * H));
  w.xf = static_cast<uint16_t*>(take(2 * T * H));
  const uint64_t Tc = (c->loss_chunk > 0 && (uint64_t)c->loss_chunk < T) ? (uint64_t)c->loss_chunk : T;
  w.chunk = (int)Tc;
  w.logits = static_cast<float*>(take(4 * Tc * V));
  w.dlogits = static_cast<uint16_t*>(take(2 * Tc * V));
  w.loss_rows = static_cast<float*>(take(4 * T));
  w.dxf = static_cast<float*>(take(4 * T * H));
  w.bad = static_cast<int32_t*>(take(4));
  w.gemm_bytes = std::max(gemm_fwd_ws_bytes((int)Tc, (int)V, (int)H), gemm_bwd_ws_bytes((int)Tc, (int)V, (int)H, 0));
  // a last, shorter chunk can split differently: size for it too
  if (T % Tc)
    w.gemm_bytes = std::max(w.gemm_bytes, std::max(gemm_fwd_ws_bytes((int)(T % Tc), (int)V, (int)H),
                                                   gemm_bwd_ws_bytes((int)(T % Tc), (int)V, (int)H, 0)));
  if (flags & LSQ_STEP_STREAM_LARGE) w.head = static_cast<uint16_t*>(take(2 * V * H));
  w.gemm = take(w.gemm_bytes);
  w.layer_bytes = layer_ws_bytes(c, B, S, keep);
  w.layer = take(w.layer_bytes);
  {
    lsq_lora_layout LL;
    lora_layout(c, &LL);
    w.lora_t = static_cast<uint16_t*>(take(2 * LL.layer_elems * (uint64_t)c->n_layers));
  }
  if (n_kept > 0) {
    w.acts_bytes = layer_acts_bytes(c, B, S);
    w.acts = static_cast<char*>(take(w.acts_bytes * (uint64_t)n_kept));
  }
  w.n_kept = n_kept;
  if (!(flags & LSQ_STEP_FORWARD_ONLY)) {
    w.ustore_bytes = layer_ustore_bytes(c, B, S);
    w.ustore = static_cast<char*>(take(w.ustore_bytes * (uint64_t)c->n_layers));
  }
  if (flags & LSQ_STEP_REFERENCE_FORWARD) {
    w.xr[0] = static_cast<float*>(take(4 * T * H));
    w.xr[1] = static_cast<float*>(take(4 * T * H));
    w.ref_loss_tmp = static_cast<float*>(take(4));
  }
  w.total = off;
  return w;
}

struct AliasCtx {
  lsq_pool* pool;
  int layer;
  int other;
  int rc;
};

// Control for the aliasing defect: hand the slot back after the recompute and
// let a different layer's copy land in it before the backward GEMMs read it.
int early_release_hook(void* vctx) {
  AliasCtx* a = static_cast<AliasCtx*>(vctx);
  lsq_pool* p = a->pool;
  const int si = find_slot(p, a->layer);
  if (si < 0) return fail(LSQ_ERR_STATE, "early release: layer %d not in a slot", a->layer);
  if (int e = layer_pool_release(p, a->layer)) return e;
  if (int e = copy_into(p, si, a->other)) return e;
  LSQ_HIP(hipStreamWaitEvent(p->compute, p->slots[si].ready, 0));
  return LSQ_OK;
}
}  // namespace

extern "C" {

size_t lsq_step_workspace_size(const lsq_model_cfg* cfg, int32_t batch, int32_t seq, int32_t flags) {
  if (check_cfg(cfg) || batch < 1 || seq < 1) return 0;
  return carve_step(cfg, batch, seq, nullptr, flags).total;
}

// The head on a final residual x, chunk by chunk of tokens (stream_loss_chunk):
// final RMSNorm (rounded to bf16 once), logits in float32, cross-entropy rows;
// with dxf, also dlogits (bf16) -> dxf = dlogits head.  Rows are independent,
// so chunking changes no value's definition, only the buffers' size.
// logits_out (nullable) receives every row's logits; loss gets the mean.
static int head_pass(const lsq_model_cfg* cfg, const lsq_resident* res, const void* head, const StepWs& w,
                     const float* x, const int32_t* ids, int B, int S, float* logits_out, float* loss_rows,
                     float* loss, float* dxf, hipStream_t s) {
  const int T = B * S, H = cfg->hidden, V = cfg->vocab;
  if (int e = rmsnorm_fwd(x, static_cast<const uint16_t*>(res->final_norm), T, H, cfg->rms_eps, w.xf, H, nullptr, s))
    return e;
  for (int r0 = 0; r0 < T; r0 += w.chunk) {
    const int n = std::min(w.chunk, T - r0);
    float* logits = logits_out ? logits_out + (int64_t)r0 * V : w.logits;
    {
      FwdParams p{};
      p.X = w.xf + (int64_t)r0 * H;
      p.ldx = H;
      p.kind = LSQ_W_BF16;
      p.W = head;
      p.M = n;
      p.N = V;
      p.K = H;
      p.r = 0;
      p.nseg = 1;
      p.seg_end[0] = V;
      p.out = logits;
      p.ldc = V;
      if (int e = gemm_fwd(p, EPI_F32, s, w.gemm, w.gemm_bytes)) return e;
    }
    if (int e = cross_entropy_rows(logits, ids, B, S, V, r0, n, loss_rows, w.dlogits, nullptr, s)) return e;
    if (!dxf) continue;
    {
      BwdParams p{};
      p.dY = w.dlogits;
      p.ldy = V;
      p.kind = LSQ_W_BF16;
      p.W = head;
      p.M = n;
      p.N = V;
      p.K = H;
      p.rr = 0;
      p.out = dxf + (int64_t)r0 * H;
      p.ldc = H;
      if (int e = gemm_bwd(p, EPI_F32, s, w.gemm, w.gemm_bytes)) return e;
    }
  }
  return loss_mean(loss_rows, B, S, loss, s);
}

// Blob-shaping fields only: a store can serve steps that differ in anything else.
static bool same_store_shape(const lsq_model_cfg* a, const lsq_model_cfg* b) {
  return a->hidden == b->hidden && a->n_heads == b->n_heads && a->n_kv_heads == b->n_kv_heads &&
         a->head_dim == b->head_dim && a->intermediate == b->intermediate && a->n_layers == b->n_layers &&
         a->qkv_bias == b->qkv_bias && a->weight_kind == b->weight_kind;
}

int lsq_train_step_ex(const lsq_model_cfg* cfg, lsq_pool* pool, const lsq_resident* res, const int32_t* ids,
                      int32_t B, int32_t S, float* loss, float* logits_out, int32_t flags, void* ws, size_t ws_bytes,
                      const lsq_step_extra* extra) {
  float* x_trace = extra ? extra->x_trace : nullptr;
  float* dx_trace = extra ? extra->dx_trace : nullptr;
  const bool ref = flags & LSQ_STEP_REFERENCE_FORWARD;
  LSQ_CHECK(!ref || (extra && (extra->ref_nll_rows || extra->ref_loss)), LSQ_ERR_INVALID,
            "lsq_train_step: the reference forward needs ref_nll_rows or ref_loss");
  if (int e = check_cfg(cfg)) return e;
  LSQ_CHECK(pool && res && ids && loss && ws, LSQ_ERR_INVALID, "lsq_train_step: null pointer");
  LSQ_CHECK(res->embed && res->head && res->final_norm && res->lora && (res->lora_grad || (flags & LSQ_STEP_FORWARD_ONLY)),
            LSQ_ERR_INVALID, "lsq_train_step: resident tensors missing");
  LSQ_CHECK(B >= 1 && S >= 2 && (int64_t)B * S < (1 << 24), LSQ_ERR_SHAPE, "lsq_train_step: bad batch/seq");
  LSQ_CHECK(same_store_shape(cfg, &pool->store->cfg), LSQ_ERR_INVALID, "lsq_train_step: cfg differs from the store's");
  LSQ_CHECK((flags & ~(LSQ_STEP_FORWARD_ONLY | LSQ_STEP_DEBUG_EARLY_RELEASE | LSQ_STEP_KEEP_ACTIVATIONS |
                       LSQ_STEP_REFERENCE_FORWARD | LSQ_STEP_STREAM_LARGE | LSQ_STEP_RECOMPUTE_ALL)) == 0,
            LSQ_ERR_INVALID, "lsq_train_step: unknown flags 0x%x", flags);
  LSQ_CHECK(!((flags & LSQ_STEP_KEEP_ACTIVATIONS) && (flags & LSQ_STEP_RECOMPUTE_ALL)), LSQ_ERR_INVALID,
            "lsq_train_step: LSQ_STEP_KEEP_ACTIVATIONS and LSQ_STEP_RECOMPUTE_ALL contradict each other");
  const bool large = flags & LSQ_STEP_STREAM_LARGE;
  LSQ_CHECK(!large || !cfg->tied, LSQ_ERR_INVALID,
            "lsq_train_step: large-layer streaming is for an untied embedding and head (a tied one stays resident)");
  LSQ_CHECK(!large || !pool->resident, LSQ_ERR_INVALID, "lsq_train_step: large-layer streaming needs a streamed pool");
  const void* embed = res->embed;
  const void* head_src = res->head;
  if (large) {
    // both live in page-locked host memory; the gather reads the embedding in place
    void* dev = nullptr;
    LSQ_CHECK(hipHostGetDevicePointer(&dev, const_cast<void*>(res->embed), 0) == hipSuccess && dev, LSQ_ERR_INVALID,
              "lsq_train_step: the embedding must be page-locked host memory for large-layer streaming");
    embed = dev;
    LSQ_CHECK(hipHostGetDevicePointer(&dev, const_cast<void*>(res->head), 0) == hipSuccess, LSQ_ERR_INVALID,
              "lsq_train_step: the head must be page-locked host memory for large-layer streaming");
  }
  const size_t need = carve_step(cfg, B, S, nullptr, flags).total;
  LSQ_CHECK(ws_bytes >= need, LSQ_ERR_WORKSPACE, "lsq_train_step: workspace %zu < %zu (flags 0x%x)", ws_bytes, need,
            flags);
  LSQ_CHECK(!(flags & LSQ_STEP_DEBUG_EARLY_RELEASE) || (cfg->n_layers >= 2 && !pool->resident), LSQ_ERR_INVALID,
            "early-release control needs a streamed pool and >= 2 layers");
  const int L = cfg->n_layers, T = B * S, H = cfg->hidden, V = cfg->vocab;
  hipStream_t s = pool->compute;
  StepWs w = carve_step(cfg, B, S, ws, flags);
  lsq_model_cfg cfg_ref = *cfg;
  cfg_ref.lora_scale = 0.f;
  std::vector<int> kslot;
  kept_layers(cfg, flags, &kslot);
  auto acts_at = [&](int i) -> void* {
    return (w.acts && kslot[i] >= 0) ? w.acts + (uint64_t)kslot[i] * w.acts_bytes : nullptr;
  };
  // a recomputed layer keeps its down projections from the forward for the recompute
  auto ustore_at = [&](int i) -> void* {
    return (w.ustore && kslot[i] < 0) ? w.ustore + (uint64_t)i * w.ustore_bytes : nullptr;
  };
  lsq_lora_layout LL;
  lora_layout(cfg, &LL);
  const uint16_t* lora = static_cast<const uint16_t*>(res->lora);
  float* xs = w.xs;
  auto x_at = [&](int i) { return xs + (uint64_t)i * T * H; };

  if (int e = zero_words(w.bad, 1, 1, 1, s)) return e;
  // once per step: the rotary table and zeroed counters of the layer
  // workspace, and the adapters transposed for the backward's products
  if (int e = layer_prepare(cfg, B, S, w.layer, s)) return e;
  if (!(flags & LSQ_STEP_FORWARD_ONLY))
    if (int e = adapter_transpose(cfg, lora, w.lora_t, L, s)) return e;
  if (int e = embed_gather(ids, static_cast<const uint16_t*>(embed), T, H, V, x_at(0), w.bad, s)) return e;
  // the head's copy is queued on the copy stream behind the forward's layer
  // copies (issued after the prefetch of the last layer) and waited for at the turn
  auto queue_head_copy = [&]() -> int {
    lsq_pool* P = pool;
    if (P->large_free_recorded) LSQ_HIP(hipEventSynchronize(P->large_free));   // as in copy_into
    const int tl = tl_begin(P, LSQ_TL_LARGE_COPY, -1, P->copy);
    LSQ_HIP(hipMemcpyAsync(w.head, head_src, (size_t)V * H * 2, hipMemcpyHostToDevice, P->copy));
    if (int e = tl_end(P, tl, P->copy)) return e;
    LSQ_HIP(hipEventRecord(P->large_ready, P->copy));
    P->stats.large_copies += 1;
    P->stats.large_bytes += (uint64_t)V * H * 2;
    return LSQ_OK;
  };
  // ---- forward: acquire, compute, release, then prefetch one ahead (the
  // copy waits on the host for the slot the previous layer released)
  if (int e = stream_layer_prefetch(pool, 0)) return e;
  if (large && L == 1)
    if (int e = queue_head_copy()) return e;
  for (int i = 0; i < L; ++i) {
    const void* blob = nullptr;
    if (int e = layer_pool_acquire(pool, i, &blob)) return e;
    const int tl = tl_begin(pool, LSQ_TL_FWD, i, s);
    if (int e = layer_fwd(cfg, blob, lora + (uint64_t)i * LL.layer_elems, x_at(i), B, S, x_at(i + 1), w.layer, s,
                          acts_at(i), ustore_at(i)))
      return e;
    if (ref) {
      // the reference model on the same bytes while they are in the slot: adapters off (scale 0)
      const float* xin = i == 0 ? x_at(0) : w.xr[(i - 1) & 1];
      if (int e = layer_fwd(&cfg_ref, blob, lora + (uint64_t)i * LL.layer_elems, xin, B, S, w.xr[i & 1], w.layer, s,
                            nullptr))
        return e;
    }
    if (int e = tl_end(pool, tl, s)) return e;
    if (int e = layer_pool_release(pool, i)) return e;
    if (i + 1 < L)
      if (int e = stream_layer_prefetch(pool, i + 1)) return e;
    if (large && i + 1 == L - 1)
      if (int e = queue_head_copy()) return e;
  }
  const int tl_head = tl_begin(pool, LSQ_TL_HEAD, -1, s);
  const void* head = head_src;
  if (large) {
    LSQ_HIP(hipStreamWaitEvent(s, pool->large_ready, 0));
    head = w.head;
  }
  if (ref) {
    if (int e = head_pass(cfg, res, head, w, w.xr[(L - 1) & 1], ids, B, S, nullptr,
                          extra->ref_nll_rows ? extra->ref_nll_rows : w.loss_rows,
                          extra->ref_loss ? extra->ref_loss : w.ref_loss_tmp, nullptr, s))
      return e;
  }
  // ---- head and loss: resident head, or the copy queued during the forward
  const bool fwd_only = flags & LSQ_STEP_FORWARD_ONLY;
  if (int e = head_pass(cfg, res, head, w, x_at(L), ids, B, S, logits_out, w.loss_rows, loss,
                        fwd_only ? nullptr : w.dxf, s))
    return e;
  if (large) {
    LSQ_HIP(hipEventRecord(pool->large_free, s));
    pool->large_free_recorded = true;
  }
  if (fwd_only) return tl_end(pool, tl_head, s);
  float* dcur = w.dxa;
  float* dnext = w.dxb;
  // dh of the last layer, and its bf16 copy where that layer's backward looks for it
  if (int e = rmsnorm_bwd(x_at(L), static_cast<const uint16_t*>(res->final_norm), w.dxf, nullptr, T, H, cfg->rms_eps,
                          dcur, layer_bwd_dy_b(cfg, B, S, w.layer), s))
    return e;
  if (int e = tl_end(pool, tl_head, s)) return e;
  const size_t act = sizeof(float) * (size_t)T * H;
  if (x_trace) LSQ_HIP(hipMemcpyAsync(x_trace, xs, act * (L + 1), hipMemcpyDeviceToDevice, s));
  if (dx_trace) LSQ_HIP(hipMemcpyAsync(dx_trace + (size_t)L * T * H, dcur, act, hipMemcpyDeviceToDevice, s));
  // ---- backward: the same stream of layers in reverse, recompute inside each
  // layer unless its forward activations were kept (the weights are re-read
  // either way: the backward needs W for dX)
  if (int e = stream_layer_prefetch(pool, L - 1)) return e;
  for (int i = L - 1; i >= 0; --i) {
    const void* blob = nullptr;
    if (int e = layer_pool_acquire(pool, i, &blob)) return e;
    const bool early = flags & LSQ_STEP_DEBUG_EARLY_RELEASE;
    AliasCtx actx{pool, i, (i + 1) % L, 0};
    LayerHook hook{early_release_hook, &actx};
    float* grad = res->lora_grad + (uint64_t)i * LL.layer_elems;
    const int tl = tl_begin(pool, LSQ_TL_BWD, i, s);
    if (int e = layer_bwd(cfg, blob, lora + (uint64_t)i * LL.layer_elems, w.lora_t + (uint64_t)i * LL.layer_elems,
                          x_at(i), dcur, B, S, dnext, grad, 0, w.layer,
                          s, early ? &hook : nullptr, acts_at(i), /*dy_b_ready=*/true, ustore_at(i)))
      return e;
    if (int e = tl_end(pool, tl, s)) return e;
    if (!early)
      if (int e = layer_pool_release(pool, i)) return e;
    if (i - 1 >= 0)
      if (int e = stream_layer_prefetch(pool, i - 1)) return e;
    std::swap(dcur, dnext);
    if (dx_trace) LSQ_HIP(hipMemcpyAsync(dx_trace + (size_t)i * T * H, dcur, act, hipMemcpyDeviceToDevice, s));
  }
  return LSQ_OK;
}

int lsq_train_step_traced(const lsq_model_cfg* cfg, lsq_pool* pool, const lsq_resident* res, const int32_t* ids,
                          int32_t B, int32_t S, float* loss, float* logits_out, int32_t flags, void* ws,
                          size_t ws_bytes, float* x_trace, float* dx_trace) {
  LSQ_CHECK(!(flags & LSQ_STEP_REFERENCE_FORWARD), LSQ_ERR_INVALID,
            "lsq_train_step_traced: the reference forward needs lsq_train_step_ex");
  lsq_step_extra ex{x_trace, dx_trace, nullptr, nullptr};
  return lsq_train_step_ex(cfg, pool, res, ids, B, S, loss, logits_out, flags, ws, ws_bytes, &ex);
}

int lsq_train_step(const lsq_model_cfg* cfg, lsq_pool* pool, const lsq_resident* res, const int32_t* ids, int32_t B,
                   int32_t S, float* loss, float* logits_out, int32_t flags, void* ws, size_t ws_bytes) {
  return lsq_train_step_traced(cfg, pool, res, ids, B, S, loss, logits_out, flags, ws, ws_bytes, nullptr, nullptr);
}

// ================================================================== pre-flight
int vram_predict_peak(const lsq_model_cfg* cfg, int32_t batch, int32_t seq, int32_t n_buffers, int32_t step_flags,
                      lsq_vram_breakdown* out) {
  if (int e = check_cfg(cfg)) return e;
  LSQ_CHECK(out && batch >= 1 && seq >= 2 && n_buffers >= 2, LSQ_ERR_INVALID, "vram_predict_peak: bad arguments");
  lsq_blob_layout BL;
  blob_layout(cfg, &BL);
  lsq_lora_layout LL;
  lora_layout(cfg, &LL);
  const uint64_t T = (uint64_t)batch * seq, H = cfg->hidden;
  out->slots = (uint64_t)n_buffers * up(BL.total_bytes, 4096);   // layer_pool_create's slot stride
  // large-layer streaming keeps the embedding and head in host memory (the
  // head's per-step device copy is part of the step workspace)
  out->resident = (step_flags & LSQ_STEP_STREAM_LARGE) ? 2 * H : 2ull * cfg->vocab * H * (cfg->tied ? 1 : 2) + 2 * H;
  out->adapters = LL.layer_elems * (uint64_t)cfg->n_layers * (2 + 4);
  out->checkpoints = 4 * T * H * (cfg->n_layers + 1);
  const StepWs sw = carve_step(cfg, batch, seq, nullptr, step_flags);
  out->saved_activations = (uint64_t)sw.acts_bytes * sw.n_kept;
  out->step_workspace = sw.total - out->checkpoints - out->saved_activations;
  // token ids and the loss scalar; each of the step's buffers (slots, embedding,
  // head, final norm, adapters, gradients, workspace, ids, loss and a few more
  // of the caller's) may be rounded up by the allocator, at most 511 bytes each
  out->caller = 4 * T + 4 + 16 * 511;
  const uint64_t sum = out->slots + out->resident + out->adapters + out->checkpoints + out->saved_activations +
                       out->step_workspace + out->caller;
  out->margin = std::max<uint64_t>(sum / 100, 1ull << 20);
  out->total = sum + out->margin;
  return LSQ_OK;
}

int lsq_preflight(const lsq_model_cfg* cfg, int32_t batch, int32_t seq, int32_t n_buffers, int32_t step_flags,
                  uint64_t free_override, lsq_vram_breakdown* out) {
  lsq_vram_breakdown b{};
  if (int e = vram_predict_peak(cfg, batch, seq, n_buffers, step_flags, &b)) return e;
  if (out) *out = b;
  uint64_t free_b = free_override;
  if (!free_b) {
    size_t f = 0, t = 0;
    LSQ_HIP(hipMemGetInfo(&f, &t));
    free_b = f;
  }
  LSQ_CHECK(b.total <= free_b, LSQ_ERR_REFUSED,
            "a streaming step is predicted to need %.2f GB of VRAM but only %.2f GB is free (batch %d x seq %d; "
            "logits %.2f GB, checkpoints %.2f GB, kept activations %.2f GB, %d layer buffers %.2f GB)",
            b.total / 1e9, free_b / 1e9, batch, seq, 6.0 * batch * seq * cfg->vocab / 1e9, b.checkpoints / 1e9,
            b.saved_activations / 1e9, n_buffers, b.slots / 1e9);
  return LSQ_OK;
}

}  // extern "C"
