// Error reporting and the kernel-timing event pool.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"

namespace lsq {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

// ------------------------------------------------------------------ profiling
// A pool of pre-created hipEvent pairs; each bracketed launch takes one pair
// and remembers its family, flops and bytes.  Nothing is created on the hot
// path once the pool exists (lsq_prof_enable creates it).
namespace {
struct ProfRec {
  int kind;
  double flops, bytes;
};
constexpr int kPoolPairs = 1 << 17;
struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev;   // 2 per pair
  std::vector<ProfRec> rec;
  int used = 0;
  int dropped = 0;
} g_prof;
const char* kNames[PROF_N] = {"gemm_fwd_nf4_lora", "gemm_bwd_nf4_lora", "lora_skinny", "attention", "other",
                              "gemm_bf16_weights", "elementwise"};
}  // namespace

bool prof_on() { return g_prof.on; }

int prof_begin(hipStream_t s) {
  if (!g_prof.on) return -1;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (g_prof.used >= kPoolPairs) {
    ++g_prof.dropped;
    return -1;
  }
  int t = g_prof.used++;
  (void)hipEventRecord(g_prof.ev[2 * t], s);
  return t;
}

void prof_end(int token, hipStream_t s, ProfKind kind, double flops, double bytes) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  (void)hipEventRecord(g_prof.ev[2 * token + 1], s);
  g_prof.rec[token] = ProfRec{kind, flops, bytes};
}

int prof_begin_kernel(hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!g_prof.on) return -1;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (g_prof.used >= kPoolPairs) {
    ++g_prof.dropped;
    return -1;
  }
  const int t = g_prof.used++;
  *start = g_prof.ev[2 * t];
  *stop = g_prof.ev[2 * t + 1];
  return t;
}

void prof_end_kernel(int token, ProfKind kind, double flops, double bytes) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.rec[token] = ProfRec{kind, flops, bytes};
}

}  // namespace lsq

extern "C" {

const char* lsq_last_error(void) { return lsq::g_err; }

int32_t lsq_version(void) { return 1; }

int lsq_prof_enable(int32_t on) {
  using namespace lsq;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (on && g_prof.ev.empty()) {
    g_prof.ev.resize(2 * kPoolPairs);
    g_prof.rec.resize(kPoolPairs);
    for (auto& e : g_prof.ev) LSQ_HIP(hipEventCreate(&e));
  }
  g_prof.on = on != 0;
  g_prof.used = 0;
  g_prof.dropped = 0;
  return LSQ_OK;
}

int lsq_prof_read(lsq_prof_entry* out, int32_t max_entries, int32_t* n_entries) {
  using namespace lsq;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  LSQ_CHECK(out && n_entries && max_entries >= PROF_N, LSQ_ERR_INVALID, "lsq_prof_read: need %d entries", PROF_N);
  for (int k = 0; k < PROF_N; ++k) {
    memset(&out[k], 0, sizeof(lsq_prof_entry));
    snprintf(out[k].name, sizeof(out[k].name), "%s", kNames[k]);
  }
  for (int t = 0; t < g_prof.used; ++t) {
    LSQ_HIP(hipEventSynchronize(g_prof.ev[2 * t + 1]));
    float ms = 0.f;
    LSQ_HIP(hipEventElapsedTime(&ms, g_prof.ev[2 * t], g_prof.ev[2 * t + 1]));
    lsq_prof_entry& e = out[g_prof.rec[t].kind];
    e.launches += 1;
    e.ms += ms;
    e.flops += g_prof.rec[t].flops;
    e.bytes += g_prof.rec[t].bytes;
  }
  *n_entries = PROF_N;
  g_prof.used = 0;
  return g_prof.dropped ? lsq::fail(LSQ_ERR_STATE, "lsq_prof_read: %d launches not timed (pool full)", g_prof.dropped)
                        : LSQ_OK;
}

}  // extern "C"
