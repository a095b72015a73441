// Opt-in per-launch timing with hipEvents. Disabled by default; when enabled every kernel the
// library enqueues is bracketed by an event pair on the caller's stream, and
// lce_timing_read() waits for the recorded pairs and returns per-kernel totals.
#include <mutex>
#include <vector>

#include "common.h"
#include "lce_masked.h"

namespace lce {
namespace {

struct Pending {
  int id;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
hipEvent_t g_open[K_COUNT];  // start event of the launch currently being bracketed
double g_ms[K_COUNT];
long long g_launches[K_COUNT];

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

const char* kNames[K_COUNT] = {
    "label_prep",         "ce_fwd_rows",           "loss_reduce",
    "ce_bwd_rows",        "flce_gemm_logits",      "flce_row_lse",
    "flce_bias_grad",     "flce_to_probs",         "flce_gemm_grad_hidden",
    "flce_gemm_grad_weight", "flce_onehot_fix",    "fill_zero",
    "flce_grad_hidden_reduce", "flce_gemm_probs", "flce_label_sort",
    "ce_fused_rows",      "flce_loss_acc",         "flce_probs_transposed",
};

}  // namespace

const char* kernel_name(int id) { return (id >= 0 && id < K_COUNT) ? kNames[id] : "?"; }

bool timing_on() { return g_on; }

void timing_start(hipStream_t stream, int id) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, stream) != hipSuccess) {  // this launch goes untimed
    g_free.push_back(e);
    return;
  }
  g_open[id] = e;
}

void timing_stop(hipStream_t stream, int id) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t s = g_open[id];
  if (!s) return;
  g_open[id] = nullptr;
  hipEvent_t e = take_event();
  if (!e) {
    g_free.push_back(s);
    return;
  }
  if (hipEventRecord(e, stream) != hipSuccess) {  // this launch goes untimed
    g_free.push_back(s);
    g_free.push_back(e);
    return;
  }
  g_pending.push_back(Pending{id, s, e});
}

}  // namespace lce

extern "C" {

int lce_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(lce::g_mu);
  lce::g_on = enable != 0;
  return LCE_OK;
}

int lce_timing_read(int max_kernels, const char** names, double* total_ms, long long* launches,
                    int* count_out) {
  if (!count_out || (max_kernels > 0 && (!names || !total_ms || !launches))) return LCE_ERR_NULL_ARG;
  std::lock_guard<std::mutex> lk(lce::g_mu);
  int rc = LCE_OK;
  for (auto& p : lce::g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      rc = LCE_ERR_HIP;
    } else {
      lce::g_ms[p.id] += ms;
      lce::g_launches[p.id] += 1;
    }
    lce::g_free.push_back(p.start);
    lce::g_free.push_back(p.stop);
  }
  lce::g_pending.clear();
  int k = 0;
  for (int id = 0; id < lce::K_COUNT; ++id) {
    if (lce::g_launches[id] == 0) continue;
    if (k < max_kernels) {
      names[k] = lce::kNames[id];
      total_ms[k] = lce::g_ms[id];
      launches[k] = lce::g_launches[id];
    }
    ++k;
    lce::g_ms[id] = 0.0;
    lce::g_launches[id] = 0;
  }
  *count_out = k;
  return rc;
}

}  // extern "C"
