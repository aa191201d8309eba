// Per-kernel HIP-event timing (profiling aid, off by default).
#include "timing.hpp"

#include <atomic>
#include <mutex>
#include <vector>

namespace fkl {

namespace {

struct Pending {
  int32_t kid;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
int64_t g_launches[KID_COUNT] = {};
double g_ms[KID_COUNT] = {};

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

// Folds finished event pairs into the totals (caller holds g_mu).
void drain_locked() {
  for (const Pending& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      g_launches[p.kid] += 1;
      g_ms[p.kid] += ms;
    }
    g_free.push_back(p.start);
    g_free.push_back(p.stop);
  }
  g_pending.clear();
}

}  // namespace

const char* kernel_name(int32_t kid) {
  static const char* names[KID_COUNT] = {
      "k_logits_lse", "k_gather_dot", "k_merge_loss", "k_reduce_loss",
      "k_bwd_prep",   "k_gprod",      "k_fixup",      "k_grad_hidden",
      "k_reduce_gh",  "k_grad_w",     "k_fill_f32",   "k_validate_idx",
      "k_g_from_z",   "k_teacher_logits", "k_topk_threshold", "k_topk_collect",
      "k_topk_final", "k_merge_lse_rows", "k_renorm_rows", "k_renorm_grad_h",
      "k_rs_hist",    "k_rs_scan",    "k_rs_place",   "k_rs_chunks",
      "k_rs_fix",     "k_rs_hot",     "k_pair_index", "k_rs_slices"};
  return (kid >= 0 && kid < KID_COUNT) ? names[kid] : nullptr;
}

ScopedTimer::ScopedTimer(int32_t kid, hipStream_t s) : kid_(kid), s_(s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t start = take_event();
  stop_ = take_event();
  if (!start || !stop_) return;
  if (hipEventRecord(start, s_) != hipSuccess) return;
  g_pending.push_back({kid_, start, stop_});
  on_ = true;
}

ScopedTimer::~ScopedTimer() {
  if (on_) (void)hipEventRecord(stop_, s_);
}

bool timing_set(bool on) { return g_on.exchange(on); }

void timing_reset() {
  std::lock_guard<std::mutex> lk(g_mu);
  drain_locked();
  for (int i = 0; i < KID_COUNT; ++i) {
    g_launches[i] = 0;
    g_ms[i] = 0.0;
  }
}

bool timing_read(int32_t kid, int64_t* launches, double* total_ms) {
  if (kid < 0 || kid >= KID_COUNT) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  drain_locked();
  if (launches) *launches = g_launches[kid];
  if (total_ms) *total_ms = g_ms[kid];
  return true;
}

}  // namespace fkl
