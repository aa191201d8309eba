// Optional per-kernel timing: while enabled, every kernel launch of the
// library is bracketed by a pair of HIP events on the launch stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkl {

enum KernelId : int32_t {
  KID_LOGITS_LSE = 0,
  KID_GATHER_DOT,
  KID_MERGE_LOSS,
  KID_REDUCE_LOSS,
  KID_BWD_PREP,
  KID_GPROD,
  KID_FIXUP,
  KID_GRAD_HIDDEN,
  KID_REDUCE_GH,
  KID_GRAD_W,
  KID_FILL,
  KID_VALIDATE,
  KID_G_FROM_Z,
  KID_TEACHER_LOGITS,
  KID_TOPK_THRESHOLD,
  KID_TOPK_COLLECT,
  KID_TOPK_FINAL,
  KID_MERGE_LSE,
  KID_RENORM_ROWS,
  KID_RENORM_GRAD_H,
  KID_RS_HIST,
  KID_RS_SCAN,
  KID_RS_PLACE,
  KID_RS_CHUNKS,
  KID_RS_FIX,
  KID_RS_HOT,
  KID_PAIR_INDEX,
  KID_RS_SLICES,
  KID_COUNT
};

const char* kernel_name(int32_t kid);

class ScopedTimer {
 public:
  ScopedTimer(int32_t kid, hipStream_t s);
  ~ScopedTimer();
  ScopedTimer(const ScopedTimer&) = delete;
  ScopedTimer& operator=(const ScopedTimer&) = delete;

 private:
  int32_t kid_;
  hipStream_t s_;
  hipEvent_t stop_ = nullptr;
  bool on_ = false;
};

bool timing_set(bool on);
void timing_reset();
// Waits for the recorded events and returns the totals for one kernel.
bool timing_read(int32_t kid, int64_t* launches, double* total_ms);

}  // namespace fkl
