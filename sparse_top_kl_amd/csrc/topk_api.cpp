// C ABI of the teacher top-K cache producer: argument validation, workspace
// planning and the chunk loop. Declarations, argument meanings, layouts and
// error behaviour are in include/fkl.h.
#include <hip/hip_runtime.h>

#include <cmath>

#include "api_common.hpp"
#include "fkl.h"
#include "kernels.hpp"

using namespace fkl_api;

namespace {

// Workspace of fkl_teacher_topk: one chunk's fp32 logits [V][lt_ld], slice
// maxima [chunk][sm_ld], thresholds, candidate lists and their counts.
struct TopkPlan {
  int64_t chunk_cap, lt_ld, nslots, sm_ld;
  size_t lt, smax, theta, count, cand, part, total;
};

TopkPlan make_topk_plan(int64_t N, int64_t V, int64_t chunk) {
  TopkPlan q{};
  q.chunk_cap = chunk < N ? chunk : N;
  if (q.chunk_cap < 1) q.chunk_cap = 1;
  q.lt_ld = fkl::round_up(q.chunk_cap, 64);
  q.nslots = fkl::ceil_div(V, fkl::kSliceVocab);
  q.sm_ld = fkl::round_up(q.nslots, 4);
  const size_t rows = static_cast<size_t>(q.chunk_cap);
  size_t off = 0;
  q.lt = off;
  off = align_up(off + static_cast<size_t>(V) * q.lt_ld * 4);
  q.smax = off;
  off = align_up(off + rows * q.sm_ld * 4);
  q.theta = off;
  off = align_up(off + rows * 4);
  q.count = off;
  off = align_up(off + rows * 4);
  q.cand = off;
  off = align_up(off + rows * fkl::topk_capacity() * 8);
  q.part = off;  // teacher LSE partials [slot][lt_ld] (optional output)
  off = align_up(off + static_cast<size_t>(fkl::lse_slots(V)) * q.lt_ld * 8);
  q.total = off;
  return q;
}

int32_t check_topk(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int32_t dtype) {
  int32_t r = check_shapes(N, d, V, 1, chunk, dtype);
  if (r) return r;
  if (K < 1 || K > V) return fail(FKL_E_ARG, "K must be in [1, V] (got %d)", K);
  if (K > 1024) return fail(FKL_E_UNSUPPORTED, "K > 1024 is not supported (got %d)", K);
  return FKL_OK;
}

}  // namespace

extern "C" int32_t fkl_topk_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                                int32_t dtype, size_t* bytes) {
  g_last_error[0] = 0;
  const int32_t r = check_topk(N, d, V, K, chunk, dtype);
  if (r) return r;
  if (bytes) *bytes = make_topk_plan(N, V, chunk).total;
  return FKL_OK;
}

static int32_t teacher_topk_impl(const void* hidden, const void* weight, int64_t N, int64_t d,
                                 int64_t V, int32_t K, int64_t chunk, int32_t dtype,
                                 uint32_t flags, float T, int32_t* topk_idx, float* topk_logit,
                                 float* teacher_lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  int32_t r = check_topk(N, d, V, K, chunk, dtype);
  if (r) return r;
  if (teacher_lse && (!std::isfinite(T) || !(T > 0.0f)))
    return fail(FKL_E_ARG, "T must be finite and > 0");
  if (!aligned(teacher_lse, 4)) return fail(FKL_E_ARG, "teacher_lse must be 4-byte aligned");
  if (flags != 0) return fail(FKL_E_ARG, "unknown flag bits");
  if (!weight || !workspace) return fail(FKL_E_ARG, "null pointer argument");
  if (N > 0 && (!hidden || !topk_idx || !topk_logit))
    return fail(FKL_E_ARG, "null pointer argument");
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16))
    return fail(FKL_E_ARG, "hidden, weight and workspace must be 16-byte aligned");
  if (!aligned(topk_idx, 4) || !aligned(topk_logit, 4))
    return fail(FKL_E_ARG, "topk_idx and topk_logit must be 4-byte aligned");
  const TopkPlan q = make_topk_plan(N, V, chunk);
  if (workspace_bytes < q.total)
    return fail(FKL_E_WORKSPACE, "top-K workspace needs %zu bytes, got %zu", q.total,
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  (void)hipGetLastError();
  if (N == 0) return FKL_OK;
  float* LT = reinterpret_cast<float*>(ws + q.lt);
  uint32_t* smax = reinterpret_cast<uint32_t*>(ws + q.smax);
  uint32_t* theta = reinterpret_cast<uint32_t*>(ws + q.theta);
  uint32_t* count = reinterpret_cast<uint32_t*>(ws + q.count);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + q.cand);
  float2* part = teacher_lse ? reinterpret_cast<float2*>(ws + q.part) : nullptr;
  const float c2 = teacher_lse ? 1.4426950408889634f / T : 0.0f;
  for (int64_t row0 = 0; row0 < N; row0 += q.chunk_cap) {
    const int64_t nrows = (N - row0) < q.chunk_cap ? (N - row0) : q.chunk_cap;
    fkl::launch_teacher_logits(dtype, weight, hidden, d, V, row0, nrows, LT, q.lt_ld, smax, q.sm_ld,
                               c2, part, s);
    fkl::launch_topk_select(LT, q.lt_ld, V, smax, q.sm_ld, q.nslots, nrows, K, theta, cand, count,
                            topk_idx + row0 * K, topk_logit + row0 * K, s);
    if (teacher_lse)
      fkl::launch_merge_lse_rows(part, q.lt_ld, q.nslots, nrows, teacher_lse + row0, s);
  }
  return hip_check("teacher top-K launch");
}

extern "C" int32_t fkl_teacher_topk(const void* hidden, const void* weight, int64_t N, int64_t d, int64_t V,
                         int32_t K, int64_t chunk, int32_t dtype, uint32_t flags,
                         int32_t* topk_idx, float* topk_logit, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return teacher_topk_impl(hidden, weight, N, d, V, K, chunk, dtype, flags, 1.0f, topk_idx,
                           topk_logit, nullptr, workspace, workspace_bytes, stream);
}

extern "C" int32_t fkl_teacher_topk_ex(const void* hidden, const void* weight, int64_t N, int64_t d,
                            int64_t V, int32_t K, int64_t chunk, int32_t dtype, uint32_t flags,
                            float T, int32_t* topk_idx, float* topk_logit, float* teacher_lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return teacher_topk_impl(hidden, weight, N, d, V, K, chunk, dtype, flags, T, topk_idx,
                           topk_logit, teacher_lse, workspace, workspace_bytes, stream);
}
