// Host helpers shared by the C ABI sources (fkl_api.cpp, topk_api.cpp): the
// per-thread error message, alignment checks, the common shape checks and
// the check of the last HIP launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "fkl.h"
#include "kernels.hpp"

namespace fkl_api {

// Message of the last failed call on this thread (fkl_last_error).
extern thread_local char g_last_error[512];

inline int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Largest offset a buffer load may reach: 2 GiB less a margin.
constexpr int64_t kMaxBlockBytes = (int64_t(1) << 31) - (int64_t(1) << 20);

inline int32_t check_shapes(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int32_t dtype) {
  if (dtype != FKL_F32 && dtype != FKL_BF16) return fail(FKL_E_UNSUPPORTED, "unknown dtype %d", dtype);
  if (N < 0) return fail(FKL_E_ARG, "N must be >= 0 (got %lld)", (long long)N);
  if (d < 8) return fail(FKL_E_ARG, "d must be >= 8 (got %lld)", (long long)d);
  if (d % 8 != 0) return fail(FKL_E_UNSUPPORTED, "d must be a multiple of 8 (got %lld)", (long long)d);
  if (V < 1) return fail(FKL_E_ARG, "V must be >= 1 (got %lld)", (long long)V);
  if (V >= (int64_t(1) << 31)) return fail(FKL_E_ARG, "V must fit in int32");
  if (K < 1 || K > V) return fail(FKL_E_ARG, "K must be in [1, V] (got %d)", K);
  if (K > 4096) return fail(FKL_E_UNSUPPORTED, "K > 4096 is not supported (got %d)", K);
  if (chunk < 1) return fail(FKL_E_ARG, "chunk must be >= 1 (got %lld)", (long long)chunk);
  const int64_t eb = dtype == FKL_BF16 ? 2 : 4;
  if (V * d * eb > kMaxBlockBytes)
    return fail(FKL_E_UNSUPPORTED, "weight larger than 2 GiB is not supported");
  return FKL_OK;
}

inline int32_t hip_check(const char* where) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FKL_E_HIP, "%s: %s", where, hipGetErrorString(e));
  return FKL_OK;
}

// Runs the device-side id check (teacher ids in [0, V), labels below V) and
// waits for its verdict.
inline int32_t validate_ids(const int32_t* idx, int64_t N, int32_t K, int64_t V, int32_t* dflag,
                     hipStream_t s, const int32_t* labels = nullptr) {
  fkl::launch_fill_f32(reinterpret_cast<float*>(dflag), 1, 0.0f, s);
  fkl::launch_validate_idx(idx, N, K, V, false, dflag, s);
  if (labels) fkl::launch_validate_idx(labels, N, 1, V, true, dflag, s);
  int32_t r = hip_check("id validation launch");
  if (r) return r;
  int32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, dflag, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(FKL_E_HIP, "id validation: %s", hipGetErrorString(e));
  if (host != 0) return fail(FKL_E_INDEX, "a teacher id is outside [0, V) or a label >= V");
  return FKL_OK;
}

}  // namespace fkl_api
