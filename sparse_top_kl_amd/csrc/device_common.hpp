// Device helpers shared by the loss kernels (kernels.hip) and the teacher
// top-K kernels (topk.hip): exp2, the log-sum-exp partials of a logit tile
// and their merge, wave reductions, and the launch configuration of the
// MFMA tile kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm_core.hpp"
#include "kernels.hpp"

namespace fkl {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Register budget of the MFMA kernels: one workgroup per CU (LDS-bound), so
// kThreads / 256 waves per SIMD.
#define FKL_WAVES_PER_EU(C) __attribute__((amdgpu_waves_per_eu(C::kThreads / 256, C::kThreads / 256)))

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum of 2^(z * c2 - max) over the accumulator rows of token column
// ni that this lane holds (rows below vlim unless kAll). c2 > 0, so the max of
// z * c2 is c2 times the max of z, bit for bit.
template <class C, bool kAll>
__device__ __forceinline__ float2 lane_lse(const f32x16_t (&acc)[C::kMI][C::kNI], int ni, int lane,
                                           int vlim, float c2) {
  float mz = -INFINITY;
#pragma unroll
  for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kAll || acc_row(mi, r, lane) < vlim) mz = fmaxf(mz, acc[mi][ni][r]);
  const float m = mz * c2;
  float s = 0.f;
#pragma unroll
  for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kAll || acc_row(mi, r, lane) < vlim) s += fast_exp2(fmaf(acc[mi][ni][r], c2, -m));
  return make_float2(m, s);
}

// Per token of the wave's sub-tile: running max and sum of 2^(z * c2) over its
// 128 vocabulary rows v0.. (those below V), stored as the partial of slot
// v0 / 128. c2 > 0.
template <class C>
__device__ __forceinline__ void lse_partials(const f32x16_t (&acc)[C::kMI][C::kNI], int64_t v0,
                                             int64_t V, int64_t t0, int64_t nrows, float c2,
                                             float2* __restrict__ part, int64_t part_ld) {
  const int lane = threadIdx.x & 63;
  const int64_t slot = v0 / kSliceVocab;
  const bool full = v0 + C::kWM <= V;
  const int vlim = full ? C::kWM : static_cast<int>(V - v0);
#pragma unroll
  for (int ni = 0; ni < C::kNI; ++ni) {
    const float2 ms = full ? lane_lse<C, true>(acc, ni, lane, vlim, c2)
                           : lane_lse<C, false>(acc, ni, lane, vlim, c2);
    const float m = ms.x, s = ms.y;
    // the other lane half holds the other 4-row groups of the same token
    const float mo = __shfl_xor(m, 32);
    const float so = __shfl_xor(s, 32);
    const float M = fmaxf(m, mo);
    const float S = (s > 0.f ? s * fast_exp2(m - M) : 0.f) + (so > 0.f ? so * fast_exp2(mo - M) : 0.f);
    const int64_t tok = t0 + ni * 32 + (lane & 31);
    if (lane < 32 && tok < nrows) part[slot * part_ld + tok] = make_float2(M, S);
  }
}

__device__ __forceinline__ void merge_ms(float& m, float& s, float mo, float so) {
  if (so <= 0.f) return;
  if (s <= 0.f) {
    m = mo;
    s = so;
    return;
  }
  const float M = fmaxf(m, mo);
  s = s * fast_exp2(m - M) + so * fast_exp2(mo - M);
  m = M;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Merge of one row's partials (running max m, sum s of 2^(z*c - m)) into the
// natural-log log-sum-exp, by one wave.
__device__ __forceinline__ float merge_lse(const float2* __restrict__ part, int64_t part_ld,
                                           int64_t nslots, int64_t row) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY, s = 0.f;
  for (int64_t sl = lane; sl < nslots; sl += 64) {
    const float2 p = part[sl * part_ld + row];
    merge_ms(m, s, p.x, p.y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mo = __shfl_xor(m, o), so = __shfl_xor(s, o);
    merge_ms(m, s, mo, so);
  }
  return (m + log2f(s)) * kLn2;
}

template <int GA, int GB>
static inline unsigned grouped_grid(int64_t mt, int64_t nt) {
  return static_cast<unsigned>(TileGroups<GA, GB>::grid(mt, nt));
}

typedef TileCfg<2, 2> Cfg4;  // 4 waves, 128x128 per wave (fp32, register-staged loop)
typedef TileCfg<2, 4> Cfg8;  // 8 waves, 128x64 per wave (bf16, ping-pong loop)

#define FKL_LAUNCH_GEMM(KERNEL, dtype, grid, s, ...)                                    \
  do {                                                                                  \
    if ((dtype) == 1)                                                                   \
      KERNEL<BF16, Cfg8><<<(grid), Cfg8::kThreads, 0, (s)>>>(__VA_ARGS__);              \
    else                                                                                \
      KERNEL<F32, Cfg4><<<(grid), Cfg4::kThreads, 0, (s)>>>(__VA_ARGS__);               \
  } while (0)

}  // namespace fkl
