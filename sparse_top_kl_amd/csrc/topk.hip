// Teacher top-K cache kernels for gfx950 (see the section comment below).
#include <math.h>

#include "device_common.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace fkl {

// ------------------------------------------------------------ teacher top-K
//
// The offline teacher cache ("Эффективная дистилляция знаний ..."
// (malakhovai.ru), second paragraph; "Wissensdestillation mit deutlich
// weniger GPU-Speicher", section "Teacher-Ausgaben einmalig
// zwischenspeichern"): per token the K largest teacher logits with their ids,
// ordered by value, ties to the lower id. Per chunk of tokens:
//   k_teacher_logits   logit tile (MFMA, the loss's tile code) -> the chunk's
//                      fp32 logits stored [vocab][token], and per (token,
//                      128-vocab slice) the largest logit;
//   k_topk_threshold   per token the K-th largest slice maximum: at least K
//                      logits are >= it, so every top-K logit is;
//   k_topk_collect     one pass over the stored logits, keeping (value, id)
//                      keys >= the threshold in a per-token list;
//   k_topk_final       per token, sort the list and write the K best; a list
//                      that overflowed (mass ties) is redone exactly by a
//                      radix select over the token's stored logits.
// Keys: the fp32 value mapped to an order-preserving uint32 (-0 as +0) in the
// high word, the complement of the id in the low word, so a larger key is a
// larger value or, among equal values, a lower id. Logits must be finite.

__device__ __forceinline__ uint32_t ord_f32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint64_t topk_key(uint32_t ord, int64_t id) {
  return (static_cast<uint64_t>(ord) << 32) | (0xffffffffu - static_cast<uint32_t>(id));
}

// With LSE the tile also leaves its per-(128-vocab slice, token) log-sum-exp
// partials at temperature 1/(c2 ln 2) in part (the teacher's lse for the tail
// bucket of the loss).
template <class P, class C, bool LSE>
__global__ __launch_bounds__(C::kThreads) FKL_WAVES_PER_EU(C) void k_teacher_logits(
    const unsigned char* __restrict__ W, const unsigned char* __restrict__ H, int64_t d, int64_t V,
    int64_t nrows, int64_t n_vt, int64_t n_tt, float* __restrict__ LT, int64_t lt_ld,
    uint32_t* __restrict__ smax, int64_t sm_ld, float c2, float2* __restrict__ part) {
  static_assert(C::kWM == kSliceVocab, "one slice maximum per wave row-slice");
  int64_t vt, tt;
  if (!TileGroups<4, 8>::coords(n_vt, n_tt, &vt, &tt)) return;
  const int64_t ld = d * P::kBytes;
  const Operand A = make_operand(W + vt * kBM * ld, ld, V - vt * kBM, d);
  const Operand B = make_operand(H + tt * kBN * ld, ld, nrows - tt * kBN, d);
  f32x16_t acc[C::kMI][C::kNI];
  gemm_tile<P, C, false, false>(acc, A, B, static_cast<int>(d));

  // A lane holds one token's logits for 64 vocabulary rows; for a fixed
  // accumulator element the 32 lanes of a half-wave hold 32 consecutive
  // tokens of one vocabulary row, so [vocab][token] stores are 128-byte rows.
  const int lane = threadIdx.x & 63;
  const int64_t v0 = vt * kBM + C::wave_m() * C::kWM;
  if (v0 >= V) return;
  if constexpr (LSE)
    lse_partials<C>(acc, v0, V, tt * kBN + C::wave_n() * C::kWN, nrows, c2, part, lt_ld);
  const int64_t slot = v0 / kSliceVocab;
  const bool full = v0 + C::kWM <= V;
  const int vlim = full ? C::kWM : static_cast<int>(V - v0);
#pragma unroll
  for (int ni = 0; ni < C::kNI; ++ni) {
    const int64_t tok = tt * kBN + C::wave_n() * C::kWN + ni * 32 + (lane & 31);
    const bool tok_ok = tok < nrows;
    uint32_t best = 0;
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vr = acc_row(mi, r, lane);
        if (full || vr < vlim) {
          const float x = acc[mi][ni][r];
          if (tok_ok) __builtin_nontemporal_store(x, LT + (v0 + vr) * lt_ld + tok);
          best = max(best, ord_f32(x));
        }
      }
    best = max(best, static_cast<uint32_t>(__shfl_xor(static_cast<int>(best), 32)));
    if (lane < 32 && tok_ok) smax[tok * sm_ld + slot] = best;
  }
}

// Digit of the k-th largest key (k >= 1) from a 256-bin histogram in LDS,
// scanned from the top by one wave: returns the digit and, in *above, how
// many keys fall in higher bins.
__device__ __forceinline__ int hist_select(const uint32_t* hist, uint32_t k, uint32_t* above) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = hist[255 - 4 * lane - j];
    local += c[j];
  }
  uint32_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), o));
    if (lane >= o) incl += y;
  }
  const uint32_t excl = incl - local;
  const bool mine = excl < k && k <= incl;
  int digit = 0;
  uint32_t ab = 0;
  if (mine) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (acc + c[j] >= k) {
        digit = 255 - 4 * lane - j;
        ab = acc;
        break;
      }
      acc += c[j];
    }
  }
  const int owner = __ffsll(static_cast<unsigned long long>(__ballot(mine))) - 1;
  *above = static_cast<uint32_t>(__shfl(static_cast<int>(ab), owner));
  return __shfl(digit, owner);
}

// One 64-thread workgroup per token: theta = the K-th largest of the token's
// nslots slice maxima (radix select, 8 bits per pass), or 0 (every logit
// qualifies) when there are fewer than K slices.
__global__ __launch_bounds__(64) void k_topk_threshold(const uint32_t* __restrict__ smax,
                                                       int64_t sm_ld, int64_t nslots, int K,
                                                       uint32_t* __restrict__ theta) {
  __shared__ uint32_t hist[256];
  const int lane = threadIdx.x;
  const int64_t tok = blockIdx.x;
  if (nslots < K) {
    if (lane == 0) theta[tok] = 0u;
    return;
  }
  const uint32_t* p = smax + tok * sm_ld;
  uint32_t prefix = 0, mask = 0, rem = static_cast<uint32_t>(K);
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[lane + 64 * j] = 0;
    __syncthreads();
    for (int64_t i = lane; i < nslots; i += 64) {
      const uint32_t x = p[i];
      if ((x & mask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint32_t above;
    const int digit = hist_select(hist, rem, &above);
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= 255u << shift;
    rem -= above;
    __syncthreads();
  }
  if (lane == 0) theta[tok] = prefix;
}

// Grid (token blocks of 256, vocabulary ranges): lane l of wave w reads
// tokens t0 + 4l .. t0 + 4l + 3 of vocabulary rows begin + w, begin + w + 4,
// ..., so each wave load is one 1 KiB row segment of the stored logits
// (streaming loads: every value is read once). Keys at or above the token's
// threshold are appended to its list (the count may pass the capacity: the
// final kernel then takes the exact path).
constexpr int kCollectTokens = 256;
__global__ __launch_bounds__(256) void k_topk_collect(const float* __restrict__ LT, int64_t lt_ld,
                                                      int64_t V, int64_t nrows, int64_t vrange,
                                                      const uint32_t* __restrict__ theta,
                                                      uint64_t* __restrict__ cand, int cap,
                                                      uint32_t* __restrict__ count) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kCollectTokens + 4 * lane;
  if (tok0 >= nrows) return;
  const int64_t vb = static_cast<int64_t>(blockIdx.y) * vrange;
  const int64_t ve = vb + vrange < V ? vb + vrange : V;
  uint32_t th[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) th[j] = tok0 + j < nrows ? theta[tok0 + j] : 0xffffffffu;
  constexpr int kU = 2;  // 16-byte loads in flight per thread (2, 4, 8 measured alike)
  for (int64_t v = vb + w; v < ve; v += 4 * kU) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    f32x4_t x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t vv = v + 4 * u;
      x[u] = vv < ve ? __builtin_nontemporal_load(
                           reinterpret_cast<const f32x4_t*>(LT + vv * lt_ld + tok0))
                     : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t vv = v + 4 * u;
      const float xs[4] = {x[u][0], x[u][1], x[u][2], x[u][3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t o = ord_f32(xs[j]);
        if (vv < ve && o >= th[j] && th[j] != 0xffffffffu) {
          const uint32_t pos = atomicAdd(&count[tok0 + j], 1u);
          if (pos < static_cast<uint32_t>(cap)) cand[(tok0 + j) * cap + pos] = topk_key(o, vv);
        }
      }
    }
  }
}

// One wave per row: the natural-log log-sum-exp from its slice partials.
__global__ __launch_bounds__(256) void k_merge_lse_rows(const float2* __restrict__ part,
                                                        int64_t part_ld, int64_t nslots,
                                                        int64_t nrows, float* __restrict__ out) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const float lse = merge_lse(part, part_ld, nslots, row);
  if ((threadIdx.x & 63) == 0) out[row] = lse;
}

constexpr int kTopkCap = 2048;  // candidate keys per token (LDS of the final kernel)

// Sorts keys[0, P) descending (P a power of two) with the whole workgroup.
__device__ __forceinline__ void bitonic_desc(uint64_t* keys, int P) {
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P / 2; i += blockDim.x) {
        const int lo = ((i & ~(stride - 1)) << 1) | (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) != 0;  // this run ends ascending (merged later)
        const uint64_t a = keys[lo], b = keys[hi];
        if (up ? (a > b) : (a < b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
}

// One 256-thread workgroup per token: the K best keys of its list, sorted, or
// (list overflowed) an exact radix select over the token's stored logits.
__global__ __launch_bounds__(256) void k_topk_final(const uint64_t* __restrict__ cand,
                                                    const uint32_t* __restrict__ count, int cap,
                                                    const float* __restrict__ LT, int64_t lt_ld,
                                                    int64_t V, int K, int32_t* __restrict__ out_idx,
                                                    float* __restrict__ out_val) {
  __shared__ uint64_t keys[kTopkCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  const int t = threadIdx.x;
  const int64_t tok = blockIdx.x;
  const uint32_t n = count[tok];
  int m;  // keys to sort
  if (n <= static_cast<uint32_t>(cap)) {
    m = static_cast<int>(n);
    for (int i = t; i < m; i += 256) keys[i] = cand[tok * cap + i];
  } else {
    // exact path: the K-th largest key over all V logits of the token
    uint64_t prefix = 0, mask = 0;
    uint32_t rem = static_cast<uint32_t>(K);
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[t] = 0;
      __syncthreads();
      for (int64_t v = t; v < V; v += 256) {
        const uint64_t key = topk_key(ord_f32(LT[v * lt_ld + tok]), v);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (t < 64) {
        uint32_t above;
        const int digit = hist_select(hist, rem, &above);
        if (t == 0) {
          sh[0] = static_cast<uint32_t>(digit);
          sh[1] = above;
        }
      }
      __syncthreads();
      prefix |= static_cast<uint64_t>(sh[0]) << shift;
      mask |= static_cast<uint64_t>(255u) << shift;
      rem -= sh[1];
      __syncthreads();
    }
    if (t == 0) sh[0] = 0;
    __syncthreads();
    for (int64_t v = t; v < V; v += 256) {  // exactly K keys are >= the K-th largest
      const uint64_t key = topk_key(ord_f32(LT[v * lt_ld + tok]), v);
      if (key >= prefix) {
        const uint32_t pos = atomicAdd(&sh[0], 1u);
        if (pos < static_cast<uint32_t>(kTopkCap)) keys[pos] = key;
      }
    }
    m = K;
  }
  int P = 2;
  while (P < m || P < K) P <<= 1;
  __syncthreads();
  for (int i = m + t; i < P; i += 256) keys[i] = 0;  // below every real key
  __syncthreads();
  bitonic_desc(keys, P);
  for (int k = t; k < K; k += 256) {
    const uint64_t key = keys[k];
    out_idx[tok * K + k] = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(key));
    out_val[tok * K + k] = unord_f32(static_cast<uint32_t>(key >> 32));
  }
}

// ------------------------------------------------------------------ launchers

void launch_teacher_logits(int dtype, const void* W, const void* H, int64_t d, int64_t V,
                           int64_t row0, int64_t nrows, float* LT, int64_t lt_ld,
                           uint32_t* smax, int64_t sm_ld, float c2, float2* part,
                           hipStream_t s) {
  ScopedTimer timer_(KID_TEACHER_LOGITS, s);
  const int64_t eb = dtype == 1 ? 2 : 4;
  const int64_t n_vt = ceil_div(V, kBM), n_tt = ceil_div(nrows, kBN);
  const unsigned char* Hc = static_cast<const unsigned char*>(H) + row0 * d * eb;
  const unsigned char* Wc = static_cast<const unsigned char*>(W);
  const unsigned grid = grouped_grid<4, 8>(n_vt, n_tt);
#define FKL_TEACHER(LSE)                                                                          \
  do {                                                                                            \
    if (dtype == 1)                                                                               \
      k_teacher_logits<BF16, Cfg8, LSE><<<grid, Cfg8::kThreads, 0, s>>>(                          \
          Wc, Hc, d, V, nrows, n_vt, n_tt, LT, lt_ld, smax, sm_ld, c2, part);                     \
    else                                                                                          \
      k_teacher_logits<F32, Cfg4, LSE><<<grid, Cfg4::kThreads, 0, s>>>(                           \
          Wc, Hc, d, V, nrows, n_vt, n_tt, LT, lt_ld, smax, sm_ld, c2, part);                     \
  } while (0)
  if (part)
    FKL_TEACHER(true);
  else
    FKL_TEACHER(false);
#undef FKL_TEACHER
}

void launch_topk_select(const float* LT, int64_t lt_ld, int64_t V, const uint32_t* smax,
                        int64_t sm_ld, int64_t nslots, int64_t nrows, int K, uint32_t* theta,
                        uint64_t* cand, uint32_t* count, int32_t* out_idx, float* out_val,
                        hipStream_t s) {
  if (nrows <= 0) return;
  {
    ScopedTimer timer_(KID_TOPK_THRESHOLD, s);
    k_topk_threshold<<<static_cast<unsigned>(nrows), 64, 0, s>>>(smax, sm_ld, nslots, K, theta);
  }
  {
    // counts start at zero (a fill kernel, not a memset node, so graph capture stays safe)
    launch_fill_f32(reinterpret_cast<float*>(count), nrows, 0.0f, s);
    ScopedTimer timer_(KID_TOPK_COLLECT, s);
    const int64_t tb = ceil_div(nrows, kCollectTokens);
    int64_t ranges = ceil_div(2048, tb);  // about 2048 workgroups
    if (ranges < 1) ranges = 1;
    if (ranges > ceil_div(V, 64)) ranges = ceil_div(V, 64);
    const int64_t vrange = ceil_div(V, ranges);
    k_topk_collect<<<dim3(static_cast<unsigned>(tb), static_cast<unsigned>(ceil_div(V, vrange))),
                     256, 0, s>>>(LT, lt_ld, V, nrows, vrange, theta, cand, kTopkCap, count);
  }
  {
    ScopedTimer timer_(KID_TOPK_FINAL, s);
    k_topk_final<<<static_cast<unsigned>(nrows), 256, 0, s>>>(cand, count, kTopkCap, LT, lt_ld, V,
                                                             K, out_idx, out_val);
  }
}

int topk_capacity() { return kTopkCap; }

void launch_merge_lse_rows(const float2* part, int64_t part_ld, int64_t nslots, int64_t nrows,
                           float* out, hipStream_t s) {
  if (nrows <= 0) return;
  ScopedTimer timer_(KID_MERGE_LSE, s);
  k_merge_lse_rows<<<static_cast<unsigned>(ceil_div(nrows, 4)), 256, 0, s>>>(part, part_ld, nslots,
                                                                            nrows, out);
}

}  // namespace fkl
