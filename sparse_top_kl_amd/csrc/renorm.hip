// Student-renormalised top-K loss for gfx950: both distributions softened by T
// and renormalised over the K cached entries of each row, so the loss reads
// the student's logits at the cached ids only (no vocabulary-wide log-sum-exp
// and no vocabulary GEMM). The pages leave open how the tail beyond the cache
// is treated ("Multiverse Computing ... (iitak.ru)", third paragraph, and
// "Wissensdestillation mit deutlich weniger GPU-Speicher", section
// "Teacher-Ausgaben einmalig zwischenspeichern", describe the cache; the
// softening and the T^2 factor follow "Дистилляция и сжатие моделей",
// section "Как это работает: мягкие метки и температура").
//
// Per row r (entries with a -inf teacher logit are padding and take part in
// neither softmax), in base-2 units with c2 = log2(e) / T:
//   p_k = 2^(l_k c2 - la),  q_k = 2^(z_k c2 - lu)   (la, lu the log2 normalisers)
//   row_loss = w_r T^2 ln2 sum_k p_k (log2 p_k - log2 q_k)
//   G_rk     = s w_r T (q_k sum_j p_j - p_k)
//   grad_h_r = sum_k G_rk W[idx_rk],  grad_W[v] = sum_{(r,k): idx_rk = v} G_rk h_r
//
// Kernels:
//   k_renorm_rows    one wave per row: the two K-entry softmaxes -> row loss
//                    (forward) or the K coefficients G_r. (backward)
//   k_renorm_grad_h  one workgroup per row: sum_k G_rk W[idx_rk] (16-byte
//                    loads of the K weight rows, eight in flight per lane)
//   grad_W without float atomics, bitwise deterministic:
//   k_rs_hist        per block of rows, the count of each id (integer atomics)
//   k_rs_colscan     per id, exclusive prefix of its counts over the blocks
//   k_rs_hot         picks the frequent ("hot") ids: count >= tau, tau the
//                    smallest power of two >= kRenormHotMin that leaves at
//                    most hot_max of them (as many as one round of 256 x 256
//                    product tiles takes); gives each a slot, and the
//                    exclusive prefix over the other ("cold") ids of their
//                    counts: bucket starts of the cold pairs
//   hot ids, a dense product: k_rs_hot_coef scatters each row's hot
//   coefficients into C [rows x hot_max] (copies of one id in a row
//   summed in entry order), k_grad_w (the loss's MFMA kernel, its rows split
//   over the XCDs its tiles alone would leave idle) forms C^T H, and
//   k_rs_hot_rows sums the splits in order into each hot id's grad_W row
//   cold ids, a sort:
//   k_rs_place       per block, its rows in order: each cold pair (r, k) goes
//                    to start[v] + (pairs of id v in earlier rows) + (copies of
//                    v earlier in row r): a stable counting sort by id
//   k_rs_chunks      fixed chunks of the sorted pairs: the sum of G h over each
//                    run of one id, written to grad_W when the chunk holds the
//                    whole bucket, else to the chunk's head or tail partial
//   k_rs_fix         per cold id whose bucket crosses chunks: its partials in
//                    chunk order; ids with no pair get a zero row
#include <math.h>

#include "device_common.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace fkl {

namespace {

__device__ __forceinline__ bool finite_logit(float l) { return l > -INFINITY && l < INFINITY; }

// Eight consecutive values from a bf16 (16 bytes) or fp32 (32 bytes) row.
template <class P>
__device__ __forceinline__ void load8(const unsigned char* p, float (&x)[8]) {
  if constexpr (P::kBytes == 2) {
    const u32x4_t u = load16(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = as_f32(u[e] << 16);
      x[2 * e + 1] = as_f32(u[e] & 0xffff0000u);
    }
  } else {
    const u32x4_t a = load16(p), b = load16(p + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = as_f32(a[e]);
      x[4 + e] = as_f32(b[e]);
    }
  }
}

template <class P>
__device__ __forceinline__ void store8(unsigned char* p, const float (&x)[8]) {
  if constexpr (P::kBytes == 2) {
    *reinterpret_cast<u32x4_t*>(p) = u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                             pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
  } else {
    *reinterpret_cast<u32x4_t*>(p) = u32x4_t{__builtin_bit_cast(uint32_t, x[0]),
                                             __builtin_bit_cast(uint32_t, x[1]),
                                             __builtin_bit_cast(uint32_t, x[2]),
                                             __builtin_bit_cast(uint32_t, x[3])};
    *reinterpret_cast<u32x4_t*>(p + 16) = u32x4_t{__builtin_bit_cast(uint32_t, x[4]),
                                                  __builtin_bit_cast(uint32_t, x[5]),
                                                  __builtin_bit_cast(uint32_t, x[6]),
                                                  __builtin_bit_cast(uint32_t, x[7])};
  }
}

constexpr int kRowWaves = 4;  // rows per k_renorm_rows block

}  // namespace

template <bool COEF>
__global__ __launch_bounds__(64 * kRowWaves) void k_renorm_rows(
    const float* __restrict__ zk, const float* __restrict__ logit,
    const float* __restrict__ row_weight, const float* __restrict__ grad_loss, int64_t N, int K,
    float T, float* __restrict__ row_loss, float* __restrict__ coef) {
  // l c2 and z c2 must be rounded products, not fused into the following
  // subtraction, so that an entry at the maximum is exactly 0 after the shift
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kRowWaves + (threadIdx.x >> 6);
  if (r >= N) return;
  const float* lr = logit + r * K;
  const float* zr = zk + r * K;
  const float w = row_weight ? row_weight[r] : 1.f;
  const float c2 = kLog2e / T;
  float ma = -INFINITY, mu = -INFINITY;
  for (int k = lane; k < K; k += 64) {
    const float l = lr[k];
    if (finite_logit(l)) {
      ma = fmaxf(ma, (l * c2));
      mu = fmaxf(mu, (zr[k] * c2));
    }
  }
  ma = wave_max(ma);
  mu = wave_max(mu);
  if (w == 0.f || ma == -INFINITY) {  // zero weight or no cached entry: nothing
    if constexpr (COEF) {
      for (int k = lane; k < K; k += 64) coef[r * K + k] = 0.f;
    } else {
      if (lane == 0) row_loss[r] = 0.f;
    }
    return;
  }
  float sa = 0.f, su = 0.f;
  for (int k = lane; k < K; k += 64) {
    const float l = lr[k];
    if (finite_logit(l)) {
      sa += fast_exp2((l * c2) - ma);
      su += fast_exp2((zr[k] * c2) - mu);
    }
  }
  sa = wave_sum(sa);
  su = wave_sum(su);
  const float lsa = log2f(sa), lsu = log2f(su);
  if constexpr (!COEF) {
    // log2 p_k - log2 q_k = (l_k c2 - ma) - (z_k c2 - mu) - (log2 sa - log2 su): each
    // side shifted by its own max first (exact at the max), so a one-entry row
    // gives exactly 0
    const float C = lsa - lsu;
    float acc = 0.f;
    for (int k = lane; k < K; k += 64) {
      const float l = lr[k];
      if (finite_logit(l)) {
        const float ea = (l * c2) - ma;
        acc += fast_exp2(ea) * ((ea - ((zr[k] * c2) - mu)) - C);
      }
    }
    acc = wave_sum(acc) / sa;
    if (lane == 0) row_loss[r] = w * T * T * kLn2 * acc;
  } else {
    float ps = 0.f;
    for (int k = lane; k < K; k += 64) {
      const float l = lr[k];
      if (finite_logit(l)) ps += fast_exp2((l * c2) - ma - lsa);
    }
    ps = wave_sum(ps);
    const float sc = (grad_loss ? *grad_loss : 1.f) * w * T;
    for (int k = lane; k < K; k += 64) {
      const float l = lr[k];
      float g = 0.f;
      if (finite_logit(l))
        g = sc * (fast_exp2((zr[k] * c2) - mu - lsu) * ps -
                  fast_exp2((l * c2) - ma - lsa));
      coef[r * K + k] = g;
    }
  }
}

// grad_hidden row r = sum_k coef[r, k] W[idx[r, k]]: one workgroup per row,
// thread t owns columns 8t .. 8t + 7 (blockDim.x * 8 >= d).
template <class P>
__global__ __launch_bounds__(1024) void k_renorm_grad_h(const unsigned char* __restrict__ W,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ coef, int K,
                                                        int64_t d, unsigned char* __restrict__ gh) {
  __shared__ int32_t sid[kRenormMaxK];
  __shared__ float sg[kRenormMaxK];
  const int64_t r = blockIdx.x;
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    sid[k] = idx[r * K + k];
    sg[k] = coef[r * K + k];
  }
  __syncthreads();
  const int64_t c0 = static_cast<int64_t>(threadIdx.x) * 8;
  if (c0 >= d) return;
  const int64_t ld = d * P::kBytes;
  const unsigned char* wc = W + c0 * P::kBytes;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= K; k += 8) {
    float x[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8<P>(wc + sid[k + u] * ld, x[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(sg[k + u], x[u][e], acc[e]);
  }
  for (; k < K; ++k) {
    float x[8];
    load8<P>(wc + sid[k] * ld, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(sg[k], x[e], acc[e]);
  }
  store8<P>(gh + r * ld + c0 * P::kBytes, acc);
}

// Counts of each id per block of rows: hist[b][v], b = pair / pairs_per_block.
__global__ __launch_bounds__(256) void k_rs_hist(const int32_t* __restrict__ idx, int64_t NK,
                                                 int64_t pairs_per_block, int64_t V,
                                                 int32_t* __restrict__ hist) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; p < NK;
       p += stride)
    atomicAdd(&hist[(p / pairs_per_block) * V + idx[p]], 1);
}

// Per id v: hist[b][v] <- sum of hist[b'][v] for b' < b; total[v] <- sum over all b.
__global__ __launch_bounds__(256) void k_rs_colscan(int32_t* __restrict__ hist, int64_t nb,
                                                    int64_t V, int32_t* __restrict__ total) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= V) return;
  int32_t acc = 0;
  for (int64_t b = 0; b < nb; ++b) {
    const int32_t c = hist[b * V + v];
    hist[b * V + v] = acc;
    acc += c;
  }
  total[v] = acc;
}

// Hot ids and the cold bucket starts, one workgroup of 1024 threads. tau =
// the smallest power of two >= hot_min with at most hot_max ids of count >=
// tau (no id is hot when even the largest power of two leaves more).
// slot[v] = the hot id's index (in id order) or -1, hot_ids[slot] = v,
// info[0] = the number of hot ids; start[v] = sum of the counts of cold ids
// below v, start[V] = the number of cold pairs. The ids go through LDS in
// tiles of kHotTile: read and written with consecutive threads on
// consecutive ids, scanned with each thread owning 8 consecutive ids.
constexpr int kHotTile = 8192;

__global__ __launch_bounds__(1024) void k_rs_hot(const int32_t* __restrict__ total, int64_t V,
                                                 int32_t hot_min, int32_t hot_max,
                                                 int32_t* __restrict__ slot,
                                                 int32_t* __restrict__ hot_ids,
                                                 int32_t* __restrict__ info,
                                                 int32_t* __restrict__ start) {
  __shared__ int32_t bins[32];
  __shared__ int32_t s_tau;
  __shared__ int32_t wsum[16][2];
  __shared__ int32_t s_carry[2];
  __shared__ int32_t tc[kHotTile];   // counts of the tile, then bucket starts
  __shared__ int32_t tsl[kHotTile];  // slots of the tile
  constexpr int kPer = kHotTile / 1024;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if (t < 32) bins[t] = 0;
  if (t < 2) s_carry[t] = 0;
  __syncthreads();
  for (int64_t v = t; v < V; v += 1024) {
    const int32_t c = total[v];
    if (c >= hot_min) atomicAdd(&bins[31 - __clz(c)], 1);
  }
  __syncthreads();
  if (t == 0) {
    // ge = ids (of count >= hot_min) whose count is >= 2^b
    int32_t tau = 0x7fffffff, ge = bins[31];
    for (int b = 30; b >= 0; --b) {
      ge += bins[b];
      if (ge > hot_max) break;
      const int32_t lo = int32_t(1) << b;
      tau = lo < hot_min ? hot_min : lo;
      if (lo <= hot_min) break;
    }
    s_tau = tau;
  }
  __syncthreads();
  const int32_t tau = s_tau;
  for (int64_t base = 0; base < V; base += kHotTile) {
    const int n = V - base < kHotTile ? static_cast<int>(V - base) : kHotTile;
    for (int i = t; i < kHotTile; i += 1024) tc[i] = i < n ? total[base + i] : 0;
    __syncthreads();
    int32_t nh = 0, nc = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = t * kPer + j;
      const int32_t c = tc[i];
      if (i < n && c >= tau) ++nh; else nc += c;
    }
    // exclusive prefixes of (hot ids, cold pairs) over the workgroup
    int32_t xh = nh, xc = nc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t yh = __shfl_up(xh, o), yc = __shfl_up(xc, o);
      if (lane >= o) {
        xh += yh;
        xc += yc;
      }
    }
    if (lane == 63) {
      wsum[wv][0] = xh;
      wsum[wv][1] = xc;
    }
    __syncthreads();
    int32_t bh = s_carry[0], bc = s_carry[1];
    for (int i = 0; i < wv; ++i) {
      bh += wsum[i][0];
      bc += wsum[i][1];
    }
    int32_t h = bh + xh - nh, run = bc + xc - nc;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = t * kPer + j;
      const int32_t c = tc[i];
      tc[i] = run;
      if (i < n && c >= tau) {
        tsl[i] = h;
        hot_ids[h] = static_cast<int32_t>(base + i);
        ++h;
      } else {
        tsl[i] = -1;
        run += c;
      }
    }
    __syncthreads();
    for (int i = t; i < n; i += 1024) {
      start[base + i] = tc[i];
      slot[base + i] = tsl[i];
    }
    if (t == 1023) {  // carry the tile's totals into the next
      s_carry[0] = bh + xh;
      s_carry[1] = bc + xc;
    }
    __syncthreads();
  }
  if (t == 0) {
    start[V] = s_carry[1];
    info[0] = s_carry[0];
  }
}

// Stable placement: block b walks its rows in order; within a row each id's
// first copy reserves its copies' slots with one returning atomic on the
// block's cursor hist[b][v] (private to the block, so the values returned
// follow the row order), and every copy lands at start[v] + base + (earlier
// copies in the row).
__global__ __launch_bounds__(256) void k_rs_place(const int32_t* __restrict__ idx, int64_t N,
                                                  int K, int64_t rows_per_block, int64_t V,
                                                  const int32_t* __restrict__ slot,
                                                  int32_t* __restrict__ hist,
                                                  const int32_t* __restrict__ start,
                                                  int32_t* __restrict__ perm) {
  __shared__ int32_t sid[kRenormMaxK];
  __shared__ int32_t sbase[kRenormMaxK];
  constexpr int kPer = kRenormMaxK / 256;
  const int64_t b = blockIdx.x;
  const int64_t r0 = b * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < N ? r0 + rows_per_block : N;
  int32_t* cur = hist + b * V;
  const int t = threadIdx.x;
  for (int64_t r = r0; r < r1; ++r) {
    for (int k = t; k < K; k += 256) {
      const int32_t v = idx[r * K + k];
      sid[k] = slot[v] < 0 ? v : -1;  // hot pairs take no part in the sort
    }
    __syncthreads();
    int dup[kPer], first[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = t + 256 * j;
      dup[j] = 0;
      first[j] = k;
      if (k < K && sid[k] >= 0) {
        const int32_t v = sid[k];
        int mult = 0, fst = -1;
        for (int k2 = 0; k2 < K; ++k2) {
          const bool eq = sid[k2] == v;
          mult += eq ? 1 : 0;
          dup[j] += (eq && k2 < k) ? 1 : 0;
          if (eq && fst < 0) fst = k2;
        }
        first[j] = fst;
        if (dup[j] == 0) sbase[k] = atomicAdd(&cur[v], mult);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = t + 256 * j;
      if (k < K && sid[k] >= 0)
        perm[start[sid[k]] + sbase[first[j]] + dup[j]] = static_cast<int32_t>(r * K + k);
    }
    __syncthreads();
  }
}

// Chunk c covers sorted positions [c * seg, min(NK, (c + 1) * seg)), seg <=
// kRenormMaxSeg. Its pairs' rows, coefficients and ids are first staged in LDS
// (one coalesced pass, the gathers all in flight at once). For each run of one
// id v inside it, the sum of coef[p] * H[p / K] over the run's pairs p in sorted
// order goes to grad_W[v] (written, or added with ACC) when the chunk holds v's
// whole bucket, else to partial[c][0] (the bucket began in an earlier chunk) or
// partial[c][1] (it begins here and continues).
template <class P>
__global__ __launch_bounds__(1024) void k_rs_chunks(
    const unsigned char* __restrict__ H, const int32_t* __restrict__ idx,
    const float* __restrict__ coef, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ start, int64_t V, int K, int64_t d, int64_t seg, bool acc_out,
    float* __restrict__ gw, float* __restrict__ partial) {
  __shared__ int32_t srow[kRenormMaxSeg];
  const int64_t NK = start[V];  // sorted (cold) pairs; chunks past them have nothing to do
  __shared__ int32_t sv[kRenormMaxSeg];
  __shared__ float sc[kRenormMaxSeg];
  const int64_t c = blockIdx.x;
  const int64_t a = c * seg, e = a + seg < NK ? a + seg : NK;
  if (a >= NK) return;
  const int n = static_cast<int>(e - a);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int32_t p = perm[a + i];
    srow[i] = p / K;
    sv[i] = idx[p];
    sc[i] = coef[p];
  }
  __syncthreads();
  const int64_t c0 = static_cast<int64_t>(threadIdx.x) * 8;
  if (c0 >= d) return;
  const int64_t ld = d * P::kBytes;
  const unsigned char* hc = H + c0 * P::kBytes;
  // The chunk's pairs are taken eight at a time whatever the runs (runs of
  // rare ids are one to a few pairs long), so eight row loads are always in
  // flight; a run's sum is written out when its last pair has been added.
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto flush = [&](int q) {  // q: the last pair of a run
    const int32_t v = sv[q];
    const int64_t bs = start[v], be = start[v + 1];
    float* dst;
    bool add = false;
    if (bs < a)
      dst = partial + (2 * c) * d + c0;
    else if (be > e)
      dst = partial + (2 * c + 1) * d + c0;
    else {
      dst = gw + static_cast<int64_t>(v) * d + c0;
      add = acc_out;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dst[j] = add ? dst[j] + acc[j] : acc[j];
      acc[j] = 0.f;
    }
  };
  int q = 0;
  for (; q + 8 <= n; q += 8) {
    float x[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8<P>(hc + srow[q + u] * ld, x[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float g = sc[q + u];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(g, x[u][j], acc[j]);
      if (q + u + 1 == n || sv[q + u + 1] != sv[q + u]) flush(q + u);
    }
  }
  for (; q < n; ++q) {
    float x[8];
    load8<P>(hc + srow[q] * ld, x);
    const float g = sc[q];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(g, x[j], acc[j]);
    if (q + 1 == n || sv[q + 1] != sv[q]) flush(q);
  }
}

// One workgroup per id: a bucket spanning chunks c0 < c1 sums the tail partial
// of c0, the head partials of c0 + 1 .. c1 in order; an id with no pair gets
// a zero row unless grad_W is accumulated.
__global__ __launch_bounds__(256) void k_rs_fix(const int32_t* __restrict__ start,
                                                const int32_t* __restrict__ slot, int64_t d,
                                                int64_t seg, bool acc_out,
                                                const float* __restrict__ partial,
                                                float* __restrict__ gw) {
  const int64_t v = blockIdx.x;
  if (slot[v] >= 0) return;  // a hot id: its row comes from the dense product
  const int64_t bs = start[v], be = start[v + 1];
  float* row = gw + v * d;
  if (be == bs) {
    if (!acc_out)
      for (int64_t j = threadIdx.x; j < d; j += blockDim.x) row[j] = 0.f;
    return;
  }
  const int64_t c0 = bs / seg, c1 = (be - 1) / seg;
  if (c0 == c1) return;
  for (int64_t j = threadIdx.x; j < d; j += blockDim.x) {
    float s = partial[(2 * c0 + 1) * d + j];
    for (int64_t c = c0 + 1; c <= c1; ++c) s += partial[(2 * c) * d + j];
    row[j] = acc_out ? row[j] + s : s;
  }
}

// Rows [r0, r0 + nrows): C[r - r0][slot[v]] = sum of coef[r][k] over the
// entries k of row r with hot id v, in entry order (one wave per row; C is
// zero elsewhere, filled beforehand; row pitch `pitch` elements).
template <class P>
__global__ __launch_bounds__(256) void k_rs_hot_coef(const int32_t* __restrict__ idx,
                                                     const float* __restrict__ coef,
                                                     const int32_t* __restrict__ slot, int64_t r0,
                                                     int64_t nrows, int K, int64_t pitch,
                                                     unsigned char* __restrict__ C) {
  const int lane = threadIdx.x & 63;
  const int64_t rl = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (rl >= nrows) return;
  const int32_t* ir = idx + (r0 + rl) * K;
  const float* cr = coef + (r0 + rl) * K;
  for (int k = lane; k < K; k += 64) {
    const int32_t v = ir[k];
    const int32_t sl = slot[v];
    if (sl < 0) continue;
    bool first = true;
    for (int k2 = 0; k2 < k && first; ++k2) first = ir[k2] != v;
    if (!first) continue;
    float g = 0.f;
    for (int k2 = k; k2 < K; ++k2)
      if (ir[k2] == v) g += cr[k2];
    unsigned char* dst = C + (rl * pitch + sl) * P::kBytes;
    if constexpr (P::kBytes == 2)
      *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16_rne(g);
    else
      *reinterpret_cast<float*>(dst) = g;
  }
}

// grad_W[hot_ids[j]] (=, or += with acc_out) the sum over the splits, in split
// order, of prod[split][j], for j < info[0].
__global__ __launch_bounds__(256) void k_rs_hot_rows(const int32_t* __restrict__ hot_ids,
                                                     const int32_t* __restrict__ info,
                                                     const float* __restrict__ prod, int64_t d,
                                                     int64_t splits, int64_t split_stride,
                                                     bool acc_out, float* __restrict__ gw) {
  const int64_t j = blockIdx.x;
  if (j >= info[0]) return;
  float* row = gw + static_cast<int64_t>(hot_ids[j]) * d;
  const float* src = prod + j * d;
  for (int64_t c = threadIdx.x; c < d; c += blockDim.x) {
    float v = src[c];
    for (int64_t i = 1; i < splits; ++i) v += src[i * split_stride + c];
    row[c] = acc_out ? row[c] + v : v;
  }
}

// ------------------------------------------------------------------ launchers

void launch_renorm_rows(bool coef_mode, const float* zk, const float* logit,
                        const float* row_weight, const float* grad_loss, int64_t N, int K,
                        float T, float* row_loss, float* coef, hipStream_t s) {
  if (N <= 0) return;
  ScopedTimer timer_(KID_RENORM_ROWS, s);
  const unsigned grid = static_cast<unsigned>(ceil_div(N, kRowWaves));
  if (coef_mode)
    k_renorm_rows<true><<<grid, 64 * kRowWaves, 0, s>>>(zk, logit, row_weight, grad_loss, N, K, T,
                                                         row_loss, coef);
  else
    k_renorm_rows<false><<<grid, 64 * kRowWaves, 0, s>>>(zk, logit, row_weight, grad_loss, N, K,
                                                          T, row_loss, coef);
}

static unsigned column_threads(int64_t d) {
  return static_cast<unsigned>(round_up(ceil_div(d, 8), 64));
}

void launch_renorm_grad_h(int dtype, const void* W, const int32_t* idx, const float* coef,
                          int64_t N, int K, int64_t d, void* gh, hipStream_t s) {
  if (N <= 0) return;
  ScopedTimer timer_(KID_RENORM_GRAD_H, s);
  const unsigned threads = column_threads(d);
  const unsigned char* Wc = static_cast<const unsigned char*>(W);
  unsigned char* out = static_cast<unsigned char*>(gh);
  if (dtype == 1)
    k_renorm_grad_h<BF16><<<static_cast<unsigned>(N), threads, 0, s>>>(Wc, idx, coef, K, d, out);
  else
    k_renorm_grad_h<F32><<<static_cast<unsigned>(N), threads, 0, s>>>(Wc, idx, coef, K, d, out);
}

void launch_renorm_grad_w(int dtype, const void* H, const int32_t* idx, const float* coef,
                          int64_t N, int K, int64_t d, int64_t V, const RenormSortPlan& q,
                          const RenormBuffers& b, bool acc_out, float* gw, hipStream_t s) {
  const int64_t NK = N * K;
  const int64_t eb = dtype == 1 ? 2 : 4;
  if (NK > 0) {
    launch_fill_f32(reinterpret_cast<float*>(b.hist), q.nb * V, 0.0f, s);  // integer zero
    {
      ScopedTimer timer_(KID_RS_HIST, s);
      const int64_t blocks = ceil_div(NK, 256) < 8192 ? ceil_div(NK, 256) : 8192;
      k_rs_hist<<<static_cast<unsigned>(blocks), 256, 0, s>>>(idx, NK, q.rows_per_block * K, V,
                                                              b.hist);
    }
    {
      ScopedTimer timer_(KID_RS_SCAN, s);
      k_rs_colscan<<<static_cast<unsigned>(ceil_div(V, 256)), 256, 0, s>>>(b.hist, q.nb, V,
                                                                          b.total);
      k_rs_hot<<<1, 1024, 0, s>>>(b.total, V, kRenormHotMin, static_cast<int32_t>(q.hot_max),
                                   b.slot, b.hot_ids, b.info, b.start);
    }
    {
      ScopedTimer timer_(KID_RS_PLACE, s);
      k_rs_place<<<static_cast<unsigned>(q.nb), 256, 0, s>>>(idx, N, K, q.rows_per_block, V,
                                                             b.slot, b.hist, b.start, b.perm);
    }
    {
      ScopedTimer timer_(KID_RS_CHUNKS, s);
      const unsigned threads = column_threads(d);
      const unsigned char* Hc = static_cast<const unsigned char*>(H);
      if (dtype == 1)
        k_rs_chunks<BF16><<<static_cast<unsigned>(q.nchunks), threads, 0, s>>>(
            Hc, idx, coef, b.perm, b.start, V, K, d, q.seg, acc_out, gw, b.partial);
      else
        k_rs_chunks<F32><<<static_cast<unsigned>(q.nchunks), threads, 0, s>>>(
            Hc, idx, coef, b.perm, b.start, V, K, d, q.seg, acc_out, gw, b.partial);
    }
  } else {
    // no pairs: every bucket is empty and no id is hot
    launch_fill_f32(reinterpret_cast<float*>(b.start), V + 1, 0.0f, s);
    launch_fill_f32(reinterpret_cast<float*>(b.slot), V, __builtin_bit_cast(float, -1), s);
  }
  {
    ScopedTimer timer_(KID_RS_FIX, s);
    k_rs_fix<<<static_cast<unsigned>(V), 256, 0, s>>>(b.start, b.slot, d, q.seg, acc_out,
                                                      b.partial, gw);
  }
  if (NK == 0) return;
  // hot ids: C^T H over row blocks of q.hot_rows rows, then the rows into grad_W
  for (int64_t r0 = 0; r0 < N; r0 += q.hot_rows) {
    const int64_t nr = N - r0 < q.hot_rows ? N - r0 : q.hot_rows;
    launch_fill_f32(reinterpret_cast<float*>(b.hot_c), nr * q.hot_max * eb / 4, 0.0f, s);
    {
      ScopedTimer timer_(KID_RS_HOT, s);
      const unsigned grid = static_cast<unsigned>(ceil_div(nr, 4));
      if (dtype == 1)
        k_rs_hot_coef<BF16><<<grid, 256, 0, s>>>(idx, coef, b.slot, r0, nr, K, q.hot_max,
                                                 b.hot_c);
      else
        k_rs_hot_coef<F32><<<grid, 256, 0, s>>>(idx, coef, b.slot, r0, nr, K, q.hot_max, b.hot_c);
    }
    launch_grad_w_split(dtype, b.hot_c, q.hot_max, H, d, q.hot_max, q.hot_max, r0, nr,
                        q.hot_splits, r0 > 0, b.hot_prod, q.hot_max * d, s);
  }
  ScopedTimer timer_(KID_RS_HOT, s);
  k_rs_hot_rows<<<static_cast<unsigned>(q.hot_max), 256, 0, s>>>(
      b.hot_ids, b.info, b.hot_prod, d, q.hot_splits, q.hot_max * d, acc_out, gw);
}

}  // namespace fkl
