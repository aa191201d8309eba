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
//   k_renorm_grad_h  one wave per (row, eighth of the columns), the eighths
//                    dealt to the XCDs: sum_k G_rk W[idx_rk] (16-byte loads,
//                    eight weight rows in flight per lane)
//   grad_W without float atomics, bitwise deterministic:
//   k_rs_hist        per block of rows, the count of each id (integer atomics)
//   k_rs_colscan     per id, exclusive prefix of its counts over the blocks
//   k_rs_tau, k_rs_hot_sums, k_rs_hot_place
//                    pick the frequent ("hot") ids: count >= tau, tau the
//                    smallest power of two >= kRenormHotMin that leaves at
//                    most hot_max of them (as many as one round of 256 x 256
//                    product tiles takes); give each a slot, and the
//                    exclusive prefix over the other ("cold") ids of their
//                    counts: bucket starts of the cold pairs
//   hot ids, a dense product: k_rs_hot_coef writes each row of C
//   [rows x hot_max], the row's hot coefficients (copies of one id in a row
//   summed in entry order) and zeros, k_grad_w (the loss's MFMA kernel, its rows split
//   over the XCDs its tiles alone would leave idle) forms C^T H, and
//   k_rs_hot_rows sums the splits in order into each hot id's grad_W row
//   cold ids, a sort:
//   k_rs_place       per block, its rows in order: each cold pair (r, k) goes
//                    to start[v] + (pairs of id v in earlier rows) + (copies of
//                    v earlier in row r): a stable counting sort by id, which
//                    writes each pair's row, id and coefficient there
//   k_rs_slices      the hidden rows copied slice-major, 64 columns a slice
//   k_rs_chunks      fixed chunks of the sorted pairs, slice by slice, each XCD
//                    walking one slice at a time: the sum of G h over each run
//                    of one id, written to grad_W when the chunk holds the
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
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kWalkLanes = kRenormSliceCols / 8;  // lanes of a k_rs_chunks group, 8 columns each
constexpr int kWalkGroups = 256 / kWalkLanes;     // groups (shares) per k_rs_chunks workgroup

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
// grad_h[r] = sum_k coef[r][k] W[idx[r][k]], one wave per (row, eighth of
// the columns): workgroup b takes rows 4 (b >> 3) .. 4 (b >> 3) + 3, a wave
// each, on column eighth b & 7. Workgroups are dealt to the 8 XCDs in turn,
// so each XCD reads one eighth of every weight row it needs, and the eighths
// of the frequent ids' rows (2048 x 768 bytes at d 3072) stay in its L2,
// where their whole rows (12.6 MB) did not fit. Each column adds its K terms
// in entry order, eight weight loads in flight per lane.
template <class P>
__global__ __launch_bounds__(256) void k_renorm_grad_h(const unsigned char* __restrict__ W,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ coef, int64_t N,
                                                       int K, int64_t d,
                                                       unsigned char* __restrict__ gh) {
  extern __shared__ int32_t sh_gh[];  // per wave: K ids, then K coefficients
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t* sid = sh_gh + w * 2 * K;
  float* sg = reinterpret_cast<float*>(sid + K);
  const int64_t x = blockIdx.x & 7;
  const int64_t cs = (d + 63) / 64 * 8;  // columns per eighth, a multiple of 8
  const int64_t c_hi = (x + 1) * cs < d ? (x + 1) * cs : d;
  const int64_t ld = d * P::kBytes;
  // groups of four rows, more than one per workgroup only when the grid is capped
  for (int64_t rb = blockIdx.x >> 3; rb * 4 < N; rb += gridDim.x >> 3) {
    const int64_t r = rb * 4 + w;
    const bool valid = r < N;
    __syncthreads();  // the previous group is done with LDS
    if (valid)
      for (int k = lane; k < K; k += 64) {
        sid[k] = idx[r * K + k];
        sg[k] = coef[r * K + k];
      }
    __syncthreads();
    if (!valid) continue;
    for (int64_t c0 = x * cs + lane * 8; c0 < c_hi; c0 += 512) {
      const unsigned char* wc = W + c0 * P::kBytes;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < K; k += 8) {
        // every load is issued (an entry past K reloads entry k), so that no
        // load waits behind a branch for the ones before it
        u32x4_t raw[8][P::kBytes / 2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const unsigned char* src = wc + sid[k + u < K ? k + u : k] * ld;
#pragma unroll
          for (int h = 0; h < P::kBytes / 2; ++h) raw[u][h] = load16(src + 16 * h);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (k + u < K) {
            const float gg = sg[k + u];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float xv;
              if constexpr (P::kBytes == 2)
                xv = as_f32((e & 1) ? (raw[u][0][e >> 1] & 0xffff0000u)
                                    : (raw[u][0][e >> 1] << 16));
              else
                xv = as_f32(raw[u][e >> 2][e & 3]);
              acc[e] = fmaf(gg, xv, acc[e]);
            }
          }
        }
      }
      store8<P>(gh + r * ld + c0 * P::kBytes, acc);
    }
  }
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
  int64_t b = 0;
  // sixteen blocks' counts loaded together, then their prefixes stored (one
  // load at a time waited on every load in turn)
  for (; b + 16 <= nb; b += 16) {
    int32_t c[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) c[u] = hist[(b + u) * V + v];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      hist[(b + u) * V + v] = acc;
      acc += c[u];
    }
  }
  for (; b < nb; ++b) {
    const int32_t c = hist[b * V + v];
    hist[b * V + v] = acc;
    acc += c;
  }
  total[v] = acc;
}

// Hot ids and the cold bucket starts. tau = the smallest power of two >=
// hot_min with at most hot_max ids of count >= tau (no id is hot when even the
// largest power of two leaves more); slot[v] = the hot id's index (in id
// order) or -1, hot_ids[slot] = v, info[0] = the number of hot ids; start[v]
// = sum of the counts of cold ids below v, start[V] = the number of cold
// pairs. Three launches: k_rs_tau (one workgroup) finds tau (info[1]);
// k_rs_hot_sums (a workgroup per tile of kHotTile ids) counts each tile's hot
// ids and cold pairs; k_rs_hot_place (a workgroup per tile) adds the earlier
// tiles' counts and writes the tile, its ids going through LDS read and
// written by consecutive threads on consecutive ids and scanned with each
// thread owning 8 consecutive ids.
constexpr int kHotTile = 8192;

__global__ __launch_bounds__(1024) void k_rs_tau(const int32_t* __restrict__ total, int64_t V,
                                                 int32_t hot_min, int32_t hot_max,
                                                 int32_t* __restrict__ info) {
  __shared__ int32_t bins[32];
  const int t = threadIdx.x;
  if (t < 32) bins[t] = 0;
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
    info[1] = tau;
  }
}

__global__ __launch_bounds__(1024) void k_rs_hot_sums(const int32_t* __restrict__ total,
                                                      int64_t V,
                                                      const int32_t* __restrict__ info,
                                                      int32_t* __restrict__ tsum) {
  __shared__ int32_t wsum[16][2];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int32_t tau = info[1];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kHotTile;
  int32_t nh = 0, nc = 0;
  for (int i = t; i < kHotTile && base + i < V; i += 1024) {
    const int32_t c = total[base + i];
    if (c >= tau)
      ++nh;
    else
      nc += c;
  }
  for (int o = 32; o > 0; o >>= 1) {
    nh += __shfl_xor(nh, o);
    nc += __shfl_xor(nc, o);
  }
  if (lane == 0) {
    wsum[wv][0] = nh;
    wsum[wv][1] = nc;
  }
  __syncthreads();
  if (t == 0) {
    int32_t h = 0, c = 0;
    for (int i = 0; i < 16; ++i) {
      h += wsum[i][0];
      c += wsum[i][1];
    }
    tsum[2 * blockIdx.x] = h;
    tsum[2 * blockIdx.x + 1] = c;
  }
}

__global__ __launch_bounds__(1024) void k_rs_hot_place(const int32_t* __restrict__ total,
                                                       int64_t V,
                                                       int32_t* __restrict__ info,
                                                       const int32_t* __restrict__ tsum,
                                                       int32_t* __restrict__ slot,
                                                       int32_t* __restrict__ hot_ids,
                                                       int32_t* __restrict__ start) {
  __shared__ int32_t wsum[16][2];
  __shared__ int32_t s_base[2];
  __shared__ int32_t tc[kHotTile];   // counts of the tile, then bucket starts
  __shared__ int32_t tsl[kHotTile];  // slots of the tile
  constexpr int kPer = kHotTile / 1024;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int32_t tau = info[1];
  const int64_t tile = blockIdx.x, base = tile * kHotTile;
  const int n = V - base < kHotTile ? static_cast<int>(V - base) : kHotTile;
  // the earlier tiles' hot ids and cold pairs
  int32_t bh = 0, bc = 0;
  for (int64_t i = t; i < tile; i += 1024) {
    bh += tsum[2 * i];
    bc += tsum[2 * i + 1];
  }
  for (int o = 32; o > 0; o >>= 1) {
    bh += __shfl_xor(bh, o);
    bc += __shfl_xor(bc, o);
  }
  if (lane == 0) {
    wsum[wv][0] = bh;
    wsum[wv][1] = bc;
  }
  for (int i = t; i < kHotTile; i += 1024) tc[i] = i < n ? total[base + i] : 0;
  __syncthreads();
  if (t == 0) {
    int32_t h = 0, c = 0;
    for (int i = 0; i < 16; ++i) {
      h += wsum[i][0];
      c += wsum[i][1];
    }
    s_base[0] = h;
    s_base[1] = c;
  }
  __syncthreads();
  int32_t nh = 0, nc = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = t * kPer + j;
    const int32_t c = tc[i];
    if (i < n && c >= tau)
      ++nh;
    else
      nc += c;
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
  if (lane == 63) {  // wsum's earlier reader (thread 0) passed the barrier above
    wsum[wv][0] = xh;
    wsum[wv][1] = xc;
  }
  __syncthreads();
  bh = s_base[0];
  bc = s_base[1];
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
  if (t == 1023 && base + kHotTile >= V) {  // the last tile: the totals
    start[V] = bc + xc;
    info[0] = bh + xh;
  }
}

// Stable placement: block b walks its rows in order, R = floor(1024 / K)
// rows at a time (one contiguous range of at most 1024 pairs). A range's cold
// entries are sorted in LDS by (id, entry) with a bitonic network, so each
// id's copies form a run in pair order; the run's first element reserves its
// copies' slots with one returning atomic on the block's cursor hist[b][v]
// (private to the block, so the values returned follow the row order), and
// the copy at rank i of the run lands at start[v] + base + i, where its row,
// id and coefficient are written. A range's ids are loaded two ranges ahead
// and their hot slots, bucket starts and coefficients one range ahead, so
// that a range waits on its atomics alone; entries past the block load entry
// 0 of the range (valid) and are not used, so no load sits behind a branch.
__global__ __launch_bounds__(256) void k_rs_place(const int32_t* __restrict__ idx,
                                                  const float* __restrict__ coef, int64_t N,
                                                  int K, int64_t rows_per_block, int64_t V,
                                                  const int32_t* __restrict__ slot,
                                                  int32_t* __restrict__ hist,
                                                  const int32_t* __restrict__ start,
                                                  int32_t* __restrict__ srow,
                                                  int32_t* __restrict__ sid,
                                                  float* __restrict__ scoef) {
  constexpr int kN = kRenormMaxK;       // sort size (a power of two)
  constexpr int kPer = kN / 256;
  __shared__ uint64_t key[kN];          // (id << 11) | entry, or ~0 for no cold entry
  __shared__ int32_t lst[kN];           // bucket start of entry e's id
  __shared__ float lcf[kN];             // coefficient of entry e
  __shared__ int32_t base[kN];          // at a run's first sorted position: its slots' base
  const int64_t b = blockIdx.x;
  const int64_t r0 = b * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < N ? r0 + rows_per_block : N;
  if (r0 >= r1) return;
  int32_t* cur = hist + b * V;
  const int t = threadIdx.x;
  const int64_t R = kN / K;           // rows per range (K <= kRenormMaxK)
  const int64_t p1 = r1 * K;          // the block's pairs end here
  // entry j of this thread in the range starting at pair q (clamped)
  auto ent = [&](int64_t q, int j) {
    const int64_t e = q + t + 256 * j;
    return e < q + R * K && e < p1 ? e : q;
  };
  auto rq = [&](int64_t q) { return q < p1 ? q : r0 * K; };  // a range past the block: any valid
  int32_t ida[kPer], idb[kPer], sl[kPer], st[kPer];
  float cf[kPer];
  const int64_t q0 = r0 * K;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    ida[j] = idx[ent(q0, j)];
    idb[j] = idx[ent(rq(q0 + R * K), j)];
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    sl[j] = slot[ida[j]];
    st[j] = start[ida[j]];
    cf[j] = coef[ent(q0, j)];
  }
  for (int64_t q = q0; q < p1; q += R * K) {
    const int n = static_cast<int>(q + R * K < p1 ? R * K : p1 - q);  // entries in the range
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = t + 256 * j;
      const bool cold = e < n && sl[j] < 0;  // hot pairs skip the sort
      key[e] = cold ? (static_cast<uint64_t>(ida[j]) << 11) | static_cast<uint64_t>(e)
                    : ~uint64_t(0);
      lst[e] = st[j];
      lcf[e] = cf[j];
    }
    // the next range's slots, starts and coefficients, the one after's ids
    int32_t idc[kPer], sl2[kPer], st2[kPer];
    float cf2[kPer];
    const int64_t qn = rq(q + R * K), qnn = rq(q + 2 * R * K);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      sl2[j] = slot[idb[j]];
      st2[j] = start[idb[j]];
      cf2[j] = coef[ent(qn, j)];
      idc[j] = idx[ent(qnn, j)];
    }
    __syncthreads();
    for (int size = 2; size <= kN; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
        for (int h = 0; h < kN / 512; ++h) {
          const int c = t + 256 * h;  // compare-exchange c of kN / 2
          const int i = 2 * stride * (c / stride) + (c % stride), i2 = i + stride;
          const uint64_t x = key[i], y = key[i2];
          if ((x > y) == ((i & size) == 0)) {
            key[i] = y;
            key[i2] = x;
          }
        }
        __syncthreads();
      }
    // run starts reserve their slots
    uint64_t kv[kPer];
    int rs[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = t + 256 * j;
      kv[j] = key[i];
      rs[j] = i;
      if (kv[j] != ~uint64_t(0)) {
        const uint64_t id = kv[j] >> 11;
        while (rs[j] > 0 && (key[rs[j] - 1] >> 11) == id) --rs[j];
        if (rs[j] == i) {
          int m = 1;
          while (i + m < kN && (key[i + m] >> 11) == id) ++m;
          base[i] = atomicAdd(&cur[id], m);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = t + 256 * j;
      if (kv[j] != ~uint64_t(0)) {
        const int e = static_cast<int>(kv[j] & 2047);
        const int32_t pos = lst[e] + base[rs[j]] + (i - rs[j]);
        srow[pos] = static_cast<int32_t>((q + e) / K);
        sid[pos] = static_cast<int32_t>(kv[j] >> 11);
        scoef[pos] = lcf[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      ida[j] = idb[j];
      idb[j] = idc[j];
      sl[j] = sl2[j];
      st[j] = st2[j];
      cf[j] = cf2[j];
    }
  }
}

// Slice-major copy of the hidden rows for the walk below: slice s holds
// columns [64 s, 64 s + 64) of every row, one row after the other (128 bytes
// a row in bf16), so that a slice of all N rows is one contiguous block whose
// lines hold only that slice. Columns past d in the last slice are
// neither written nor read.
template <class P>
__global__ __launch_bounds__(256) void k_rs_slices(const unsigned char* __restrict__ H,
                                                   int64_t N, int64_t d,
                                                   unsigned char* __restrict__ hs) {
  const int64_t groups = d / 8;  // eight columns each
  const int64_t total = N * groups;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = u / groups, c8 = u - r * groups;
    float x[8];
    load8<P>(H + (r * d + c8 * 8) * P::kBytes, x);
    const int64_t sl = c8 / (kRenormSliceCols / 8), part = c8 - sl * (kRenormSliceCols / 8);
    store8<P>(hs + ((sl * N + r) * kRenormSliceCols + part * 8) * P::kBytes, x);
  }
}

// Chunk c of the sorted cold pairs (positions [c seg, min(NK, (c + 1) seg)),
// seg <= kRenormMaxSeg) on the kRenormSliceCols (64) columns of slice s. Work
// items are dealt so that each XCD (workgroups go to the 8 XCDs in turn) takes
// its slices one after the other, every chunk of a slice before the next
// slice, and the slice of the hidden rows it reads (N x 128 bytes in bf16)
// stays in its L2
// (all columns at once read each pair's whole row from memory, the pairs
// being sorted by id and their rows scattered). The grid is persistent: a
// workgroup loops over items, their number known only on the device.
//
// The chunk's rows, ids and coefficients are staged in LDS; 32 groups of
// eight lanes (eight columns a lane) take equal shares of its positions and
// sum coef * H[row] over each run (the pairs of one id) in sorted order, eight
// row loads in flight across runs (four in fp32). A run that lies inside one share is
// written out at once; the pieces of a run that crosses shares go to LDS, and
// after a barrier the share where the run began adds them in share order.
// A run's sum goes to grad_W[v] (or is added to it, with acc_out) when the
// chunk holds v's whole bucket, else to the chunk's head partial (the bucket
// began in an earlier chunk: only the chunk's first run) or tail partial (it
// continues: only the last run).
template <class P>
__global__ __launch_bounds__(256, 4) void k_rs_chunks(
    const unsigned char* __restrict__ hs, const int32_t* __restrict__ srow,
    const int32_t* __restrict__ sid, const float* __restrict__ scoef,
    const int32_t* __restrict__ start, int64_t N, int64_t V, int64_t d, int64_t seg,
    int64_t nslices, bool acc_out, float* __restrict__ gw, float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sh_walk[];
  float* piece = reinterpret_cast<float*>(sh_walk);  // [shares][2][slice columns]
  int32_t* lrow = reinterpret_cast<int32_t*>(piece + kWalkGroups * 2 * kRenormSliceCols);
  int32_t* lid = lrow + seg;
  float* lcoef = reinterpret_cast<float*>(lid + seg);
  __shared__ int32_t lcont[2];  // the first run continues a bucket, the last run's continues
  const int64_t NK = start[V];  // sorted (cold) pairs
  const int64_t nch = (NK + seg - 1) / seg;
  const int64_t items = (nslices + 7) / 8 * nch;
  const int g = threadIdx.x / kWalkLanes, l = threadIdx.x % kWalkLanes;
  constexpr int64_t ld = kRenormSliceCols * P::kBytes;
  const int64_t xcd = blockIdx.x & 7;
  for (int64_t j = blockIdx.x >> 3; j < items; j += gridDim.x >> 3) {
    const int64_t s = (j / nch) * 8 + xcd, c = j - (j / nch) * nch;
    if (s >= nslices) continue;  // uniform over the workgroup
    const int64_t a = c * seg, e = a + seg < NK ? a + seg : NK;
    const int n = static_cast<int>(e - a);
    __syncthreads();  // the previous item is done with LDS
    // four positions a thread per load, all loads in flight at once (the
    // arrays are padded so that a quad may run past the last pair; a thread
    // past the chunk reloads its first quad, so no load waits on a branch)
    u32x4_t qr[kRenormMaxSeg / 1024], qi[kRenormMaxSeg / 1024], qc[kRenormMaxSeg / 1024];
#pragma unroll
    for (int h = 0; h < kRenormMaxSeg / 1024; ++h) {
      const int i4 = (threadIdx.x + 256 * h) * 4;
      const int64_t o = a + (i4 < n ? i4 : 0);
      qr[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(srow + o));
      qi[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(sid + o));
      qc[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(scoef + o));
    }
#pragma unroll
    for (int h = 0; h < kRenormMaxSeg / 1024; ++h) {
      const int i4 = (threadIdx.x + 256 * h) * 4;
      if (i4 < n) {
        *reinterpret_cast<u32x4_t*>(lrow + i4) = qr[h];
        *reinterpret_cast<u32x4_t*>(lid + i4) = qi[h];
        *reinterpret_cast<u32x4_t*>(lcoef + i4) = qc[h];
      }
    }
    if (threadIdx.x == 0) {
      lcont[0] = a > 0 && sid[a - 1] == sid[a];
      lcont[1] = e < NK && sid[e] == sid[e - 1];
    }
    __syncthreads();
    const int64_t c0 = s * kRenormSliceCols + l * 8;
    const bool live = c0 < d;  // the last slice may be narrower than the others
    const int32_t first_id = lid[0], last_id = lid[n - 1];
    const bool head_cont = lcont[0] != 0, tail_cont = lcont[1] != 0;
    // eight columns as two 16-byte streaming stores (c0 is a multiple of 8)
    auto write_run = [&](int32_t v, const float (&x)[8]) {
      float* dst;
      bool add = false;
      if (head_cont && v == first_id)
        dst = partial + (2 * c) * d + c0;
      else if (tail_cont && v == last_id)
        dst = partial + (2 * c + 1) * d + c0;
      else {
        dst = gw + static_cast<int64_t>(v) * d + c0;
        add = acc_out;
      }
      f32x4_t* d4 = reinterpret_cast<f32x4_t*>(dst);
      f32x4_t lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
      if (add) {
        lo += d4[0];
        hi += d4[1];
      }
      __builtin_nontemporal_store(lo, d4);
      __builtin_nontemporal_store(hi, d4 + 1);
    };
    const int p0 = g * n / kWalkGroups, p1 = (g + 1) * n / kWalkGroups;
    // this share's first run began in an earlier share
    const bool open = p0 < p1 && p0 > 0 && lid[p0] == lid[p0 - 1];
    float* my = piece + (g * 2) * kRenormSliceCols + l * 8;
    const unsigned char* hc = hs + (s * N * kRenormSliceCols + l * 8) * P::kBytes;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int rs = p0;  // first position of the current run inside the share
    // eight rows in flight (four in fp32, whose rows take twice the registers)
    constexpr int kB = P::kBytes == 2 ? 8 : 4;
    for (int q = p0; q < p1; q += kB) {
      const int m = p1 - q < kB ? p1 - q : kB;
      // raw 16-byte loads, widened to fp32 as they are used (fewer registers
      // per load in flight)
      // Every load is issued (a position past the share reloads the first
      // row of the batch, and a lane past d reads columns of its own slice
      // that hold no data): loads behind a branch were each preceded by a
      // wait for all earlier ones.
      u32x4_t raw[kB][P::kBytes / 2];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const unsigned char* src = hc + lrow[u < m ? q + u : q] * ld;
#pragma unroll
        for (int h = 0; h < P::kBytes / 2; ++h) raw[u][h] = load16(src + 16 * h);
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (u < m) {
          const int qq = q + u;
          const float gg = lcoef[qq];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            float xv;
            if constexpr (P::kBytes == 2)
              xv = as_f32((k & 1) ? (raw[u][0][k >> 1] & 0xffff0000u) : (raw[u][0][k >> 1] << 16));
            else
              xv = as_f32(raw[u][k >> 2][k & 3]);
            acc[k] = fmaf(gg, xv, acc[k]);
          }
          const bool run_end = qq + 1 == n || lid[qq + 1] != lid[qq];
          if (run_end || qq + 1 == p1) {
            if (rs == p0 && open) {  // a piece of a run that began before the share
#pragma unroll
              for (int k = 0; k < 8; ++k) my[k] = acc[k];
            } else if (!run_end) {  // a run that continues past the share
#pragma unroll
              for (int k = 0; k < 8; ++k) my[kRenormSliceCols + k] = acc[k];
            } else if (live) {
              write_run(lid[qq], acc);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = 0.f;
            rs = qq + 1;
          }
        }
      }
    }
    __syncthreads();  // every piece is in LDS
    // The share whose last run began in it and continues adds the pieces of
    // the following shares (skipping empty ones) up to the run's end.
    if (p0 < p1 && p1 < n && lid[p1] == lid[p1 - 1] && !(open && lid[p0] == lid[p1 - 1]) &&
        live) {
      const int32_t v = lid[p1 - 1];
      float sum[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) sum[k] = my[kRenormSliceCols + k];
      for (int g2 = g + 1; g2 < kWalkGroups; ++g2) {
        const int b0 = g2 * n / kWalkGroups, b1 = (g2 + 1) * n / kWalkGroups;
        if (b0 == b1) continue;
        const float* pc = piece + (g2 * 2) * kRenormSliceCols + l * 8;
#pragma unroll
        for (int k = 0; k < 8; ++k) sum[k] += pc[k];
        if (b1 == n || lid[b1] != v) break;
      }
      write_run(v, sum);
    }
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
// entries k of row r with hot id v, in entry order, and 0 in the other
// columns (the whole row is written; row pitch `pitch` elements, a multiple
// of 8). One wave per row, four rows a workgroup: the row's ids are staged in
// LDS, its values built in an fp32 LDS row (the first copy of an id sums its
// copies), then written out 16 bytes a lane.
template <class P>
__global__ __launch_bounds__(256) void k_rs_hot_coef(const int32_t* __restrict__ idx,
                                                     const float* __restrict__ coef,
                                                     const int32_t* __restrict__ slot, int64_t r0,
                                                     int64_t nrows, int K, int64_t pitch,
                                                     unsigned char* __restrict__ C) {
  extern __shared__ int32_t sh_hc[];  // per wave: K ids, then pitch fp32 values
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t* lid = sh_hc + w * (K + pitch);
  float* val = reinterpret_cast<float*>(lid + K);
  const int64_t rl = static_cast<int64_t>(blockIdx.x) * 4 + w;
  const bool valid = rl < nrows;
  if (valid) {
    const int32_t* ir = idx + (r0 + rl) * K;
    for (int k = lane; k < K; k += 64) lid[k] = ir[k];
    for (int64_t c = lane; c < pitch; c += 64) val[c] = 0.f;
  }
  __syncthreads();
  if (valid) {
    const float* cr = coef + (r0 + rl) * K;
    for (int k = lane; k < K; k += 64) {
      const int32_t v = lid[k];
      const int32_t sl = slot[v];
      if (sl < 0) continue;
      bool first = true;
      for (int k2 = 0; k2 < k && first; ++k2) first = lid[k2] != v;
      if (!first) continue;
      float g = 0.f;
      for (int k2 = k; k2 < K; ++k2)
        if (lid[k2] == v) g += cr[k2];
      val[sl] = g;
    }
  }
  __syncthreads();
  if (!valid) return;
  unsigned char* dst = C + rl * pitch * P::kBytes;
  for (int64_t c = lane * 8; c < pitch; c += 512) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = val[c + e];
    store8<P>(dst + c * P::kBytes, x);
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

void launch_renorm_grad_h(int dtype, const void* W, const int32_t* idx, const float* coef,
                          int64_t N, int K, int64_t d, void* gh, hipStream_t s) {
  if (N <= 0) return;
  ScopedTimer timer_(KID_RENORM_GRAD_H, s);
  // eight workgroups per four rows, at most 2^23 (a grid of 2^32 work-items is the limit)
  const int64_t groups = ceil_div(N, 4) < (int64_t(1) << 20) ? ceil_div(N, 4) : int64_t(1) << 20;
  const unsigned grid = static_cast<unsigned>(8 * groups);
  const unsigned char* Wc = static_cast<const unsigned char*>(W);
  unsigned char* out = static_cast<unsigned char*>(gh);
  const size_t lds = static_cast<size_t>(4) * 2 * K * 4;
  if (dtype == 1)
    k_renorm_grad_h<BF16><<<grid, 256, lds, s>>>(Wc, idx, coef, N, K, d, out);
  else
    k_renorm_grad_h<F32><<<grid, 256, lds, s>>>(Wc, idx, coef, N, K, d, out);
}

void launch_renorm_grad_w(int dtype, const void* H, const int32_t* idx, const float* coef,
                          int64_t N, int K, int64_t d, int64_t V, const RenormSortPlan& q,
                          const RenormBuffers& b, bool acc_out, float* gw, hipStream_t s) {
  const int64_t NK = N * K;
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
      const unsigned tiles = static_cast<unsigned>(ceil_div(V, kHotTile));
      k_rs_tau<<<1, 1024, 0, s>>>(b.total, V, kRenormHotMin, static_cast<int32_t>(q.hot_max),
                                   b.info);
      k_rs_hot_sums<<<tiles, 1024, 0, s>>>(b.total, V, b.info, b.tsum);
      k_rs_hot_place<<<tiles, 1024, 0, s>>>(b.total, V, b.info, b.tsum, b.slot, b.hot_ids,
                                            b.start);
    }
    {
      ScopedTimer timer_(KID_RS_PLACE, s);
      k_rs_place<<<static_cast<unsigned>(q.nb), 256, 0, s>>>(
          idx, coef, N, K, q.rows_per_block, V, b.slot, b.hist, b.start, b.srow, b.sid, b.scoef);
    }
    const unsigned char* Hc = static_cast<const unsigned char*>(H);
    {
      ScopedTimer timer_(KID_RS_SLICES, s);
      const int64_t blocks = ceil_div(N * (d / 8), 256) < 65536 ? ceil_div(N * (d / 8), 256)
                                                                 : 65536;
      if (dtype == 1)
        k_rs_slices<BF16><<<static_cast<unsigned>(blocks), 256, 0, s>>>(Hc, N, d, b.hs);
      else
        k_rs_slices<F32><<<static_cast<unsigned>(blocks), 256, 0, s>>>(Hc, N, d, b.hs);
    }
    {
      ScopedTimer timer_(KID_RS_CHUNKS, s);
      // persistent: four workgroups per CU (256 CUs), fewer when there are
      // fewer (slice, chunk) items than that, a multiple of the 8 XCDs
      int64_t grid = round_up(q.nslices, 8) * q.nchunks;
      if (grid > 8 * 128) grid = 8 * 128;
      const size_t lds = (kWalkGroups * 2 * kRenormSliceCols + 3 * q.seg) * 4;
      if (dtype == 1)
        k_rs_chunks<BF16><<<static_cast<unsigned>(grid), 256, lds, s>>>(
            b.hs, b.srow, b.sid, b.scoef, b.start, N, V, d, q.seg, q.nslices, acc_out, gw,
            b.partial);
      else
        k_rs_chunks<F32><<<static_cast<unsigned>(grid), 256, lds, s>>>(
            b.hs, b.srow, b.sid, b.scoef, b.start, N, V, d, q.seg, q.nslices, acc_out, gw,
            b.partial);
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
    {
      ScopedTimer timer_(KID_RS_HOT, s);
      const unsigned grid = static_cast<unsigned>(ceil_div(nr, 4));
      const size_t lds = static_cast<size_t>(4) * (K + q.hot_max) * 4;
      if (dtype == 1)
        k_rs_hot_coef<BF16><<<grid, 256, lds, s>>>(idx, coef, b.slot, r0, nr, K, q.hot_max,
                                                   b.hot_c);
      else
        k_rs_hot_coef<F32><<<grid, 256, lds, s>>>(idx, coef, b.slot, r0, nr, K, q.hot_max,
                                                  b.hot_c);
    }
    launch_grad_w_split(dtype, b.hot_c, q.hot_max, H, d, q.hot_max, q.hot_max, r0, nr,
                        q.hot_splits, r0 > 0, b.hot_prod, q.hot_max * d, s);
  }
  ScopedTimer timer_(KID_RS_HOT, s);
  k_rs_hot_rows<<<static_cast<unsigned>(q.hot_max), 256, 0, s>>>(
      b.hot_ids, b.info, b.hot_prod, d, q.hot_splits, q.hot_max * d, acc_out, gw);
}

}  // namespace fkl
