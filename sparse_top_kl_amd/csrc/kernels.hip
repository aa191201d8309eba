// Kernels of the fused chunked top-K KL loss for gfx950.
//
// Method: "Multiverse Computing ... (iitak.ru)", third paragraph, and
// "Wissensdestillation mit deutlich weniger GPU-Speicher", section
// "KL-Verlust wird in Blöcken berechnet": the output projection is fused into
// the loss, rows are processed block by block without keeping their logits,
// and the backward pass recomputes them. Temperature and the T^2 factor:
// "Дистилляция и сжатие моделей", section "Как это работает: мягкие метки и
// температура".
//
// Forward, per chunk of rows:
//   k_logits_lse   z tile (MFMA) -> per (128-vocab slice, row) running max and
//                  sum of 2^(z * log2(e)/T); z never leaves registers.
//   k_merge_loss   merge the slices into lse, teacher softmax over the K cached
//                  logits, per-row KL.
// once: k_gather_dot (z at the teacher ids), k_reduce_loss (fixed-order sum).
// Backward, per block of rows (as many as the chunk x V budget allows) and,
// inside it, per vocabulary slice:
//   k_bwd_prep     (per row block) teacher probabilities scaled by s*T, lse in
//                  base 2.
//   k_gprod        recompute the z tile (same tile code as the forward) and
//                  write the dense part of the logit gradient,
//                  s*T*sum(p)*softmax, rounded once into the G block.
//   k_fixup        subtract s*T*p at the teacher ids inside the slice
//                  (recomputing the same value from z at the id, so each entry
//                  is rounded once).
//   k_grad_hidden  MFMA product G . W_slice, accumulated over the slices into
//                  an fp32 accumulator of the row block;
//   k_reduce_gh    (per row block) accumulator -> grad_hidden rows.
//   k_grad_w       MFMA product G^T . H_block into the fp32 grad_W rows of the
//                  slice, accumulated over the row blocks.
// Loss options (per-row weights, hard labels mixed in with alpha) change the
// per-row coefficients (k_merge_loss, k_bwd_prep), add a second set of LSE
// partials at temperature 1 when T != 1 (k_logits_lse<..., CE2>) and a second
// softmax term to the G producers (GradValue<CE2>), and the label entry to the
// exact entries (k_fixup, k_g_from_z).
// Forward-chunked variant (the logits are kept instead of recomputed):
//   k_logits_lse<..., KEEP>  also stores the tile's logits in the input dtype;
//   k_g_from_z               turns a kept row into its G row in place;
//   then k_grad_hidden over all rows and k_grad_w over row blocks.
// The teacher top-K cache kernels are in topk.hip; helpers shared with them
// are in device_common.hpp.
#include <math.h>

#include <cstdlib>
#include <type_traits>

#include "device_common.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace fkl {

// out (+)= v for an fp32 output element that receives exactly one
// contribution per launch (launches on one stream are ordered), so the sum is
// the same as a read-modify-write but the wave never waits for the old value:
// the add is a fire-and-forget atomic performed in L2.
__device__ __forceinline__ void accumulate_out(float* p, float v, int accumulate) {
  if (accumulate)
    (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// ------------------------------------------------------------------ forward

template <class P>
__device__ __forceinline__ void store4(unsigned char* p, const float (&v)[4]) {
  if constexpr (P::kBytes == 2) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Values the logit-tile kernels write per accumulator element (a raw logit z
// of token `tok` at output column `col`): row() loads what a token row needs,
// the call operator gives the value.
struct LogitValue {  // z itself, zero in the padding columns >= vlim
  int64_t vlim;
  struct Row {};
  __device__ __forceinline__ Row row(int64_t) const { return Row{}; }
  __device__ __forceinline__ float value(const Row&, float z) const { return z; }
  __device__ __forceinline__ float operator()(const Row& r, float z, int64_t col) const {
    return col < vlim ? value(r, z) : 0.f;
  }
};
// Dense part of the logit gradient, acoef * 2^(z*c2 - lse2), plus with CE2
// the separate temperature-1 softmax of the cross-entropy term,
// bcoef * 2^(z*log2(e) - lse1_2).
template <bool CE2>
struct GradValue {
  const float* acoef;
  const float* lse2;
  const float* bcoef;
  const float* lse1_2;
  float c2;
  int64_t vlim;   // columns >= vlim lie past the vocabulary (written as zero)
  int64_t nrows;  // tokens of the block
  struct Row {
    float a, l2, b, l1;
  };
  __device__ __forceinline__ Row row(int64_t tok) const {
    if (tok >= nrows) return Row{0.f, 0.f, 0.f, 0.f};
    if constexpr (CE2) return Row{acoef[tok], lse2[tok], bcoef[tok], lse1_2[tok]};
    return Row{acoef[tok], lse2[tok], 0.f, 0.f};
  }
  __device__ __forceinline__ float value(const Row& r, float z) const {
    float g = r.a * fast_exp2(z * c2 - r.l2);
    if constexpr (CE2) g += r.b * fast_exp2(z * kLog2e - r.l1);
    return g;
  }
  __device__ __forceinline__ float operator()(const Row& r, float z, int64_t col) const {
    return col < vlim ? value(r, z) : 0.f;
  }
};

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// Writes f(z) for the wave's sub-tile of a logit tile (accumulator rows =
// output columns w0.., accumulator columns = tokens t0..) into Out[token][column]
// (row pitch out_ld bytes), for tokens < nrows and columns < ncols; f gives 0
// at columns >= f.vlim. Called by every thread of the workgroup after the
// k-loop. NT marks the stores nontemporal (data not read again soon). hook()
// runs before the global stores are issued (loads placed there overlap them).
template <class P, class C, bool NT = false, class F, class Hook = NoHook>
__device__ __forceinline__ void store_token_rows(const f32x16_t (&acc)[C::kMI][C::kNI], const F& f,
                                                 int64_t w0, int64_t t0, int64_t nrows,
                                                 int64_t ncols, unsigned char* __restrict__ out,
                                                 int64_t out_ld, const Hook& hook = Hook{}) {
  const int lane = threadIdx.x & 63;
  if constexpr (P::kBytes == 2) {
    // A lane holds 4 consecutive columns of one token, so direct stores would
    // put 16 bytes into each of 32 output rows per instruction. Each wave
    // instead transposes its 128 x 64 sub-tile through 16 KiB of the (now
    // idle) stage LDS, laid out [token][column] in 256-byte rows, and writes 16
    // bytes per lane, 16 lanes per contiguous row segment. The 16-byte unit u
    // of row t sits at unit u ^ (t % 16), its 8-byte halves swapped when bit 4
    // of t is set, so the 32 rows one write instruction touches hit 32
    // distinct 8-byte bank positions.
    static_assert(C::kWM == 128 && C::kWN == 64, "transpose layout of the eight-wave tile");
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    __syncthreads();  // every wave has drained its loads: the stage LDS is free
    const int w = static_cast<int>(threadIdx.x >> 6);
    const auto st = PingPongLoop<C, false, false>::stage_arrays();
    // an LDS-space pointer, so the staging uses ds_write / ds_read
    lds_u8* const tp = (lds_u8*)(w < 4 ? st.s[0] : st.s[1]) +
                       (w & 3) * (kDStageBytes / 4);
    // Sub-tiles whose columns all lie below f.vlim (all but the vocabulary's
    // last) skip the per-element column test.
    auto fill = [&](auto all_cols) {
      constexpr bool kAll = decltype(all_cols)::value;
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni) {
        const int tl = ni * 32 + (lane & 31);
        const typename F::Row rw = f.row(t0 + tl);
        const int half = (lane >> 5) ^ ((tl >> 4) & 1);
#pragma unroll
        for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int64_t col = w0 + mi * 32 + 8 * g4 + 4 * (lane >> 5);
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              v[j] = kAll ? f.value(rw, acc[mi][ni][4 * g4 + j]) : f(rw, acc[mi][ni][4 * g4 + j], col + j);
            const int unit = (mi * 4 + g4) ^ (tl & 15);
            *(__attribute__((address_space(3))) u32x2_t*)(tp + tl * 256 + unit * 16 + half * 8) =
                u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
      }
    };
    if (w0 + C::kWM <= f.vlim)
      fill(std::true_type{});
    else
      fill(std::false_type{});
    hook();
    if (w0 >= ncols) return;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int tl = it * 4 + (lane >> 4), u = lane & 15;
      u32x4_t x = *(const __attribute__((address_space(3))) u32x4_t*)(tp + tl * 256 + (u ^ (tl & 15)) * 16);
      if ((tl >> 4) & 1) x = u32x4_t{x[2], x[3], x[0], x[1]};
      const int64_t tok = t0 + tl, col = w0 + u * 8;
      if (tok < nrows && col < ncols) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + tok * out_ld + col * P::kBytes);
        if constexpr (NT)
          __builtin_nontemporal_store(x, dst);
        else
          *dst = x;
      }
    }
    return;
  }
  hook();
  if (w0 >= ncols) return;
#pragma unroll
  for (int ni = 0; ni < C::kNI; ++ni) {
    const int64_t tok = t0 + ni * 32 + (lane & 31);
    if (tok >= nrows) continue;
    const typename F::Row rw = f.row(tok);
    unsigned char* orow = out + tok * out_ld;
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int64_t col = w0 + mi * 32 + 8 * g4 + 4 * (lane >> 5);
        if (col >= ncols) continue;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = f(rw, acc[mi][ni][4 * g4 + j], col + j);
        store4<P>(orow + col * P::kBytes, v);
      }
  }
}


// ------------------------------------------------------------------ pair index

constexpr int kPairThreads = 1024;

__device__ __forceinline__ uint32_t pack_pair(int k, int tl, int32_t v) {
  return static_cast<uint32_t>(k) | (static_cast<uint32_t>(tl) << 13) |
         (static_cast<uint32_t>(v & 2047) << 21);
}

// One workgroup per row tile t (rows 256 t .. 256 t + 255 below N): counts its
// pairs per vocabulary bucket in LDS, scans the counts into start[t], then
// places each pair at its bucket's cursor. Pairs without a valid id get z = 0
// in zk / zy (when those are given) and no entry.
__global__ __launch_bounds__(kPairThreads) void k_pair_index(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ labels, int64_t N, int K,
    int64_t V, int bw_log2, int64_t n_vb, int32_t* __restrict__ start,
    uint32_t* __restrict__ entry, int64_t cap, float* __restrict__ zk, float* __restrict__ zy) {
  __shared__ int32_t cnt[kPairMaxBuckets];
  __shared__ int32_t wsum[kPairThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 256;
  const int rows = static_cast<int>(N - r0 < 256 ? N - r0 : 256);
  const int Kp = K + (labels ? 1 : 0);
  const int npairs = rows * Kp;
  const int nb = static_cast<int>(n_vb);
  for (int b = tid; b < nb; b += kPairThreads) cnt[b] = 0;
  __syncthreads();
  for (int p = tid; p < npairs; p += kPairThreads) {
    const int rl = p / Kp, k = p - rl * Kp;
    const int64_t r = r0 + rl;
    const int32_t v = k < K ? idx[r * K + k] : labels[r];
    if (v >= 0 && v < V)
      atomicAdd(&cnt[v >> bw_log2], 1);
    else if (k < K) {
      if (zk) zk[r * K + k] = 0.f;
    } else if (zy) {
      zy[r] = 0.f;
    }
  }
  __syncthreads();
  // exclusive scan of cnt[0, nb): each thread takes a run of consecutive
  // buckets; runs are scanned across the wave, then across the waves
  const int per = (nb + kPairThreads - 1) / kPairThreads;
  const int b0 = tid * per, b1 = b0 + per < nb ? b0 + per : nb;
  int run = 0;
  for (int b = b0; b < b1; ++b) run += cnt[b];
  int x = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < w; ++i) wbase += wsum[i];
  int acc = wbase + x - run;
  int32_t* st = start + static_cast<int64_t>(blockIdx.x) * (n_vb + 1);
  for (int b = b0; b < b1; ++b) {
    const int c = cnt[b];
    cnt[b] = acc;
    st[b] = acc;
    acc += c;
  }
  if (tid == kPairThreads - 1) st[nb] = wbase + x;  // all pairs of the tile
  __syncthreads();
  uint32_t* ent = entry + static_cast<int64_t>(blockIdx.x) * cap;
  for (int p = tid; p < npairs; p += kPairThreads) {
    const int rl = p / Kp, k = p - rl * Kp;
    const int64_t r = r0 + rl;
    const int32_t v = k < K ? idx[r * K + k] : labels[r];
    if (v >= 0 && v < V) ent[atomicAdd(&cnt[v >> bw_log2], 1)] = pack_pair(k, rl, v);
  }
}

// The teacher-id pairs of one logit tile: rows [g_lo, g_hi) of the batch (at
// most 256, tile columns tl = r - g_lo) and ids [va, vb) (vb - va <= 256,
// c = v - va). The buckets overlapping [va, vb) span fewer than 2048 ids, so
// an entry's low 11 id bits fix its id. The entry ranges of the tile's (at
// most two) row tiles are read when the kernel starts, so that their latency
// hides behind the k-loop; after the loop each thread loads one pair; pairs
// beyond one per thread (tiles of very frequent ids only) are read from memory
// as they are visited.
struct TilePairs {
  int64_t g_lo, g_hi, va, vb, gt0;
  int32_t raw[4];  // range bounds as loaded: [start, end) in the first and second row tile
  bool two;        // the rows span a second row tile
  int32_t e0[2];   // first entry of the range in each row tile   (set after the loop)
  int32_t n0, n;   // pairs in the first row tile's range; in both (set after the loop)
  uint32_t mine;   // this thread's pair: bit 31 set, k | tl << 13 | c << 21; else 0
};

// Issues the loads of the range bounds only: nothing uses them before the
// k-loop has run, so their latency is not waited for at the start.
__device__ __forceinline__ TilePairs tile_pairs_begin(const PairIndex& pi, int64_t g_lo,
                                                      int64_t g_hi, int64_t va, int64_t vb) {
  TilePairs tp;
  tp.g_lo = g_lo;
  tp.g_hi = g_hi;
  tp.va = va;
  tp.vb = vb;
  tp.gt0 = g_lo >> 8;
  tp.mine = 0u;
  const bool empty = g_hi <= g_lo || vb <= va;
  tp.two = !empty && ((g_hi - 1) >> 8) != tp.gt0;
  int64_t b0 = 0, b1 = 0;
  if (!empty) {
    b0 = va >> pi.bw_log2;
    b1 = ((vb - 1) >> pi.bw_log2) + 1;
    if (b1 > pi.n_vb) b1 = pi.n_vb;
  }
  // vector (buffer) loads: their results land in VGPRs that nothing touches
  // until after the loop (scalar loads were waited for at once to free SGPRs)
  const Operand st = make_operand(reinterpret_cast<const unsigned char*>(
                                      pi.start + tp.gt0 * (pi.n_vb + 1)),
                                  0, 0, 0);
  const uint32_t o1 = tp.two ? static_cast<uint32_t>((pi.n_vb + 1) * 4) : 0u;
  tp.raw[0] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(st.rsrc, b0 * 4, 0, 0));
  tp.raw[1] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(st.rsrc, b1 * 4, 0, 0));
  tp.raw[2] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(st.rsrc, o1 + b0 * 4, 0, 0));
  tp.raw[3] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(st.rsrc, o1 + b1 * 4, 0, 0));
  return tp;
}

// Pair i (0 <= i < tp.n) in the packed form, or 0 if it lies outside the tile.
__device__ __forceinline__ uint32_t tile_pair_at(const PairIndex& pi, const TilePairs& tp,
                                                 int32_t i) {
  const bool first = i < tp.n0;
  const int64_t gt = first ? tp.gt0 : tp.gt0 + 1;
  const uint32_t e = pi.entry[gt * pi.cap + (first ? tp.e0[0] + i : tp.e0[1] + (i - tp.n0))];
  const int64_t r = gt * 256 + ((e >> 13) & 0xffu);
  const int64_t c = (static_cast<int64_t>(e >> 21) - tp.va) & 2047;
  if (r < tp.g_lo || r >= tp.g_hi || tp.va + c >= tp.vb) return 0u;
  return 0x80000000u | (e & 0x1fffu) | (static_cast<uint32_t>(r - tp.g_lo) << 13) |
         (static_cast<uint32_t>(c) << 21);
}

// After the k-loop: the ranges, and thread t's pair.
__device__ __forceinline__ void tile_pairs_load(const PairIndex& pi, TilePairs& tp, int t) {
  tp.e0[0] = tp.raw[0];
  tp.n0 = tp.raw[1] - tp.raw[0];
  tp.e0[1] = tp.raw[2];
  tp.n = tp.n0 + (tp.two ? tp.raw[3] - tp.raw[2] : 0);
  tp.mine = t < tp.n ? tile_pair_at(pi, tp, t) : 0u;
}

__device__ __forceinline__ int pair_tl(uint32_t m) { return (m >> 13) & 0xffu; }
__device__ __forceinline__ int pair_k(uint32_t m) { return m & 0x1fffu; }
__device__ __forceinline__ int pair_c(uint32_t m) { return (m >> 21) & 0xffu; }

// f(m) for every pair m of the tile: thread t's own, then those beyond one
// per thread (threads t = 0 .. nth - 1 share them).
template <class F>
__device__ __forceinline__ void tile_pairs_each(const PairIndex& pi, const TilePairs& tp, int t,
                                                int nth, F&& f) {
  if (tp.mine) f(tp.mine);
  for (int32_t i = nth + t; i < tp.n; i += nth) {
    const uint32_t m = tile_pair_at(pi, tp, i);
    if (m) f(m);
  }
}

// The two 64 KiB halves of the idle k-loop LDS of a tile kernel (the
// instantiation the kernels' gemm_tile<P, C, false, false> uses).
template <class P, class C>
__device__ __forceinline__ void loop_lds_halves(unsigned char** lo, unsigned char** hi) {
  if constexpr (P::kBytes == 2) {
    const auto st = PingPongLoop<C, false, false>::stage_arrays();
    *lo = st.s[0];
    *hi = st.s[1];
  } else {
    unsigned char* l = TileLoop<P, C, false, false>::smem();
    *lo = l;
    *hi = l + 65536;
  }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// z at the teacher-id pairs inside a logit tile (TilePairs, the thread's own
// pair loaded): the pairs' positions are marked in a per-tile bitmap, the
// waves holding marked accumulators write them (in groups of four vocabulary
// rows) to an fp32 staging area [token][128 vocabulary] in the idle k-loop LDS,
// one vocabulary half at a time, and the pair's thread reads its value back
// and stores it: zk[r][k] (k < K) or zy[r] (k = K, the label).
template <class P, class C>
__device__ __forceinline__ void gather_tile_pairs(const f32x16_t (&acc)[C::kMI][C::kNI],
                                                  const PairIndex& pi, const TilePairs& tp,
                                                  float* __restrict__ zk, float* __restrict__ zy) {
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  __shared__ uint32_t bits[256 * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int nth = C::kThreads;
  unsigned char *glo, *ghi;
  loop_lds_halves<P, C>(&glo, &ghi);
  lds_u8* const stage_lo = (lds_u8*)glo;
  lds_u8* const stage_hi = (lds_u8*)ghi;
  for (int i = tid; i < 256 * 8; i += nth) bits[i] = 0u;
  __syncthreads();  // every wave has left the k-loop: its LDS is free
  tile_pairs_each(pi, tp, tid, nth, [&](uint32_t m) {
    const int c = pair_c(m);
    atomicOr(&bits[pair_tl(m) * 8 + (c >> 5)], 1u << (c & 31));
  });
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (C::wave_m() == h) {  // this wave holds tile rows 128 h .. 128 h + 127
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni) {
        const int tl = C::wave_n() * C::kWN + ni * 32 + (lane & 31);
        lds_u8* const row = (tl < 128 ? stage_lo : stage_hi) + (tl & 127) * 512;
#pragma unroll
        for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int vl = mi * 32 + 8 * g4 + 4 * (lane >> 5);  // row within the half
            const uint32_t word = bits[tl * 8 + h * 4 + (vl >> 5)];
            if ((word >> (vl & 31)) & 0xfu)
              *(__attribute__((address_space(3))) f32x4_t*)(row + vl * 4) =
                  f32x4_t{acc[mi][ni][4 * g4], acc[mi][ni][4 * g4 + 1], acc[mi][ni][4 * g4 + 2],
                          acc[mi][ni][4 * g4 + 3]};
          }
      }
    }
    __syncthreads();
    tile_pairs_each(pi, tp, tid, nth, [&](uint32_t m) {
      const int c = pair_c(m) - h * 128;
      if (c < 0 || c >= 128) return;
      const int tl = pair_tl(m), k = pair_k(m);
      const float z = *(const __attribute__((address_space(3))) float*)(
          (tl < 128 ? stage_lo : stage_hi) + (tl & 127) * 512 + c * 4);
      const int64_t r = tp.g_lo + tl;
      if (k < pi.K)
        zk[r * pi.K + k] = z;
      else
        zy[r] = z;
    });
    __syncthreads();
  }
}

// With KEEP the tile's logits are also written, rounded to the element type,
// into Z[token][v] (row pitch zld bytes) for v < zcols, as zero for v >= V
// (streaming stores: the backward reads them much later).
// With CE2 the partials at temperature 1 (c = log2(e)) go to part_ce as well.
// With pi.entry non-null, z at the teacher-id pairs of the tile goes to zk /
// zy (gather_tile_pairs); row0 is the batch row of the chunk's first row.
template <class P, class C, bool KEEP, bool CE2>
__global__ __launch_bounds__(C::kThreads) FKL_WAVES_PER_EU(C) void k_logits_lse(
    const unsigned char* __restrict__ W, const unsigned char* __restrict__ H, int64_t d, int64_t V,
    int64_t nrows, int64_t n_vt, int64_t n_tt, float c2, float2* __restrict__ part,
    int64_t part_ld, float2* __restrict__ part_ce, unsigned char* __restrict__ Z, int64_t zld,
    int64_t zcols, PairIndex pi, int64_t row0, float* __restrict__ zk, float* __restrict__ zy) {
  static_assert(C::kWM == kSliceVocab, "one LSE partial per wave row-slice");
  int64_t vt, tt;
  if (!TileGroups<4, 8>::coords(n_vt, n_tt, &vt, &tt)) return;
  const int64_t ld = d * P::kBytes;
  TilePairs tp;
  if (pi.entry) {
    const int64_t va = vt * kBM, ntok = nrows - tt * kBN < kBN ? nrows - tt * kBN : kBN;
    tp = tile_pairs_begin(pi, row0 + tt * kBN, row0 + tt * kBN + ntok, va,
                          va + kBM < V ? va + kBM : V);
  }
  // MFMA rows = vocabulary entries (weight rows), columns = tokens, so each
  // lane's accumulators belong to one token and the reduction over the
  // vocabulary is mostly in-lane.
  const Operand A = make_operand(W + vt * kBM * ld, ld, V - vt * kBM, d);
  const Operand B = make_operand(H + tt * kBN * ld, ld, nrows - tt * kBN, d);
  f32x16_t acc[C::kMI][C::kNI];
  gemm_tile<P, C, false, false>(acc, A, B, static_cast<int>(d));
  if (pi.entry) tile_pairs_load(pi, tp, static_cast<int>(threadIdx.x));

  const int64_t v0 = vt * kBM + C::wave_m() * C::kWM;
  if (v0 < V) {
    lse_partials<C>(acc, v0, V, tt * kBN + C::wave_n() * C::kWN, nrows, c2, part, part_ld);
    if constexpr (CE2)
      lse_partials<C>(acc, v0, V, tt * kBN + C::wave_n() * C::kWN, nrows, kLog2e, part_ce,
                      part_ld);
  }
  if (pi.entry) gather_tile_pairs<P, C>(acc, pi, tp, zk, zy);
  if constexpr (KEEP)
    store_token_rows<P, C, true>(acc, LogitValue{V}, v0, tt * kBN + C::wave_n() * C::kWN, nrows, zcols,
                           Z, zld);
}

template <class P>
__device__ __forceinline__ float dot16(u32x4_t a, u32x4_t b, float acc) {
  if constexpr (P::kBytes == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(as_f32(a[e] << 16), as_f32(b[e] << 16), acc);
      acc = fmaf(as_f32(a[e] & 0xffff0000u), as_f32(b[e] & 0xffff0000u), acc);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = fmaf(as_f32(a[e]), as_f32(b[e]), acc);
  }
  return acc;
}

// One wave per row; four 16-lane groups take every fourth teacher id and
// stream that weight row. With STAGE the block's four hidden rows are first
// copied to LDS (each is read once per id), otherwise read from memory.
template <class P, bool STAGE>
__global__ __launch_bounds__(256) void k_gather_dot(const unsigned char* __restrict__ W,
                                                    const unsigned char* __restrict__ H,
                                                    const int32_t* __restrict__ idx, int64_t d,
                                                    int64_t nrows, int K, float* __restrict__ zk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sh_rows[];
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int64_t rb = d * P::kBytes;
  const int64_t nvec = rb / 16;
  const unsigned char* h = H + row * rb;
  if constexpr (STAGE) {
    unsigned char* hs = sh_rows + (threadIdx.x >> 6) * rb;  // this wave's row
    for (int64_t j = lane; j < nvec; j += 64) lds_store16(hs + j * 16, load16(h + j * 16));
    h = hs;  // each wave reads back only what it wrote: no barrier needed
  }
  for (int k = g; k < K; k += 4) {
    const int64_t v = idx[row * K + k];
    if (v < 0) {  // no id (a row without a hard label)
      if (li == 0) zk[row * K + k] = 0.f;
      continue;
    }
    const unsigned char* wr = W + v * rb;
    // four independent loads and partial sums in flight per lane
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int64_t j = li;
    for (; j + 48 < nvec; j += 64) {
      const u32x4_t w0 = load16(wr + j * 16), w1 = load16(wr + (j + 16) * 16);
      const u32x4_t w2 = load16(wr + (j + 32) * 16), w3 = load16(wr + (j + 48) * 16);
      a0 = dot16<P>(STAGE ? lds_load16(h + j * 16) : load16(h + j * 16), w0, a0);
      a1 = dot16<P>(STAGE ? lds_load16(h + (j + 16) * 16) : load16(h + (j + 16) * 16), w1, a1);
      a2 = dot16<P>(STAGE ? lds_load16(h + (j + 32) * 16) : load16(h + (j + 32) * 16), w2, a2);
      a3 = dot16<P>(STAGE ? lds_load16(h + (j + 48) * 16) : load16(h + (j + 48) * 16), w3, a3);
    }
    for (; j < nvec; j += 16) {
      const u32x4_t hv = STAGE ? lds_load16(h + j * 16) : load16(h + j * 16);
      a0 = dot16<P>(hv, load16(wr + j * 16), a0);
    }
    float acc = (a0 + a1) + (a2 + a3);
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (li == 0) zk[row * K + k] = acc;
  }
}

// The loss of one row of the chunk given its lse at T and at temperature 1
// (called by one whole wave): the teacher softmax over the K entries, the
// row's KL term and, with labels, its cross-entropy; row_loss = w (a_kl T^2 KL
// + a_ce CE). zk, logit, lse_out and row_loss start at the chunk's first row;
// the option arrays are indexed by absolute row (row0 + row).
__device__ __forceinline__ void merge_row_loss(const float* __restrict__ zk,
                                               const float* __restrict__ logit, int64_t row0,
                                               int64_t row, int K, float T, float lse, float lse1,
                                               float* __restrict__ lse_out,
                                               float* __restrict__ row_loss, const MergeOpts& o,
                                               int lane) {
  const int64_t ar = row0 + row;
  const float w = o.row_weight ? o.row_weight[ar] : 1.0f;
  float term = 0.f;
  if (w != 0.f) {  // uniform per wave; a weight-0 (padding) row may lack teacher entries
    const float invT = 1.0f / T;
    const float* lg = logit + row * K;
    const float* z = zk + row * K;
    // log p_k = lg/T - logZ: renormalised over the K entries, or (tail bucket)
    // the cached ids' share of the teacher's full distribution
    float logZ;
    if (o.teacher_lse) {
      logZ = o.teacher_lse[ar];
    } else {
      float ma = -INFINITY;
      for (int k = lane; k < K; k += 64) ma = fmaxf(ma, lg[k] * invT);
      ma = wave_max(ma);
      float zsum = 0.f;
      for (int k = lane; k < K; k += 64) zsum += expf(lg[k] * invT - ma);
      logZ = ma + logf(wave_sum(zsum));
    }
    float psum = 0.f, S = 0.f;
    for (int k = lane; k < K; k += 64) {
      const float lp = lg[k] * invT - logZ;
      const float p = expf(lp);
      const float lq = z[k] * invT - lse;
      if (p > 0.f) term += p * (lp - lq);
      psum += p;
      S += expf(lq);
    }
    term = wave_sum(term);
    if (o.teacher_lse) {  // the tail bucket: p_tail (log p_tail - log(1 - S))
      psum = wave_sum(psum);
      S = wave_sum(S);
      const float pt = fmaxf(0.f, 1.f - psum);
      if (pt > 0.f) term += pt * (logf(pt) - log1pf(-fminf(S, 1.f - 1e-7f)));
    }
  }
  if (lane == 0) {
    lse_out[row] = lse;
    if (o.lse1) o.lse1[ar] = lse1;
    float ce = 0.f;
    if (o.labels && o.labels[ar] >= 0) ce = lse1 - o.zy[ar];
    if (row_loss) row_loss[row] = w != 0.f ? w * (o.a_kl * T * T * term + o.a_ce * ce) : 0.f;
  }
}

// Rows per k_merge_loss block: 16 consecutive rows share each 128-byte line of
// the [slot][row] partials, so the merge reads whole lines.
constexpr int kMergeRows = 16;

// Per row of the chunk: lse at T (and at temperature 1 with partials there)
// from the (vocabulary slice, row) partials, then the row's loss. A block of
// 16 waves takes 16 rows: in the merge, lane (sub, r) of wave wv reads slots
// 4 wv + sub + 64 j of row r, four loads in flight; the four subs of a wave,
// then the 16 waves, are merged in a fixed order. Then wave wv computes the
// loss of row wv.
constexpr int kMergeWaves = 16;

__global__ __launch_bounds__(64 * kMergeWaves) void k_merge_loss(
    const float2* __restrict__ part, int64_t part_ld, int64_t nslots,
    const float* __restrict__ zk, const float* __restrict__ logit, int64_t row0, int64_t nrows,
    int K, float T, float* __restrict__ lse_out, float* __restrict__ row_loss, MergeOpts o) {
  __shared__ float2 red[2][kMergeWaves][kMergeRows];
  __shared__ float s_lse[2][kMergeRows];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t rb = static_cast<int64_t>(blockIdx.x) * kMergeRows;
  {
    const int r = lane & 15, sub = lane >> 4;
    const bool valid = rb + r < nrows;
    constexpr int kStride = 4 * kMergeWaves;
    for (int t = 0; t < (o.part_ce ? 2 : 1); ++t) {
      const float2* P = t ? o.part_ce : part;
      float m = -INFINITY, sm = 0.f;
      if (valid) {
        for (int64_t sl = 4 * wv + sub; sl < nslots; sl += 4 * kStride) {
          float2 q[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            q[u] = sl + u * kStride < nslots ? P[(sl + u * kStride) * part_ld + rb + r]
                                             : make_float2(-INFINITY, 0.f);
#pragma unroll
          for (int u = 0; u < 4; ++u) merge_ms(m, sm, q[u].x, q[u].y);
        }
      }
#pragma unroll
      for (int x = 16; x <= 32; x <<= 1) {
        const float mo = __shfl_xor(m, x), so = __shfl_xor(sm, x);
        merge_ms(m, sm, mo, so);
      }
      if (sub == 0) red[t][wv][r] = make_float2(m, sm);
    }
  }
  __syncthreads();
  if (threadIdx.x < 2 * kMergeRows) {
    const int t = threadIdx.x / kMergeRows, r = threadIdx.x % kMergeRows;
    float m = -INFINITY, sm = 0.f;
    for (int i = 0; i < kMergeWaves; ++i) merge_ms(m, sm, red[t][i][r].x, red[t][i][r].y);
    s_lse[t][r] = (m + log2f(sm)) * kLn2;
  }
  __syncthreads();
  const int64_t row = rb + wv;
  if (row < nrows)
    merge_row_loss(zk, logit, row0, row, K, T, s_lse[0][wv], o.part_ce ? s_lse[1][wv] : s_lse[0][wv],
                   lse_out, row_loss, o, lane);
}


__global__ __launch_bounds__(1024) void k_reduce_loss(const float* __restrict__ row_loss, int64_t N,
                                                      float* __restrict__ loss) {
  __shared__ double sh[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) acc += static_cast<double>(row_loss[i]);
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = static_cast<float>(sh[0]);
}

// ------------------------------------------------------------------ backward

// One wave (workgroup) per row, coefficients of its logit gradient with s the
// upstream scale, w the row weight and y the label:
//   pcoef_k = s w a_kl T p_k,  ycoef = s w a_ce [y >= 0],
//   acoef = s w a_kl T sum_k p_k (+ ycoef when the cross-entropy shares the
//   softmax, i.e. T = 1), bcoef = ycoef when it has its own (two_sm),
//   lse2 = lse log2(e), lse1_2 = lse1 log2(e).
// With sub / tmul (row pitch K + 1; dynamic LDS of 8 K bytes) also the
// constants of the exact entries at the row's pairs: for entry k with id v,
//   sub_k = sum of pcoef over the entries with id v (+ ycoef if v = y),
//   tmul_k = tcoef x (number of entries with id v);
// for the label (entry K): sub = ycoef, tmul = 0, or NaN when y is also a
// teacher id (those entries then carry it).
// logit, lse, idx and the outputs start at the block's first row; row_weight,
// labels and lse1 are indexed by absolute row (row0 + row).
__global__ __launch_bounds__(64) void k_bwd_prep(
    const float* __restrict__ logit, const float* __restrict__ lse,
    const float* __restrict__ grad_loss, int64_t row0, int64_t nrows, int K, float T,
    const float* __restrict__ row_weight, const int32_t* __restrict__ labels, float a_kl,
    float a_ce, const float* __restrict__ lse1, bool two_sm,
    const float* __restrict__ teacher_lse, const float* __restrict__ zk,
    float* __restrict__ pcoef, float* __restrict__ acoef, float* __restrict__ lse2,
    float* __restrict__ bcoef, float* __restrict__ lse1_2, float* __restrict__ ycoef,
    float* __restrict__ tcoef, const int32_t* __restrict__ idx, float* __restrict__ sub,
    float* __restrict__ tmul) {
  extern __shared__ int32_t sh_prep[];
  int32_t* sid = sh_prep;
  float* sp = reinterpret_cast<float*>(sh_prep + K);
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  if (row >= nrows) return;
  const int64_t ar = row0 + row;
  const float s = grad_loss ? *grad_loss : 1.0f;
  const float w = row_weight ? row_weight[ar] : 1.0f;
  const bool has_y = labels && labels[ar] >= 0;
  const float yc = has_y ? s * w * a_ce : 0.f;
  const float scale = s * w * a_kl * T;
  float psum = 0.f, tail = 0.f, tc = 0.f;
  if (w != 0.f) {
    const float invT = 1.0f / T;
    const float* lg = logit + row * K;
    float logZ;  // as in k_merge_loss
    if (teacher_lse) {
      logZ = teacher_lse[ar];
    } else {
      float ma = -INFINITY;
      for (int k = lane; k < K; k += 64) ma = fmaxf(ma, lg[k] * invT);
      ma = wave_max(ma);
      float zsum = 0.f;
      for (int k = lane; k < K; k += 64) zsum += expf(lg[k] * invT - ma);
      logZ = ma + logf(wave_sum(zsum));
    }
    float S = 0.f;
    for (int k = lane; k < K; k += 64) {
      const float p = expf(lg[k] * invT - logZ);
      psum += p;
      pcoef[row * K + k] = scale * p;
      if (sub) sp[k] = scale * p;
      if (teacher_lse) S += expf(zk[row * K + k] * invT - lse[row]);
    }
    psum = wave_sum(psum);
    if (teacher_lse) {
      // tail bucket: d/dz of p_tail (log p_tail - log(1 - S)) is
      // T p_tail (Q - q S) / (1 - S): the dense coefficient loses
      // p_tail S / (1 - S), each cached id gains p_tail / (1 - S)
      S = wave_sum(S);
      const float pt = fmaxf(0.f, 1.f - psum);
      const float inv = 1.f / fmaxf(1.f - S, 1e-7f);
      tail = pt * S * inv;
      tc = scale * pt * inv;
    }
  } else {
    for (int k = lane; k < K; k += 64) {
      pcoef[row * K + k] = 0.f;
      if (sub) sp[k] = 0.f;
    }
  }
  if (lane == 0) {
    acoef[row] = scale * (psum - tail) + (two_sm ? 0.f : yc);
    if (tcoef) tcoef[row] = tc;
    lse2[row] = lse[row] * kLog2e;
    if (bcoef) bcoef[row] = two_sm ? yc : 0.f;
    if (lse1_2) lse1_2[row] = two_sm ? lse1[ar] * kLog2e : 0.f;
    if (ycoef) ycoef[row] = yc;
  }
  if (sub) {
    const int Kp = K + 1;
    const int32_t y = has_y ? labels[ar] : -1;
    for (int k = lane; k < K; k += 64) sid[k] = idx[row * K + k];
    // the wave's LDS writes are visible to its own later reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bool found = false;  // y is one of the row's ids
    for (int k = lane; k < K; k += 64) {
      const int32_t v = sid[k];
      found |= v == y;
      float ps = 0.f, m = 0.f;
      int k2 = 0;
      for (; k2 + 4 <= K; k2 += 4) {  // K is a multiple of 4 only by chance: tail below
        int32_t ids[4];
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ids[u] = sid[k2 + u];
          pv[u] = sp[k2 + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ps += ids[u] == v ? pv[u] : 0.f;
          m += ids[u] == v ? 1.f : 0.f;
        }
      }
      for (; k2 < K; ++k2) {
        const bool eq = sid[k2] == v;
        ps += eq ? sp[k2] : 0.f;
        m += eq ? 1.f : 0.f;
      }
      sub[row * Kp + k] = ps + (v == y ? yc : 0.f);
      tmul[row * Kp + k] = tc * m;
    }
    found = __any(found);
    if (lane == 0) {
      sub[row * Kp + K] = found ? __builtin_nanf("") : yc;
      tmul[row * Kp + K] = 0.f;
    }
  }
}

// Recompute the logit tile of rows [0, nrows) x vocabulary [v0, v0 + Vw) and
// write the dense part of G (GradValue) into the G block G[row][v - v0]
// (row pitch gpitch elements; entries with v >= V are written as zero).
// Dense part of G at one logit for one row's coefficients.
struct DenseCoef {
  float a, l2, b, l1;
};
__device__ __forceinline__ DenseCoef row_dense(const RowCoef& rc, int64_t row) {
  return DenseCoef{rc.acoef[row], rc.lse2[row], rc.bcoef ? rc.bcoef[row] : 0.f,
                   rc.lse1_2 ? rc.lse1_2[row] : 0.f};
}
__device__ __forceinline__ float dense_g(const DenseCoef& c, float z, float c2) {
  float g = c.a * fast_exp2(z * c2 - c.l2);
  if (c.b != 0.f) g += c.b * fast_exp2(z * kLog2e - c.l1);
  return g;
}

template <class P>
__device__ __forceinline__ void store_one(unsigned char* grow, int64_t col, float val) {
  if constexpr (P::kBytes == 2)
    reinterpret_cast<uint16_t*>(grow)[col] = f32_to_bf16_rne(val);
  else
    reinterpret_cast<float*>(grow)[col] = val;
}

// With pp.pi.entry non-null, after the tile's dense entries have been stored,
// the exact entries at the teacher-id and label pairs of the tile overwrite
// them (PairPatch; each entry is rounded once, from the gathered fp32 logit).
// row0 is the batch row of the block's first row.
template <class P, class C, bool CE2>
__global__ __launch_bounds__(C::kThreads) FKL_WAVES_PER_EU(C) void k_gprod(
    const unsigned char* __restrict__ W, const unsigned char* __restrict__ H, int64_t d, int64_t V,
    int64_t v0, int64_t Vw, int64_t gpitch, int64_t nrows, int64_t n_vt, int64_t n_tt, float c2,
    RowCoef rc, unsigned char* __restrict__ G, int64_t row0, PairPatch pp) {
  int64_t vt, tt;
  if (!TileGroups<4, 8>::coords(n_vt, n_tt, &vt, &tt)) return;
  const int64_t ld = d * P::kBytes;
  const int64_t vbase = v0 + vt * kBM;  // first vocabulary entry of the tile
  TilePairs tp;
  if (pp.pi.entry) {
    int64_t vb = vbase + kBM;
    if (vb > v0 + Vw) vb = v0 + Vw;
    if (vb > V) vb = V;
    const int64_t ntok = nrows - tt * kBN < kBN ? nrows - tt * kBN : kBN;
    tp = tile_pairs_begin(pp.pi, row0 + tt * kBN, row0 + tt * kBN + ntok, vbase, vb);
  }
  const Operand A = make_operand(W + vbase * ld, ld, V - vbase, d);
  const Operand B = make_operand(H + tt * kBN * ld, ld, nrows - tt * kBN, d);
  f32x16_t acc[C::kMI][C::kNI];
  gemm_tile<P, C, false, false>(acc, A, B, static_cast<int>(d));
  if (pp.pi.entry) tile_pairs_load(pp.pi, tp, static_cast<int>(threadIdx.x));

  const int64_t w0 = vt * kBM + C::wave_m() * C::kWM;  // slice-relative column of the wave
  const int64_t t0 = tt * kBN + C::wave_n() * C::kWN;  // first token of the wave
  const GradValue<CE2> f{rc.acoef, rc.lse2, rc.bcoef, rc.lse1_2, c2, V - v0, nrows};
  if (!pp.pi.entry) {
    store_token_rows<P, C>(acc, f, w0, t0, nrows, Vw, G, gpitch * P::kBytes);
    return;
  }
  // Exact entries at the tile's pairs: the values a pair needs are loaded
  // while the dense part is staged and written, and the exact entry replaces
  // the dense one once every dense store of the tile has completed (a thread's
  // stores complete in order; the wait and the barrier order them across the
  // workgroup).
  const int Kp = pp.pi.K + 1;
  struct Vals {
    float z, sub, tmul;
    DenseCoef dc;
  };
  auto vals = [&](uint32_t m) {
    const int64_t rb = tt * kBN + pair_tl(m);  // row of the block
    const int k = pair_k(m);
    return Vals{k < pp.pi.K ? pp.zk[rb * pp.pi.K + k] : pp.zy[rb], pp.sub[rb * Kp + k],
                pp.tmul[rb * Kp + k], row_dense(rc, rb)};
  };
  auto put = [&](uint32_t m, const Vals& x) {
    if (x.sub != x.sub) return;  // a label that is also a teacher id: its entries write it
    float g = dense_g(x.dc, x.z, c2) - x.sub;
    if (x.tmul != 0.f) g += x.tmul * fast_exp2(x.z * c2 - x.dc.l2);
    const int64_t rb = tt * kBN + pair_tl(m);
    store_one<P>(G + rb * gpitch * P::kBytes, vt * kBM + pair_c(m), g);
  };
  Vals mine{};
  store_token_rows<P, C>(acc, f, w0, t0, nrows, Vw, G, gpitch * P::kBytes, [&]() {
    if (tp.mine) mine = vals(tp.mine);
  });
  wait_vmcnt_lgkm0<0>();
  __syncthreads();
  if (tp.mine) put(tp.mine, mine);
  for (int32_t i = C::kThreads + static_cast<int>(threadIdx.x); i < tp.n; i += C::kThreads) {
    const uint32_t m = tile_pair_at(pp.pi, tp, i);
    if (m) put(m, vals(m));
  }
}

// The exact entries of one row of G inside columns [v0, v0 + Vw): at each
// teacher id v, dense(z_v) - (sum of pcoef over the ids equal to v) - (ycoef
// if v is the label) + (tail bucket) tcoef * q_v per cached copy of v; at a
// label that is no teacher id, dense(z_y) - ycoef.
// z at an id or the label is the fp32 gathered logit, so every entry is
// rounded once. sid / sp hold the row's ids and pcoef (LDS); threads
// t = 0 .. nthreads - 1 of the workgroup share the work.
template <class P>
__device__ __forceinline__ void write_exact_entries(unsigned char* grow, int64_t v0, int64_t Vw,
                                                    const int32_t* sid, const float* sp, int K,
                                                    const float* zk_row, const DenseCoef& dc,
                                                    float c2, int32_t y, float yc, float zy,
                                                    float tc, int t, int nthreads) {
  for (int k = t; k < K; k += nthreads) {
    const int32_t v = sid[k];
    if (v < v0 || v >= v0 + Vw) continue;
    float sum = 0.f, mult = 0.f;
    for (int k2 = 0; k2 < K; ++k2) {
      const bool eq = sid[k2] == v;
      sum += eq ? sp[k2] : 0.f;
      mult += eq ? 1.f : 0.f;
    }
    const float z = zk_row[k];
    float g = dense_g(dc, z, c2) - sum - (v == y ? yc : 0.f);
    if (tc != 0.f) g += tc * mult * fast_exp2(z * c2 - dc.l2);
    store_one<P>(grow, v - v0, g);
  }
  if (t == 0 && y >= 0 && y >= v0 && y < v0 + Vw) {
    bool found = false;
    for (int k2 = 0; k2 < K; ++k2) found |= (sid[k2] == y);
    if (!found) store_one<P>(grow, y - v0, dense_g(dc, zy, c2) - yc);
  }
}

// One wave per row: the exact entries of the slice [v0, v0 + Vw) of its G
// row (write_exact_entries). Arrays start at the block's first row.
template <class P>
__global__ __launch_bounds__(64) void k_fixup(unsigned char* __restrict__ G, int64_t gpitch,
                                              int64_t v0, int64_t Vw,
                                              const int32_t* __restrict__ idx,
                                              const float* __restrict__ zk, RowCoef rc, int K,
                                              float c2) {
  extern __shared__ int32_t sh_fix[];
  int32_t* sid = sh_fix;
  float* sp = reinterpret_cast<float*>(sh_fix + K);
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  for (int k = lane; k < K; k += 64) {
    sid[k] = idx[row * K + k];
    sp[k] = rc.pcoef[row * K + k];
  }
  __syncthreads();
  const int32_t y = rc.labels ? rc.labels[row] : -1;
  write_exact_entries<P>(G + row * gpitch * P::kBytes, v0, Vw, sid, sp, K, zk + row * K,
                         row_dense(rc, row), c2, y, rc.ycoef ? rc.ycoef[row] : 0.f,
                         y >= 0 ? rc.zy[row] : 0.f, rc.tcoef ? rc.tcoef[row] : 0.f, lane, 64);
}

// Kept-logits backward, one workgroup per row: turns the row's kept logits
// z (element type P, zcols entries, the ones at v >= V zero) into its logit
// gradient in place: the dense part below V, zero above, then the exact
// teacher-id and label entries (write_exact_entries, as k_fixup does for a
// slice). Arrays are indexed by row.
constexpr int kGzThreads = 256;

template <class P>
__global__ __launch_bounds__(kGzThreads) void k_g_from_z(unsigned char* __restrict__ Z, int64_t zld,
                                                  int64_t V, int64_t zcols,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ zk, RowCoef rc, int K,
                                                  float c2) {
  extern __shared__ int32_t sh_gz[];
  int32_t* sid = sh_gz;
  float* sp = reinterpret_cast<float*>(sh_gz + K);
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  unsigned char* zr = Z + row * zld;
  const DenseCoef dc = row_dense(rc, row);
  // Each element is read and written once: streaming (nontemporal) accesses
  // keep the row out of the caches' reuse sets.
  constexpr int kPer = 16 / P::kBytes;  // elements per 16-byte vector
  constexpr int kU = 4;                 // vectors in flight per thread
  const int64_t nvec = zcols / kPer;    // zcols is a multiple of the vector width
  for (int64_t i0 = 0; i0 < nvec; i0 += kGzThreads * kU) {
    u32x4_t x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + u * kGzThreads + t;
      if (i < nvec) x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(zr + i * 16));
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + u * kGzThreads + t;
      if (i >= nvec) continue;
      const int64_t v = i * kPer;
      u32x4_t y;
      if constexpr (P::kBytes == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z0 = as_f32(x[u][e] << 16), z1 = as_f32(x[u][e] & 0xffff0000u);
          const float g0 = v + 2 * e < V ? dense_g(dc, z0, c2) : 0.f;
          const float g1 = v + 2 * e + 1 < V ? dense_g(dc, z1, c2) : 0.f;
          y[e] = pack_bf16x2(g0, g1);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = __builtin_bit_cast(uint32_t, v + e < V ? dense_g(dc, as_f32(x[u][e]), c2) : 0.f);
      }
      __builtin_nontemporal_store(y, reinterpret_cast<u32x4_t*>(zr + i * 16));
    }
  }
  for (int k = t; k < K; k += kGzThreads) {
    sid[k] = idx[row * K + k];
    sp[k] = rc.pcoef[row * K + k];
  }
  __syncthreads();  // the dense stores of the row are done before the exact entries are written
  const int32_t y = rc.labels ? rc.labels[row] : -1;
  write_exact_entries<P>(zr, 0, zcols, sid, sp, K, zk + row * K, dc, c2, y,
                         rc.ycoef ? rc.ycoef[row] : 0.f, y >= 0 ? rc.zy[row] : 0.f,
                         rc.tcoef ? rc.tcoef[row] : 0.f, t, kGzThreads);
}

// acc[row][col] (+)= sum over the slice of G[row][v - v0] W[v][col], for the rows
// of one block; the slice is Vw entries wide (Vlim of them below V). With
// splits > 1 the slice is cut into parts of split_k columns (a multiple of the
// stage depth), part sp contracted into its own copy out + sp * out_split_stride
// (each copy receives one contribution per element per launch; the copies are
// summed in a fixed order afterwards).
template <class P, class C>
__global__ __launch_bounds__(C::kThreads) FKL_WAVES_PER_EU(C) void k_grad_hidden(
    const unsigned char* __restrict__ G, int64_t gpitch, const unsigned char* __restrict__ W,
    int64_t d, int64_t Vw, int64_t Vlim, int64_t nrows, int64_t n_tt, int64_t n_dt,
    int accumulate, float* __restrict__ out, int64_t splits, int64_t split_k,
    int64_t out_split_stride) {
  int64_t tt, dt, sp;
  if (!TileGroups<8, 4>::coords_split(n_tt, n_dt, splits, &tt, &dt, &sp)) return;
  const int64_t gld = gpitch * P::kBytes, wld = d * P::kBytes;
  const int64_t k0 = sp * split_k;
  const int64_t kn = Vw - k0 < split_k ? Vw - k0 : split_k;  // columns of this part
  out += sp * out_split_stride;
  // A = G rows of this tile (k = slice column), B = W rows of the slice (k = v), columns of
  // this tile
  const Operand A = make_operand(G + tt * kBM * gld + k0 * P::kBytes, gld, nrows - tt * kBM, kn);
  const Operand B = make_operand(W + dt * kBN * P::kBytes + k0 * wld, wld, d - dt * kBN, Vlim - k0);
  f32x16_t acc[C::kMI][C::kNI];
  gemm_tile<P, C, false, true>(acc, A, B, static_cast<int>(kn > 0 ? kn : 0));

  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = tt * kBM + C::wave_m() * C::kWM + acc_row(mi, r, lane);
      if (row >= nrows) continue;
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni) {
        const int64_t col = dt * kBN + C::wave_n() * C::kWN + ni * 32 + (lane & 31);
        if (col < d) accumulate_out(out + row * d + col, acc[mi][ni][r], accumulate);
      }
    }
}

template <class P>
__global__ __launch_bounds__(256) void k_reduce_gh(const float* __restrict__ part, int64_t splits,
                                                   int64_t nrows, int64_t d,
                                                   unsigned char* __restrict__ out) {
  const int64_t n4 = nrows * d / 4;
  const int64_t stride = nrows * d;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int64_t sp = 1; sp < splits; ++sp) {
      const float4 q = reinterpret_cast<const float4*>(part + sp * stride)[i];
      s.x += q.x;
      s.y += q.y;
      s.z += q.z;
      s.w += q.w;
    }
    const float v[4] = {s.x, s.y, s.z, s.w};
    store4<P>(out + i * 4 * P::kBytes, v);
  }
}

// grad_W[v0 + v][col] (+)= sum over the block's rows of G[row][v] H[row][col].
template <class P, class C>
__global__ __launch_bounds__(C::kThreads) FKL_WAVES_PER_EU(C) void k_grad_w(
    const unsigned char* __restrict__ G, int64_t gpitch, const unsigned char* __restrict__ H,
    int64_t d, int64_t Vw, int64_t Vlim, int64_t nrows, int64_t n_vt, int64_t n_dt, int accumulate,
    float* __restrict__ grad_w, int64_t splits, int64_t split_rows, int64_t out_split_stride) {
  int64_t vt, dt, sp;
  if (!TileGroups<8, 4>::coords_split(n_vt, n_dt, splits, &vt, &dt, &sp)) return;
  // split sp contracts rows [sp * split_rows, ...) into its own output copy
  {
    const int64_t r0 = sp * split_rows;
    G += r0 * gpitch * P::kBytes;
    H += r0 * d * P::kBytes;
    nrows = nrows - r0 < split_rows ? nrows - r0 : split_rows;
    if (nrows < 0) nrows = 0;
    grad_w += sp * out_split_stride;
  }
  // A = G^T (stored [row][v], k = row), B = H (stored [row][col], k = row)
  const Operand A = make_operand(G + vt * kBM * P::kBytes, gpitch * P::kBytes, Vw - vt * kBM, nrows);
  const Operand B = make_operand(H + dt * kBN * P::kBytes, d * P::kBytes, d - dt * kBN, nrows);
  f32x16_t acc[C::kMI][C::kNI];
  gemm_tile<P, C, true, true>(acc, A, B, static_cast<int>(nrows));

  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t v = vt * kBM + C::wave_m() * C::kWM + acc_row(mi, r, lane);
      if (v >= Vlim) continue;
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni) {
        const int64_t col = dt * kBN + C::wave_n() * C::kWN + ni * 32 + (lane & 31);
        if (col < d) accumulate_out(grad_w + v * d + col, acc[mi][ni][r], accumulate);
      }
    }
}

// ------------------------------------------------------------------ utilities

__global__ void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = v;
}

// Every id in [0, V) (with allow_negative: every id below V).
__global__ __launch_bounds__(256) void k_validate_idx(const int32_t* __restrict__ idx, int64_t n,
                                                      int64_t V, int allow_negative,
                                                      int32_t* __restrict__ flag) {
  int bad = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int32_t v = idx[i];
    bad |= ((v < 0 && !allow_negative) || v >= V);
  }
  if (bad) atomicOr(flag, 1);
}

// ------------------------------------------------------------------ launchers

void launch_pair_index(const int32_t* idx, const int32_t* labels, int64_t N, int K, int64_t V,
                       int bw_log2, int64_t n_vb, int32_t* start, uint32_t* entry, int64_t cap,
                       float* zk, float* zy, hipStream_t s) {
  if (N <= 0) return;
  ScopedTimer timer_(KID_PAIR_INDEX, s);
  k_pair_index<<<static_cast<unsigned>(ceil_div(N, 256)), kPairThreads, 0, s>>>(
      idx, labels, N, K, V, bw_log2, n_vb, start, entry, cap, zk, zy);
}

void launch_logits_lse(int dtype, const void* W, const void* H, int64_t d, int64_t V,
                       int64_t row0, int64_t nrows, float c2, float2* part, int64_t part_ld,
                       float2* part_ce, void* Z, int64_t zpitch, const PairIndex* pi, float* zk,
                       float* zy, hipStream_t s) {
  ScopedTimer timer_(KID_LOGITS_LSE, s);
  const PairIndex pix = pi ? *pi : PairIndex{};
  const int64_t eb = dtype == 1 ? 2 : 4;
  const int64_t n_vt = ceil_div(V, kBM), n_tt = ceil_div(nrows, kBN);
  const unsigned char* Hc = static_cast<const unsigned char*>(H) + row0 * d * eb;
  const unsigned char* Wc = static_cast<const unsigned char*>(W);
  const unsigned grid = grouped_grid<4, 8>(n_vt, n_tt);
  unsigned char* Zc = Z ? static_cast<unsigned char*>(Z) + row0 * zpitch * eb : nullptr;
  const int64_t zld = zpitch * eb;
#define FKL_LOGITS(KEEP, CE2)                                                                     \
  do {                                                                                            \
    if (dtype == 1)                                                                               \
      k_logits_lse<BF16, Cfg8, KEEP, CE2><<<grid, Cfg8::kThreads, 0, s>>>(                        \
          Wc, Hc, d, V, nrows, n_vt, n_tt, c2, part, part_ld, part_ce, Zc, zld, zpitch, pix,      \
          row0, zk, zy);                                                                          \
    else                                                                                          \
      k_logits_lse<F32, Cfg4, KEEP, CE2><<<grid, Cfg4::kThreads, 0, s>>>(                         \
          Wc, Hc, d, V, nrows, n_vt, n_tt, c2, part, part_ld, part_ce, Zc, zld, zpitch, pix,      \
          row0, zk, zy);                                                                          \
  } while (0)
  if (Z && part_ce)
    FKL_LOGITS(true, true);
  else if (Z)
    FKL_LOGITS(true, false);
  else if (part_ce)
    FKL_LOGITS(false, true);
  else
    FKL_LOGITS(false, false);
#undef FKL_LOGITS
}

void launch_gather_dot(int dtype, const void* W, const void* H, const int32_t* idx, int64_t d,
                       int64_t row0, int64_t nrows, int K, float* zk, hipStream_t s) {
  if (nrows <= 0) return;
  ScopedTimer timer_(KID_GATHER_DOT, s);
  const int64_t eb = dtype == 1 ? 2 : 4;
  const unsigned char* Hc = static_cast<const unsigned char*>(H) + row0 * d * eb;
  const unsigned blocks = static_cast<unsigned>(ceil_div(nrows, 4));
  const unsigned char* Wc = static_cast<const unsigned char*>(W);
  const size_t lds = static_cast<size_t>(4 * d * eb);  // four hidden rows
  const bool stage = lds <= 64 * 1024;
  if (dtype == 1) {
    if (stage)
      k_gather_dot<BF16, true><<<blocks, 256, lds, s>>>(Wc, Hc, idx + row0 * K, d, nrows, K,
                                                        zk + row0 * K);
    else
      k_gather_dot<BF16, false><<<blocks, 256, 0, s>>>(Wc, Hc, idx + row0 * K, d, nrows, K,
                                                       zk + row0 * K);
  } else {
    if (stage)
      k_gather_dot<F32, true><<<blocks, 256, lds, s>>>(Wc, Hc, idx + row0 * K, d, nrows, K,
                                                       zk + row0 * K);
    else
      k_gather_dot<F32, false><<<blocks, 256, 0, s>>>(Wc, Hc, idx + row0 * K, d, nrows, K,
                                                      zk + row0 * K);
  }
}

void launch_merge_loss(const float2* part, int64_t part_ld, int64_t nslots, const float* zk,
                       const float* logit, int64_t row0, int64_t nrows, int K, float T,
                       float* lse, float* row_loss, const MergeOpts& opts, hipStream_t s) {
  ScopedTimer timer_(KID_MERGE_LOSS, s);
  const unsigned blocks = static_cast<unsigned>(ceil_div(nrows, kMergeRows));
  k_merge_loss<<<blocks, 64 * kMergeWaves, 0, s>>>(part, part_ld, nslots, zk + row0 * K, logit + row0 * K,
                                      row0, nrows, K, T, lse + row0,
                                      row_loss ? row_loss + row0 : nullptr, opts);
}

void launch_reduce_loss(const float* row_loss, int64_t N, float* loss, hipStream_t s) {
  ScopedTimer timer_(KID_REDUCE_LOSS, s);
  k_reduce_loss<<<1, 1024, 0, s>>>(row_loss, N, loss);
}

void launch_bwd_prep(const float* logit, const float* lse, const float* grad_loss, int64_t row0,
                     int64_t nrows, int K, float T, const float* row_weight,
                     const int32_t* labels, float a_kl, float a_ce, const float* lse1,
                     bool two_sm, const float* teacher_lse, const float* zk, float* pcoef,
                     float* acoef, float* lse2, float* bcoef, float* lse1_2, float* ycoef,
                     float* tcoef, const int32_t* idx, float* sub, float* tmul, hipStream_t s) {
  if (nrows <= 0) return;
  ScopedTimer timer_(KID_BWD_PREP, s);
  const size_t shm = sub ? static_cast<size_t>(K) * 8 : 0;
  k_bwd_prep<<<static_cast<unsigned>(nrows), 64, shm, s>>>(
      logit + row0 * K, lse + row0, grad_loss, row0, nrows, K, T, row_weight, labels, a_kl, a_ce,
      lse1, two_sm, teacher_lse, zk, pcoef, acoef, lse2, bcoef, lse1_2, ycoef, tcoef, idx, sub,
      tmul);
}

void launch_gprod(int dtype, const void* W, const void* H, int64_t d, int64_t V, int64_t v0,
                  int64_t Vw, int64_t gpitch, int64_t row0, int64_t nrows, float c2,
                  const RowCoef& rc, void* G, const PairPatch* pp, hipStream_t s) {
  ScopedTimer timer_(KID_GPROD, s);
  const PairPatch ppx = pp ? *pp : PairPatch{};
  const int64_t eb = dtype == 1 ? 2 : 4;
  const int64_t n_vt = ceil_div(Vw, kBM), n_tt = ceil_div(nrows, kBN);
  const unsigned char* Hc = static_cast<const unsigned char*>(H) + row0 * d * eb;
  const unsigned char* Wc = static_cast<const unsigned char*>(W);
  const unsigned grid = grouped_grid<4, 8>(n_vt, n_tt);
  unsigned char* Gc = static_cast<unsigned char*>(G);
#define FKL_GPROD(CE2)                                                                            \
  do {                                                                                            \
    if (dtype == 1)                                                                               \
      k_gprod<BF16, Cfg8, CE2><<<grid, Cfg8::kThreads, 0, s>>>(                                   \
          Wc, Hc, d, V, v0, Vw, gpitch, nrows, n_vt, n_tt, c2, rc, Gc, row0, ppx);                \
    else                                                                                          \
      k_gprod<F32, Cfg4, CE2><<<grid, Cfg4::kThreads, 0, s>>>(                                    \
          Wc, Hc, d, V, v0, Vw, gpitch, nrows, n_vt, n_tt, c2, rc, Gc, row0, ppx);                \
  } while (0)
  if (rc.bcoef)
    FKL_GPROD(true);
  else
    FKL_GPROD(false);
#undef FKL_GPROD
}

void launch_fixup(int dtype, void* G, int64_t gpitch, int64_t v0, int64_t Vw, const int32_t* idx,
                  const float* zk, const RowCoef& rc, int64_t row0, int64_t nrows, int K,
                  float c2, hipStream_t s) {
  if (nrows <= 0) return;
  ScopedTimer timer_(KID_FIXUP, s);
  const size_t shm = static_cast<size_t>(K) * 8;
  if (dtype == 1)
    k_fixup<BF16><<<static_cast<unsigned>(nrows), 64, shm, s>>>(
        static_cast<unsigned char*>(G), gpitch, v0, Vw, idx + row0 * K, zk, rc, K, c2);
  else
    k_fixup<F32><<<static_cast<unsigned>(nrows), 64, shm, s>>>(
        static_cast<unsigned char*>(G), gpitch, v0, Vw, idx + row0 * K, zk, rc, K, c2);
}

void launch_g_from_z(int dtype, void* Z, int64_t zpitch, int64_t V, const int32_t* idx,
                     const float* zk, const RowCoef& rc, int64_t nrows, int K, float c2,
                     hipStream_t s) {
  if (nrows <= 0) return;
  ScopedTimer timer_(KID_G_FROM_Z, s);
  const size_t shm = static_cast<size_t>(K) * 8;
  const unsigned blocks = static_cast<unsigned>(nrows);
  unsigned char* Zc = static_cast<unsigned char*>(Z);
  if (dtype == 1)
    k_g_from_z<BF16><<<blocks, kGzThreads, shm, s>>>(Zc, zpitch * 2, V, zpitch, idx, zk, rc, K, c2);
  else
    k_g_from_z<F32><<<blocks, kGzThreads, shm, s>>>(Zc, zpitch * 4, V, zpitch, idx, zk, rc, K, c2);
}

void launch_grad_hidden(int dtype, const void* G, int64_t gpitch, const void* W, int64_t d,
                        int64_t v0, int64_t Vw, int64_t Vlim, int64_t nrows, bool accumulate,
                        float* acc, int64_t splits, hipStream_t s) {
  ScopedTimer timer_(KID_GRAD_HIDDEN, s);
  const int64_t eb = dtype == 1 ? 2 : 4;
  const int64_t n_tt = ceil_div(nrows, kBM), n_dt = ceil_div(d, kBN);
  const unsigned char* Ws = static_cast<const unsigned char*>(W) + v0 * d * eb;
  if (splits < 1) splits = 1;
  const int64_t split_k = round_up(ceil_div(Vw, splits), 64);
  const unsigned grid = static_cast<unsigned>(TileGroups<8, 4>::grid_split(n_tt, n_dt, splits));
  FKL_LAUNCH_GEMM(k_grad_hidden, dtype, grid, s,
                  static_cast<const unsigned char*>(G), gpitch, Ws, d, Vw, Vlim, nrows, n_tt, n_dt,
                  accumulate ? 1 : 0, acc, splits, split_k, nrows * d);
}

void launch_reduce_grad_hidden(int dtype, const float* part, int64_t splits, int64_t nrows,
                               int64_t d, void* grad_hidden, int64_t row0, hipStream_t s) {
  const int64_t eb = dtype == 1 ? 2 : 4;
  unsigned char* out = static_cast<unsigned char*>(grad_hidden) + row0 * d * eb;
  const int64_t n4 = nrows * d / 4;
  int64_t blocks = ceil_div(n4, 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) return;
  ScopedTimer timer_(KID_REDUCE_GH, s);
  if (dtype == 1)
    k_reduce_gh<BF16><<<static_cast<unsigned>(blocks), 256, 0, s>>>(part, splits, nrows, d, out);
  else
    k_reduce_gh<F32><<<static_cast<unsigned>(blocks), 256, 0, s>>>(part, splits, nrows, d, out);
}

void launch_grad_w_split(int dtype, const void* G, int64_t gpitch, const void* H, int64_t d,
                         int64_t Vw, int64_t Vlim, int64_t row0, int64_t nrows, int64_t splits,
                         bool accumulate, float* out, int64_t out_split_stride, hipStream_t s) {
  ScopedTimer timer_(KID_GRAD_W, s);
  const int64_t eb = dtype == 1 ? 2 : 4;
  const int64_t n_vt = ceil_div(Vw, kBM), n_dt = ceil_div(d, kBN);
  const unsigned char* Hc = static_cast<const unsigned char*>(H) + row0 * d * eb;
  const unsigned grid = static_cast<unsigned>(TileGroups<8, 4>::grid_split(n_vt, n_dt, splits));
  const int64_t split_rows = ceil_div(nrows, splits);
  FKL_LAUNCH_GEMM(k_grad_w, dtype, grid, s,
                  static_cast<const unsigned char*>(G), gpitch, Hc, d, Vw, Vlim, nrows, n_vt, n_dt,
                  accumulate ? 1 : 0, out, splits, split_rows, out_split_stride);
}

void launch_grad_w(int dtype, const void* G, int64_t gpitch, const void* H, int64_t d,
                   int64_t v0, int64_t Vw, int64_t Vlim, int64_t row0, int64_t nrows,
                   bool accumulate, float* grad_w, hipStream_t s) {
  launch_grad_w_split(dtype, G, gpitch, H, d, Vw, Vlim, row0, nrows, 1, accumulate, grad_w + v0 * d,
                      0, s);
}

void launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return;
  ScopedTimer timer_(KID_FILL, s);
  int64_t blocks = ceil_div(n, 256);
  if (blocks > 8192) blocks = 8192;
  k_fill_f32<<<static_cast<unsigned>(blocks), 256, 0, s>>>(p, n, v);
}

void launch_validate_idx(const int32_t* idx, int64_t N, int K, int64_t V, bool allow_negative,
                         int32_t* flag, hipStream_t s) {
  const int64_t n = N * K;
  if (n <= 0) return;
  ScopedTimer timer_(KID_VALIDATE, s);
  int64_t blocks = ceil_div(n, 256);
  if (blocks > 4096) blocks = 4096;
  k_validate_idx<<<static_cast<unsigned>(blocks), 256, 0, s>>>(idx, n, V, allow_negative ? 1 : 0,
                                                               flag);
}

}  // namespace fkl
