// MFMA tile core for gfx950 (CDNA4): one 256x256 output tile per workgroup.
//
// Every contraction of the loss (the logit tile z = W_tile . H_tile^T, its
// recompute in the backward, grad_hidden = G . W and grad_W = G^T . H) runs
// through gemm_tile(). Operands are staged through LDS in a k-contiguous
// layout with a padded row pitch; an operand whose storage is contiguous along
// its m/n index instead ("MN-major", e.g. W read as [v][d] when v is the
// contraction index) is transposed in registers on the way into LDS, so the
// fragment reads are always one 16-byte ds_read per lane.
//
// Tile shape: 256 threads = 4 wave64s in a 2x2 grid, each wave owning a
// 128x128 sub-tile as 4x4 MFMA blocks of 32x32 (bf16: v_mfma_f32_32x32x16_bf16;
// fp32: v_mfma_f32_32x32x2_f32). One pipeline stage covers 128 bytes of K per
// row (64 bf16 or 32 fp32); two stages are double-buffered in LDS (144 KiB),
// with the next stage's global loads in flight during the current stage's
// MFMAs.
//
// Accumulator layout (32x32 MFMA result, as documented for CDNA3/CDNA4):
// element r of block (mi, ni) in lane l is row
//   mi*32 + 8*(r/4) + 4*(l/32) + (r%4)   and column   ni*32 + (l%32)
// of the wave's sub-tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBM = 256;  // tile rows (MFMA A side)
constexpr int kBN = 256;  // tile columns (MFMA B side)
constexpr int kWM = 128;  // wave sub-tile rows
constexpr int kWN = 128;  // wave sub-tile columns
constexpr int kMI = kWM / 32;
constexpr int kNI = kWN / 32;
constexpr int kRowBytes = 128;                     // K bytes per stage and row
constexpr int kPitch = kRowBytes + 16;             // padded LDS row pitch
constexpr int kStageBytes = (kBM + kBN) * kPitch;  // 73728
constexpr int kLdsBytes = 2 * kStageBytes;         // 147456 (of 160 KiB)

// Element kinds. bf16 is carried as raw 16-bit patterns.
struct BF16 {
  typedef uint16_t storage;
  static constexpr int kBytes = 2;
  static constexpr int kVec = 8;  // elements per 16-byte vector
};
struct F32 {
  typedef float storage;
  static constexpr int kBytes = 4;
  static constexpr int kVec = 4;
};

// A stored matrix seen as an operand indexed (mn, k).
//   k-major  (KC): element (mn, k) at base + mn*ld + k*bytes   (stored [mn][k])
//   mn-major (MC): element (mn, k) at base + k*ld + mn*bytes   (stored [k][mn])
// Reads with mn >= mn_lim or k >= k_lim return zero. For KC, k_lim must be a
// multiple of the vector width; for MC, mn_lim must be.
struct Operand {
  const unsigned char* base;
  int64_t ld;  // bytes between consecutive stored rows
  int64_t mn0;
  int64_t mn_lim;
  int64_t k_lim;
};

// Bit-level reinterpretation of one 32-bit lane value. Taking the argument
// by value matters: applying __builtin_bit_cast directly to a vector-element
// subscript (v[e]) reads element 0 regardless of e with this compiler.
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

__device__ __forceinline__ u32x4_t load16(const unsigned char* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void store16(unsigned char* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// k-major operand: each thread moves (BX * 128 / 16) / 256 16-byte vectors.
template <class P, int BX>
struct StageKC {
  static constexpr int kN = BX * (kRowBytes / 16) / kThreads;
  u32x4_t r[kN];
  __device__ __forceinline__ void load(const Operand& op, int64_t k0, int tid) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + i * kThreads;
      const int row = c >> 3, kc = c & 7;
      const int64_t mn = op.mn0 + row;
      const int64_t k = k0 + kc * P::kVec;
      if (mn < op.mn_lim && k < op.k_lim)
        r[i] = load16(op.base + mn * op.ld + k * P::kBytes);
      else
        r[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(unsigned char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + i * kThreads;
      store16(lds + (c >> 3) * kPitch + (c & 7) * 16, r[i]);
    }
  }
};

// mn-major operand: each thread moves kVec x kVec blocks (kVec k-rows of one
// 16-byte mn-vector), transposes them in registers and writes kVec LDS rows.
// Lane mapping (kb fastest) keeps both the global reads (8 lanes per 128-byte
// row segment) and the LDS writes (8 lanes per LDS row) conflict-free.
template <class P, int BX>
struct StageMC {
  static constexpr int V = P::kVec;
  static constexpr int kN = (kRowBytes / 16) * (BX / V) / kThreads;
  u32x4_t r[kN][V];
  __device__ __forceinline__ void load(const Operand& op, int64_t k0, int tid) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int b = tid + i * kThreads;
      const int kb = b & 7, mb = b >> 3;
      const int64_t mn = op.mn0 + mb * V;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int64_t k = k0 + kb * V + e;
        if (mn < op.mn_lim && k < op.k_lim)
          r[i][e] = load16(op.base + k * op.ld + mn * P::kBytes);
        else
          r[i][e] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(unsigned char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int b = tid + i * kThreads;
      const int kb = b & 7, mb = b >> 3;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        u32x4_t o;
        if constexpr (P::kBytes == 2) {
          // output dword w holds k = 2w (low half) and 2w+1 (high half) of mn j
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t lo = r[i][2 * w][j >> 1];
            const uint32_t hi = r[i][2 * w + 1][j >> 1];
            o[w] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                           : ((lo & 0xffffu) | (hi << 16));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = r[i][e][j];
        }
        store16(lds + (mb * V + j) * kPitch + kb * 16, o);
      }
    }
  }
};

template <class P>
__device__ __forceinline__ void mfma_16B(f32x16_t& c, u32x4_t a, u32x4_t b) {
  if constexpr (P::kBytes == 2) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(as_f32(a[e]), as_f32(b[e]), c, 0, 0, 0);
  }
}

// One LDS stage: 4 k-steps of 32 bytes per row; lane half h reads the 16-byte
// chunk 2s+h of its row, the same k-positions for both operands.
template <class P>
__device__ __forceinline__ void compute_stage(f32x16_t (&acc)[kMI][kNI], const unsigned char* la,
                                              const unsigned char* lb, int wm, int wn, int lane) {
  const unsigned char* pa = la + (wm * kWM + (lane & 31)) * kPitch + (lane >> 5) * 16;
  const unsigned char* pb = lb + (wn * kWN + (lane & 31)) * kPitch + (lane >> 5) * 16;
#pragma unroll
  for (int s = 0; s < kRowBytes / 32; ++s) {
    u32x4_t a[kMI], b[kNI];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) a[mi] = load16(pa + mi * 32 * kPitch + s * 32);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) b[ni] = load16(pb + ni * 32 * kPitch + s * 32);
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) mfma_16B<P>(acc[mi][ni], a[mi], b[ni]);
  }
}

template <bool MC, class P, int BX>
struct StageSel {
  typedef StageKC<P, BX> type;
};
template <class P, int BX>
struct StageSel<true, P, BX> {
  typedef StageMC<P, BX> type;
};

// acc = A[mn tile, k_begin:k_end] . B[mn tile, k_begin:k_end]^T
// k_begin must be a multiple of the stage depth unless it is 0; steps past
// k_end read zeros only if the operands' k_lim says so (callers split K on
// stage boundaries and end the last split at k_lim).
template <class P, bool A_MC, bool B_MC>
__device__ __forceinline__ void gemm_tile(f32x16_t (&acc)[kMI][kNI], const Operand& A,
                                          const Operand& B, int64_t k_begin, int64_t k_end,
                                          unsigned char* lds) {
  constexpr int BK = kRowBytes / P::kBytes;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int64_t nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;
  typename StageSel<A_MC, P, kBM>::type sa;
  typename StageSel<B_MC, P, kBN>::type sb;
  sa.load(A, k_begin, tid);
  sb.load(B, k_begin, tid);
  sa.store(lds, tid);
  sb.store(lds + kBM * kPitch, tid);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    unsigned char* cur = lds + (kt & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load(A, k_begin + (kt + 1) * BK, tid);
      sb.load(B, k_begin + (kt + 1) * BK, tid);
    }
    compute_stage<P>(acc, cur, cur + kBM * kPitch, wm, wn, lane);
    if (more) {
      unsigned char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
      sa.store(nxt, tid);
      sb.store(nxt + kBM * kPitch, tid);
    }
    __syncthreads();
  }
}

// Row offset, inside the wave sub-tile, of accumulator element r of block mi.
__device__ __forceinline__ int acc_row(int mi, int r, int lane) {
  return mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD b % 8).
// Give each XCD one contiguous range of tile indices so that tiles sharing an
// operand panel run on the same XCD and hit its L2. The grid is launched with
// 8 * ceil(total / 8) blocks; indices >= total exit.
__device__ __forceinline__ int64_t xcd_tile_index(int64_t total) {
  const int64_t b = blockIdx.x;
  const int64_t per = (total + 7) / 8;
  return (b & 7) * per + (b >> 3);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

}  // namespace fkl
