// MFMA tile core for gfx950 (CDNA4): one 256x256 output tile per workgroup.
//
// Every contraction of the loss (the logit tile z = W_tile . H_tile^T, its
// recompute in the backward, grad_hidden = G . W and grad_W = G^T . H) runs
// through gemm_tile(). bf16 operands go through the direct-to-LDS ping-pong
// loop further down (eight waves, 128 x 64 outputs each); fp32 operands
// through the register-staged loop below (four waves, 128 x 128 each).
//
// Global reads are raw buffer loads: the buffer's record count makes reads
// past the end of the operand return zero, and lanes whose element lies
// outside the operand use an offset beyond the record count, so tails need no
// branches.
//
// Register-staged loop (fp32): two LDS stages of 128 bytes of K per row with a
// padded pitch; an operand stored contiguous along its m/n index ("MN-major",
// e.g. W read as [v][d] when v is the contraction index) is transposed in
// registers on its way into LDS, so every fragment read is one 16-byte
// ds_read. The registers of each thread hold the global data of stage t+1
// while the waves run the MFMAs of stage t; early in stage t those registers
// are written to the other LDS buffer and refilled with stage t+2. One
// barrier per stage.
//
// Accumulator layout (32x32 MFMA result): element r of block (mi, ni) in lane
// l is row  mi*32 + 8*(r/4) + 4*(l/32) + (r%4)  and column  ni*32 + (l%32)
// of the wave's sub-tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;                           // tile rows (MFMA A side)
constexpr int kBN = 256;                           // tile columns (MFMA B side)
constexpr int kRowBytes = 128;                     // K bytes per stage and row
constexpr int kPitch = kRowBytes + 16;             // padded LDS row pitch
constexpr int kStageBytes = (kBM + kBN) * kPitch;  // 73728
constexpr int kLdsBytes = 2 * kStageBytes;         // 147456 (of 160 KiB)
constexpr uint32_t kOOB = 0x80000000u;             // offset past any record count

// Wave grid of a workgroup: WM x WN waves, each owning (256/WM) x (256/WN).
template <int WM, int WN>
struct TileCfg {
  static constexpr int kWavesM = WM;
  static constexpr int kWavesN = WN;
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kWM = kBM / WM;
  static constexpr int kWN = kBN / WN;
  static constexpr int kMI = kWM / 32;
  static constexpr int kNI = kWN / 32;
  __device__ static int wave_m() { return static_cast<int>(threadIdx.x >> 6) / WN; }
  __device__ static int wave_n() { return static_cast<int>(threadIdx.x >> 6) % WN; }
};

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

// Bit-level reinterpretation of one 32-bit lane value. Taking the argument
// by value matters: applying __builtin_bit_cast directly to a vector-element
// subscript (v[e]) reads element 0 regardless of e with this compiler.
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

__device__ __forceinline__ u32x4_t lds_load16(const unsigned char* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void lds_store16(unsigned char* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}
__device__ __forceinline__ u32x4_t load16(const unsigned char* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// A stored matrix seen as an operand indexed (mn, k), restricted to one tile:
//   k-major  (KC): element (mn, k) at base + mn*ld + k*bytes   (stored [mn][k])
//   mn-major (MC): element (mn, k) at base + k*ld + mn*bytes   (stored [k][mn])
// with base pointing at the tile's first mn (and first k). Elements with
// mn >= mn_count or k >= k_lim read as zero. For KC, k_lim must be a multiple
// of the vector width; for MC, mn_count must be. Every byte offset the tile
// can reach from base must stay below 2^31 (checked on the host); invalid
// elements use an offset past the record count, which the hardware returns
// as zero.
struct Operand {
  __amdgpu_buffer_rsrc_t rsrc;
  u32x4_t words;  // the same descriptor as four scalar words (for the LDS DMA loads)
  uint32_t ld;
  int32_t mn_count;
  int32_t k_lim;
};

__device__ __forceinline__ int32_t clamp_i32(int64_t x) {
  return static_cast<int32_t>(x < 0 ? 0 : (x > 0x7fffffffLL ? 0x7fffffffLL : x));
}

// The arguments are wave-uniform (kernel arguments and block indices); the
// base address is passed through readfirstlane so the descriptor lives in
// scalar registers even where the compiler cannot prove uniformity (otherwise
// each buffer load is wrapped in a loop over lanes).
__device__ __forceinline__ Operand make_operand(const unsigned char* base, int64_t ld,
                                                int64_t mn_count, int64_t k_lim) {
  Operand op;
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  unsigned char* ub = reinterpret_cast<unsigned char*>((static_cast<uint64_t>(hi) << 32) | lo);
  op.rsrc = __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, 0x7fffffff, 0x00020000);
  // base[31:0], base[47:32] with stride 0, record count, format/flags word
  op.words = u32x4_t{lo, hi & 0xffffu, 0x7fffffffu, 0x00020000u};
  op.ld = static_cast<uint32_t>(ld);
  op.mn_count = clamp_i32(mn_count);
  op.k_lim = clamp_i32(k_lim);
  return op;
}

__device__ __forceinline__ u32x4_t buffer_load16(const Operand& op, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(op.rsrc, off, 0, 0));
}

// k-major operand: each thread moves 16-byte vectors of BX rows x 128 bytes.
template <class P, int BX, int NT>
struct StageKC {
  static constexpr int kN = BX * (kRowBytes / 16) / NT;
  u32x4_t r[kN];
  uint32_t off[kN];  // byte offset of the thread's vector at k = 0 (kOOB if its row is invalid)
  int kc[kN];        // k index of the vector within a stage
  __device__ __forceinline__ void init(const Operand& op, int tid) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + i * NT;
      const int row = c >> 3;
      kc[i] = (c & 7) * P::kVec;
      off[i] = row < op.mn_count ? static_cast<uint32_t>(row) * op.ld + kc[i] * P::kBytes : kOOB;
    }
  }
  __device__ __forceinline__ void load(const Operand& op, int k0) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const uint32_t o = (k0 + kc[i] < op.k_lim) ? off[i] + k0 * P::kBytes : kOOB;
      r[i] = buffer_load16(op, o);
    }
  }
  __device__ __forceinline__ void store(unsigned char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + i * NT;
      lds_store16(lds + (c >> 3) * kPitch + (c & 7) * 16, r[i]);
    }
  }
};

// mn-major operand: each thread moves kVec x kVec blocks (kVec k-rows of one
// 16-byte mn-vector), transposes them in registers and writes kVec LDS rows.
// Lane mapping (k-block fastest) keeps both the global reads (8 lanes per
// 128-byte row segment) and the LDS writes (8 lanes per LDS row) conflict-free.
template <class P, int BX, int NT>
struct StageMC {
  static constexpr int V = P::kVec;
  static constexpr int kBlocks = (kRowBytes / 16) * (BX / V);
  static constexpr int kN = (kBlocks + NT - 1) / NT;  // blocks per thread (threads past kBlocks idle)
  u32x4_t r[kN][V];
  uint32_t off[kN];  // byte offset of the block's first element at k = 0 (kOOB if invalid)
  int kb[kN];        // first k of the block within a stage
  __device__ __forceinline__ void init(const Operand& op, int tid) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int b = tid + i * NT;
      const int mb = b >> 3;
      kb[i] = (b & 7) * V;
      off[i] = (b < kBlocks && mb * V < op.mn_count)
                   ? static_cast<uint32_t>(kb[i]) * op.ld + mb * V * P::kBytes
                   : kOOB;
    }
  }
  __device__ __forceinline__ void load(const Operand& op, int k0) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const uint32_t base = off[i] + static_cast<uint32_t>(k0) * op.ld;
      const bool ok = off[i] != kOOB;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const bool v = ok && (k0 + kb[i] + e < op.k_lim);
        r[i][e] = buffer_load16(op, v ? base + e * op.ld : kOOB);
      }
    }
  }
  __device__ __forceinline__ void store(unsigned char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int b = tid + i * NT;
      if (kBlocks % NT != 0 && b >= kBlocks) continue;
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
            o[w] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = r[i][e][j];
        }
        lds_store16(lds + (mb * V + j) * kPitch + kb * 16, o);
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

template <bool MC, class P, int BX, int NT>
struct StageSel {
  typedef StageKC<P, BX, NT> type;
};
template <class P, int BX, int NT>
struct StageSel<true, P, BX, NT> {
  typedef StageMC<P, BX, NT> type;
};

template <class P, class C, bool A_MC, bool B_MC>
struct TileLoop {
  static constexpr int BK = kRowBytes / P::kBytes;
  typedef typename StageSel<A_MC, P, kBM, C::kThreads>::type SA;
  typedef typename StageSel<B_MC, P, kBN, C::kThreads>::type SB;

  // Fragments of k-step s (32 bytes per row per step; lane half h reads the
  // 16-byte chunk 2s+h of its row, the same k-positions for both operands).
  __device__ __forceinline__ static void read_frags(u32x4_t (&fa)[C::kMI], u32x4_t (&fb)[C::kNI],
                                                    const unsigned char* pa,
                                                    const unsigned char* pb, int s) {
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi) fa[mi] = lds_load16(pa + mi * 32 * kPitch + s * 32);
#pragma unroll
    for (int ni = 0; ni < C::kNI; ++ni) fb[ni] = lds_load16(pb + ni * 32 * kPitch + s * 32);
  }

  __device__ __forceinline__ static void mfmas(f32x16_t (&acc)[C::kMI][C::kNI],
                                               const u32x4_t (&fa)[C::kMI],
                                               const u32x4_t (&fb)[C::kNI]) {
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni) mfma_16B<P>(acc[mi][ni], fa[mi], fb[ni]);
  }

  // Issue counts per thread and stage, used to lay out the instruction schedule.
  static constexpr int kMfmaPerStep = C::kMI * C::kNI * (P::kBytes == 2 ? 1 : 4);
  static constexpr int kFragReads = C::kMI + C::kNI;
  static constexpr int kStageWrites = (A_MC ? SA::kN * P::kVec : SA::kN) + (B_MC ? SB::kN * P::kVec : SB::kN);
  static constexpr int kStageLoads = kStageWrites;

  // Pins the order of one k-step: MFMAs evenly interleaved with the fragment
  // reads of the next k-step and, when present, the stage's LDS writes or
  // global loads. Without it the scheduler sinks the global loads to the end
  // of the stage, where their latency is no longer hidden.
  template <int NW, int NL, int NR>
  __device__ __forceinline__ static void schedule_step() {
#pragma unroll
    for (int i = 0; i < kMfmaPerStep; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if ((i * NR) / kMfmaPerStep != ((i + 1) * NR) / kMfmaPerStep)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      if ((i * NW) / kMfmaPerStep != ((i + 1) * NW) / kMfmaPerStep)
        __builtin_amdgcn_sched_group_barrier(0x200, (NW + kMfmaPerStep - 1) / kMfmaPerStep, 0);  // DS write
      if ((i * NL) / kMfmaPerStep != ((i + 1) * NL) / kMfmaPerStep)
        __builtin_amdgcn_sched_group_barrier(0x020, (NL + kMfmaPerStep - 1) / kMfmaPerStep, 0);  // VMEM read
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // k-step S of a stage: read the fragments of step S+1, do the stage's LDS
  // writes (S == 0) or global loads (S == 1), run the MFMAs of step S.
  template <int S, bool STORE_NEXT, bool LOAD_NEXT>
  __device__ __forceinline__ static void kstep(f32x16_t (&acc)[C::kMI][C::kNI],
                                               u32x4_t (&fa)[2][C::kMI], u32x4_t (&fb)[2][C::kNI],
                                               SA& sa, SB& sb, const Operand& A, const Operand& B,
                                               const unsigned char* pa, const unsigned char* pb,
                                               unsigned char* nxt, int k_next, int tid) {
    constexpr int kSteps = kRowBytes / 32;
    if constexpr (S + 1 < kSteps) read_frags(fa[(S + 1) & 1], fb[(S + 1) & 1], pa, pb, S + 1);
    if constexpr (STORE_NEXT && S == 0) {
      sa.store(nxt, tid);
      sb.store(nxt + kBM * kPitch, tid);
    }
    if constexpr (LOAD_NEXT && S == 1) {
      sa.load(A, k_next);
      sb.load(B, k_next);
    }
    mfmas(acc, fa[S & 1], fb[S & 1]);
    constexpr int nr = (S + 1 < kSteps) ? kFragReads : 0;
    constexpr int nw = (STORE_NEXT && S == 0) ? kStageWrites : 0;
    constexpr int nl = (LOAD_NEXT && S == 1) ? kStageLoads : 0;
    schedule_step<nw, nl, nr>();
  }

  // One stage: MFMAs on LDS buffer `cur`; optionally move the prefetched
  // registers into `nxt` and refill them from global stage k_next.
  template <bool STORE_NEXT, bool LOAD_NEXT>
  __device__ __forceinline__ static void stage(f32x16_t (&acc)[C::kMI][C::kNI], SA& sa, SB& sb,
                                               const Operand& A, const Operand& B,
                                               const unsigned char* cur, unsigned char* nxt,
                                               int k_next, int tid, int lane) {
    static_assert(kRowBytes / 32 == 4, "four k-steps per stage");
    const unsigned char* pa = cur + (C::wave_m() * C::kWM + (lane & 31)) * kPitch + (lane >> 5) * 16;
    const unsigned char* pb =
        cur + kBM * kPitch + (C::wave_n() * C::kWN + (lane & 31)) * kPitch + (lane >> 5) * 16;
    u32x4_t fa[2][C::kMI], fb[2][C::kNI];
    read_frags(fa[0], fb[0], pa, pb, 0);
    __builtin_amdgcn_sched_barrier(0);
    kstep<0, STORE_NEXT, LOAD_NEXT>(acc, fa, fb, sa, sb, A, B, pa, pb, nxt, k_next, tid);
    kstep<1, STORE_NEXT, LOAD_NEXT>(acc, fa, fb, sa, sb, A, B, pa, pb, nxt, k_next, tid);
    kstep<2, STORE_NEXT, LOAD_NEXT>(acc, fa, fb, sa, sb, A, B, pa, pb, nxt, k_next, tid);
    kstep<3, STORE_NEXT, LOAD_NEXT>(acc, fa, fb, sa, sb, A, B, pa, pb, nxt, k_next, tid);
    __syncthreads();
  }

  // The loop's LDS (one array per kernel; epilogues may reuse it once every
  // wave has left the loop).
  __device__ __forceinline__ static unsigned char* smem() {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    return lds;
  }

  // acc = A[tile, k_begin:k_end] . B[tile, k_begin:k_end]^T. k_begin is 0 or
  // a multiple of the stage depth; the operands' k_lim zeroes anything past
  // the true end of K.
  __device__ __forceinline__ static void run(f32x16_t (&acc)[C::kMI][C::kNI], const Operand& A,
                                             const Operand& B, int k_begin, int k_end) {
    unsigned char* const lds = smem();
    const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    const int nk = (k_end - k_begin + BK - 1) / BK;
    if (nk <= 0) return;
    SA sa;
    SB sb;
    sa.init(A, tid);
    sb.init(B, tid);
    sa.load(A, k_begin);
    sb.load(B, k_begin);
    sa.store(lds, tid);
    sb.store(lds + kBM * kPitch, tid);
    if (nk > 1) {
      sa.load(A, k_begin + BK);
      sb.load(B, k_begin + BK);
    }
    __syncthreads();
    int kt = 0;
    for (; kt + 2 < nk; ++kt)
      stage<true, true>(acc, sa, sb, A, B, lds + (kt & 1) * kStageBytes,
                        lds + ((kt + 1) & 1) * kStageBytes, k_begin + (kt + 2) * BK, tid, lane);
    if (kt + 1 < nk) {
      stage<true, false>(acc, sa, sb, A, B, lds + (kt & 1) * kStageBytes,
                         lds + ((kt + 1) & 1) * kStageBytes, 0, tid, lane);
      ++kt;
    }
    stage<false, false>(acc, sa, sb, A, B, lds + (kt & 1) * kStageBytes, nullptr, 0, tid, lane);
  }
};

// ---------------------------------------------------------------------------
// Direct-to-LDS pipeline for bf16 operands.
//
// Global data goes straight into LDS with buffer_load ... lds (16 bytes per
// lane, one 1 KiB block per wave instruction), so no registers hold staged
// data. A stage holds 64 values of K for all 256 rows of both operands
// (64 KiB); two stages fill 128 KiB of LDS. Each DMA instruction moves whole
// 128-byte lines: the L1 path into LDS serves one cache line per clock, so a
// row segment of 64 bytes per line would halve its throughput. Loads past K
// or past the operand read out of range, which returns zeros, so tails need
// no branches.
//
// Stage layout of one operand (32 KiB, 32 blocks of 1 KiB):
//  * k-major (stored [mn][k]): 256 rows of 128 bytes, block b = rows 8b..8b+7;
//    the eight 16-byte chunks of row r are XOR-swizzled by (r / 2) % 8, so the
//    16 rows one 256-byte (64-bank) LDS cycle serves land on 16 distinct chunk
//    positions. Fragments are one ds_read_b128.
//  * mn-major (stored [k][mn]): two halves of 128 mn values, each 64 k-rows of
//    256 bytes, block b = k-rows 4(b%16)..4(b%16)+3 of half b/16; the 16
//    chunks of k-row k are XOR-swizzled by 4 * (k % 4). Fragments are two
//    ds_read_b64_tr_b16: within a group of 16 lanes, source lane s reads k-row
//    kb + s/4 at mn = base + 4*(s%4) and lane j receives the 4 k-values of
//    mn = base + j, so two reads give each lane the same 8 consecutive k as
//    the k-major path.
// Both swizzles make the fragment reads bank-conflict free.
constexpr int kDRowBytes = 128;
constexpr int kDStages = 2;
constexpr int kDOperandBytes = 256 * kDRowBytes;  // 32 KiB
constexpr int kDStageBytes = 2 * kDOperandBytes;   // 64 KiB

__device__ __forceinline__ void raw_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding; expcnt unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// The DMA load below sets M0 itself. The compiler treats M0 as reserved and
// warns that clobbering it is not preserved; that is intended: it only writes
// M0 immediately before an instruction that reads it, and on gfx950 no
// instruction these kernels compile to reads M0 except these loads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// One 1 KiB LDS DMA load: lane l's 16 bytes at byte offset voff of the buffer
// go to LDS address lds + 16*l. Written as inline asm so that the compiler's
// wait-count insertion does not see it: it would otherwise guard LDS reads it
// cannot disambiguate from the DMA target with vmcnt(0), draining every load
// in flight. The pipeline places all vmcnt waits for these loads explicitly.
// The load writes no registers; M0 is set (plus the required wait state) in
// the same block.
__device__ __forceinline__ void dma_load16(const u32x4_t& words, uint32_t voff, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)lds)));
  __asm__ volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(words), "s"(m0)
      : "memory", "m0");
}

#pragma clang diagnostic pop

// NINST consecutive blocks of one operand's stage, starting at block `base`,
// moved by one wave: per-lane byte offsets (at k0 = 0) and the k each lane's
// chunk starts at.
template <bool MC, int NINST>
struct DirectOperand {
  uint32_t off[NINST];  // offset at stage k0 = 0 (kOOB if the lane's mn is invalid)
  int kk[NINST];        // k of the lane's data within a stage
  int base;             // first block (wave-uniform)

  __device__ __forceinline__ void init(const Operand& op, int w, int lane, int blk0) {
    base = blk0 + w * NINST;
#pragma unroll
    for (int j = 0; j < NINST; ++j) {
      const int blk = base + j;
      if constexpr (!MC) {
        const int row = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        kk[j] = c * 8;
        off[j] = row < op.mn_count ? static_cast<uint32_t>(row) * op.ld + c * 16 : kOOB;
      } else {
        const int half = blk >> 4;
        const int krow = 4 * (blk & 15) + (lane >> 4);
        const int c = (lane & 15) ^ (4 * (krow & 3));
        kk[j] = krow;
        off[j] = half * 128 + c * 8 < op.mn_count
                     ? static_cast<uint32_t>(krow) * op.ld + half * 256 + c * 16
                     : kOOB;
      }
    }
  }

  // Loads of the stage starting at k0 into the operand region at dst.
  __device__ __forceinline__ void issue(const Operand& op, int k0, unsigned char* dst) const {
#pragma unroll
    for (int j = 0; j < NINST; ++j) {
      uint32_t o;
      if constexpr (!MC)
        o = (k0 + kk[j] < op.k_lim) ? off[j] + k0 * 2 : kOOB;
      else
        o = (off[j] != kOOB && k0 + kk[j] < op.k_lim) ? off[j] + static_cast<uint32_t>(k0) * op.ld
                                                       : kOOB;
      dma_load16(op.words, o, dst + (base + j) * 1024);
    }
  }

  // Fragment of 32 rows (mn0 .. mn0 + 31 of the tile) for k-step s of a stage.
  __device__ __forceinline__ static u32x4_t frag(const unsigned char* src, int mn0, int s, int lane) {
    if constexpr (!MC) {
      const int row = mn0 + (lane & 31);
      const int c = (2 * s + (lane >> 5)) ^ ((row >> 1) & 7);
      return lds_load16(src + row * kDRowBytes + c * 16);
    } else {
      const int g = lane >> 4, sl = lane & 15;
      const int mn = mn0 + 16 * (g & 1) + 4 * (sl & 3);
      const unsigned char* hsrc = src + (mn >> 7) * (kDOperandBytes / 2);
      const int mh = mn & 127;
      const int kb = 16 * s + 8 * (g >> 1) + (sl >> 2);
      u32x4_t r;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = kb + 4 * h;
        const int c = (mh >> 3) ^ (4 * (k & 3));
        const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(hsrc + k * 256 + c * 16 + (mh & 7) * 2));
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t u = __builtin_bit_cast(u32x2_t, v);
        r[2 * h] = u[0];
        r[2 * h + 1] = u[1];
      }
      return r;
    }
  }
};

// ---------------------------------------------------------------------------
// Ping-pong k-loop (eight waves, 128 x 64 outputs each). The two waves that
// share a SIMD (w and w + 4) sit in different groups, G0 = waves 0-3 and
// G1 = waves 4-7, which run the same program one phase apart. A wave
// alternates LOAD (the fragments of a k-block of two k-steps, LDS to
// registers, plus a quarter of a stage's DMA traffic) and COMPUTE (that
// k-block's 16 MFMAs at raised issue priority), with a workgroup barrier
// between phases. While one wave of a SIMD computes, the other loads, so the
// matrix pipe is fed in back-to-back bursts.
//
// Only loading waves issue DMA: a wave issues in order, and a DMA load stalls
// at issue while the address unit is busy with earlier ones, so a computing
// wave that issued DMA would starve its MFMAs. Each LOAD phase moves 16 KiB
// (four 1 KiB loads per wave, after the fragment reads), about as long at the
// address unit as the other group's MFMA burst.
//
// G0 loads k-block j in phase 2j and computes it in 2j+1; G1 loads it in 2j+1
// and computes it in 2j+2; stage s holds k-blocks 2s and 2s+1 in slot s % 2.
// G0 reads rows 0-127 of A ("A-lo") and all of B, G1 rows 128-255 ("A-hi")
// and all of B, so for stage s the slot's A-lo is last read in phase 4s+2 and
// the rest in 4s+3. Stage s+2 is moved into the slot in four parts:
//   phase 4s+3, G1: A-lo            phase 4s+4, G0: B rows 0-127
//   phase 4s+5, G1: B rows 128-255  phase 4s+6, G0: A-hi
// Stage s+2 is first read by G0 in phase 4s+8 and by G1 in 4s+9; each wave
// waits for the parts it moved before the barrier that opens that phase (A-lo
// and B at the end of phase 4s+7, A-hi at the end of 4s+8), counting the four
// loads it issued after them (the hardware returns loads in order). The
// barriers carry no memory fence, which would drain every load in flight.
template <class C, bool A_MC, bool B_MC>
struct PingPongLoop {
  static_assert(C::kThreads == 512 && C::kWavesM == 2, "two groups of four waves");
  static constexpr int BK = kDRowBytes / 2;  // 64 bf16 of K per stage

  __device__ __forceinline__ static void fence() { __builtin_amdgcn_sched_barrier(0); }
  __device__ __forceinline__ static void phase_barrier() {
    fence();
    raw_barrier();
    fence();
  }

  // The stages live in distinct __shared__ arrays (the slot is a compile-time
  // index of the unrolled loop).
  struct Stages {
    unsigned char* s[kDStages];
  };
  __device__ __forceinline__ static Stages stage_arrays() {
    __shared__ __attribute__((aligned(1024))) unsigned char st0[kDStageBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[kDStageBytes];
    static_assert(kDStages == 2, "two stages");
    Stages r;
    r.s[0] = st0;
    r.s[1] = st1;
    return r;
  }

  __device__ __forceinline__ static void frags(u32x4_t (&fa)[C::kMI], u32x4_t (&fb)[C::kNI],
                                               const unsigned char* stage, int s, int lane) {
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi)
      fa[mi] = DirectOperand<A_MC, 1>::frag(stage, C::wave_m() * C::kWM + mi * 32, s, lane);
#pragma unroll
    for (int ni = 0; ni < C::kNI; ++ni)
      fb[ni] = DirectOperand<B_MC, 1>::frag(stage + kDOperandBytes,
                                            C::wave_n() * C::kWN + ni * 32, s, lane);
  }

  __device__ __forceinline__ static void mfmas(f32x16_t (&acc)[C::kMI][C::kNI],
                                               const u32x4_t (&fa)[C::kMI],
                                               const u32x4_t (&fb)[C::kNI]) {
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni) mfma_16B<BF16>(acc[mi][ni], fa[mi], fb[ni]);
  }

  // What one group moves, four blocks per wave each: G0 B rows 0-127 (p) and
  // A rows 128-255 (q), G1 A rows 0-127 (p) and B rows 128-255 (q).
  template <int G>
  struct Stream {
    DirectOperand<G == 0 ? B_MC : A_MC, 4> p;
    DirectOperand<G == 0 ? A_MC : B_MC, 4> q;
    static constexpr int kP = G == 0 ? kDOperandBytes : 0;  // slot offset of p's operand
    static constexpr int kQ = kDOperandBytes - kP;
  };

  // One k-block: R = j % 4 fixes the slot (stage parity) and the half.
  // P and Q are the operands of the group's p and q parts.
  template <int G, int R>
  __device__ __forceinline__ static void block(f32x16_t (&acc)[C::kMI][C::kNI],
                                               u32x4_t (&fa)[2][C::kMI], u32x4_t (&fb)[2][C::kNI],
                                               const Stream<G>& str, const Operand& P,
                                               const Operand& Q, const Stages& st, int j,
                                               int lane) {
    constexpr int h = R & 1, sp = R >> 1;
    const int s = j >> 1;
    unsigned char* cur = st.s[sp];
    unsigned char* other = st.s[1 - sp];
    // LOAD(j)
    frags(fa[0], fb[0], cur, 2 * h, lane);
    frags(fa[1], fb[1], cur, 2 * h + 1, lane);
    if constexpr (G == 0 && h == 0) {
      if (j >= 2) str.p.issue(P, (s + 1) * BK, other + Stream<G>::kP);  // B rows 0-127, stage s+1
      wait_vmcnt_lgkm0<4>();  // A rows 128-255 of stage s landed
    } else if constexpr (G == 0 && h == 1) {
      str.q.issue(Q, (s + 1) * BK, other + Stream<G>::kQ);  // A rows 128-255, stage s+1
      wait_vmcnt_lgkm0<63>();
    } else if constexpr (G == 1 && h == 1) {
      str.p.issue(P, (s + 2) * BK, cur + Stream<G>::kP);  // A rows 0-127, stage s+2
      wait_vmcnt_lgkm0<4>();  // A rows 0-127 and B rows 128-255 of stage s+1 landed
    } else {
      if (j >= 2) str.q.issue(Q, (s + 1) * BK, other + Stream<G>::kQ);  // B rows 128-255, stage s+1
      wait_vmcnt_lgkm0<63>();
    }
    phase_barrier();
    // COMPUTE(j)
    __builtin_amdgcn_s_setprio(1);
    mfmas(acc, fa[0], fb[0]);
    mfmas(acc, fa[1], fb[1]);
    fence();
    __builtin_amdgcn_s_setprio(0);
    if constexpr (G == 0 && h == 1) wait_vmcnt_lgkm0<4>();  // B rows 0-127 of stage s+1 landed
    phase_barrier();
  }

  template <int G>
  __device__ __forceinline__ static void program(f32x16_t (&acc)[C::kMI][C::kNI], const Operand& P,
                                                 const Operand& Q, const Stages& st, int nk,
                                                 int wg, int lane) {
    Stream<G> str;
    str.p.init(P, wg, lane, 0);
    str.q.init(Q, wg, lane, 16);
    // prologue: stages 0 and 1; stage 0 landed, stage 1 (8 loads) may still be in flight
#pragma unroll
    for (int t = 0; t < kDStages; ++t) {
      str.p.issue(P, t * BK, st.s[t] + Stream<G>::kP);
      str.q.issue(Q, t * BK, st.s[t] + Stream<G>::kQ);
    }
    wait_vmcnt_lgkm0<8>();
    phase_barrier();
    u32x4_t fa[2][C::kMI], fb[2][C::kNI];
    if constexpr (G == 1) phase_barrier();  // G1 runs one phase behind
    const int J = 2 * nk;
    int j = 0;
    for (; j + 4 <= J; j += 4) {
      block<G, 0>(acc, fa, fb, str, P, Q, st, j, lane);
      block<G, 1>(acc, fa, fb, str, P, Q, st, j + 1, lane);
      block<G, 2>(acc, fa, fb, str, P, Q, st, j + 2, lane);
      block<G, 3>(acc, fa, fb, str, P, Q, st, j + 3, lane);
    }
    if (j < J) {  // odd number of stages: one more in slot 0
      block<G, 0>(acc, fa, fb, str, P, Q, st, j, lane);
      block<G, 1>(acc, fa, fb, str, P, Q, st, j + 1, lane);
    }
    if constexpr (G == 0) phase_barrier();  // pairs with G1's last one
  }

  __device__ __forceinline__ static void run(f32x16_t (&acc)[C::kMI][C::kNI], const Operand& A,
                                             const Operand& B, int K) {
    const Stages st = stage_arrays();
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
#pragma unroll
    for (int mi = 0; mi < C::kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    const int nk = (K + BK - 1) / BK;
    if (nk <= 0) return;
    if (w < 4)
      program<0>(acc, B, A, st, nk, w, lane);
    else
      program<1>(acc, A, B, st, nk, w - 4, lane);
    // drain the out-of-range loads before the LDS is reused
    wait_vmcnt_lgkm0<0>();
  }
};

// acc = A[tile, 0:K] . B[tile, 0:K]^T for one 256 x 256 tile: bf16 through the
// direct-to-LDS ping-pong loop (eight waves), fp32 through the register-staged
// loop.
template <class P, class C, bool A_MC, bool B_MC>
__device__ __forceinline__ void gemm_tile(f32x16_t (&acc)[C::kMI][C::kNI], const Operand& A,
                                          const Operand& B, int K) {
  if constexpr (P::kBytes == 2)
    PingPongLoop<C, A_MC, B_MC>::run(acc, A, B, K);
  else
    TileLoop<P, C, A_MC, B_MC>::run(acc, A, B, 0, K);
}

// Grouped, XCD-aware tile order. Blocks are dealt round-robin over the 8 XCDs
// (launch block b runs on XCD b % 8) and each XCD runs ~32 workgroups at a
// time (one per CU). The output tiles are laid out in strips of GB tile
// columns, each strip row-major, and each XCD takes an equal contiguous share
// of that order (its blocks in launch order walk its share): whole strips
// when they split evenly over the XCDs, else a share rounded up to whole
// rounds of 32. The 32 workgroups an XCD runs at once are consecutive
// tiles: (32 / GB) tile rows of one strip (GA x GB for full strips), so one L2
// serves their GA panels of one operand and GB of the other instead of each
// streaming its own; and every XCD has at most ceil(ceil(T / 8) / 32) rounds
// of a grid of T tiles (whole groups of 32 per XCD left some XCDs a round
// more than others whenever the group count was not a multiple of 8). Launch
// with grid() blocks; blocks past the grid exit.
template <int GA, int GB>
struct TileGroups {
  static_assert(GA * GB == 32, "one group per XCD round of workgroups");
  // Tiles per XCD: whole strips when the strips split evenly over the 8 XCDs
  // (each XCD then walks its own strips from their first row); otherwise an
  // equal share rounded up to whole rounds of 32, so that each round is one
  // aligned group of the strip order. Either way the same number of rounds
  // as the exact share (ceil(x / 32) = round_up(x, 32) / 32).
  static __host__ __device__ __forceinline__ int64_t share(int64_t mt, int64_t nt,
                                                           int64_t splits) {
    const int64_t total = mt * nt * splits;
    if (splits == 1 && nt % GB == 0 && (nt / GB) % 8 == 0) return total / 8;
    return ((total + 7) / 8 + 31) / 32 * 32;
  }
  static int64_t grid(int64_t mt, int64_t nt) { return 8 * share(mt, nt, 1); }
  // Tile of position t (0 <= t < mt * nt) in the strip order.
  __device__ __forceinline__ static void tile_of(int64_t t, int64_t mt, int64_t nt, int64_t* tm,
                                                 int64_t* tn) {
    const int64_t full = (nt / GB) * GB * mt;  // tiles in full-width strips
    if (t < full) {
      const int64_t s = t / (GB * mt), r = t - s * (GB * mt);
      *tm = r / GB;
      *tn = s * GB + r % GB;
    } else {
      const int64_t ws = nt % GB, r = t - full;
      *tm = r / ws;
      *tn = (nt / GB) * GB + r % ws;
    }
  }
  __device__ __forceinline__ static bool coords(int64_t mt, int64_t nt, int64_t* tm, int64_t* tn) {
    const int64_t total = mt * nt, per = share(mt, nt, 1);
    const int64_t b = blockIdx.x;
    const int64_t t = (b & 7) * per + (b >> 3);
    if ((b >> 3) >= per || t >= total) return false;
    tile_of(t, mt, nt, tm, tn);
    return true;
  }
  // The same with `splits` copies of the tile grid (a split of the
  // contraction): position t runs over splits x tiles, split-major, so the
  // copies are spread over the XCDs like any other tiles. splits = 1 is coords().
  static int64_t grid_split(int64_t mt, int64_t nt, int64_t splits) {
    return 8 * share(mt, nt, splits);
  }
  __device__ __forceinline__ static bool coords_split(int64_t mt, int64_t nt, int64_t splits,
                                                      int64_t* tm, int64_t* tn, int64_t* sp) {
    const int64_t tiles = mt * nt, total = tiles * splits, per = share(mt, nt, splits);
    const int64_t b = blockIdx.x;
    const int64_t t = (b & 7) * per + (b >> 3);
    if ((b >> 3) >= per || t >= total) return false;
    *sp = t / tiles;
    tile_of(t - *sp * tiles, mt, nt, tm, tn);
    return true;
  }
};

// Row offset, inside the wave sub-tile, of accumulator element r of block mi.
__device__ __forceinline__ int acc_row(int mi, int r, int lane) {
  return mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Two fp32 values rounded to nearest-even bf16 and packed (lo in bits 0-15):
// one v_cvt_pk_bf16_f32. Over every non-NaN fp32 input it gives the same bits
// as adding 0x7fff plus the lowest kept bit and truncating.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.f));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

}  // namespace fkl
