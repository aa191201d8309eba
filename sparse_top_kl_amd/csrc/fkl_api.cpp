// C ABI of libfkl: argument validation, workspace planning and the chunk loop.
// The declarations, argument meanings, layouts and error behaviour are in
// include/fkl.h.
#include "fkl.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "api_common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace fkl_api {
thread_local char g_last_error[512] = "";
}  // namespace fkl_api

using namespace fkl_api;

namespace {

// The backward keeps one block of the logit gradient G: bw_rows rows of a
// vocabulary slice bw_width wide, with bw_rows * bw_width <= chunk * Vpad (the
// memory the chunk size allows); rows are padded to bw_pitch, a multiple of 64
// elements, so every row starts on a 128-byte line.
struct Plan {
  int64_t chunk_cap;  // forward rows per pass (<= N, >= 1)
  int64_t Vpad;       // vocabulary rounded up to 8
  int64_t nslots;     // vocabulary slices holding a partial (valid ones)
  int64_t slot_cap;   // partial slots allocated per row
  // backward blocking: row blocks of bw_rows x vocabulary slices of bw_width;
  // grad_hidden's contraction over a slice cut in gh_splits parts (separate
  // fp32 accumulators) when its tiles alone would leave CUs idle
  int64_t bw_rows, bw_width, bw_pitch, gh_splits;
  // teacher-id pair index (kernels.hpp PairIndex): bucket width, buckets, row
  // tiles, entries per row tile (room for a label per row); pair_log2 < 0 when
  // the vocabulary is too wide to bucket (the separate gather and fixup
  // kernels are used instead)
  int pair_log2;
  int64_t n_vb, n_rt, pair_cap;
  // forward workspace offsets
  size_t f_part, f_part_ce, f_rowloss, f_topkz, f_zy, f_pstart, f_pentry, f_flag, f_total;
  // backward workspace offsets
  size_t b_G, b_ghacc, b_pcoef, b_acoef, b_lse2, b_zk, b_bcoef, b_lse12, b_ycoef, b_zy, b_tcoef,
      b_pstart, b_pentry, b_sub, b_tmul, b_flag, b_total;
};

// Rounds of 256 x 256 tiles a launch of `tiles` tiles takes: every XCD (8 of
// 32 CUs) runs an equal share of the tiles, 32 at a time (TileGroups).
inline int64_t tile_rounds(int64_t tiles) { return fkl::ceil_div(fkl::ceil_div(tiles, 8), 32); }

// Predicted cost of the backward contractions for row blocks of rc rows and
// vocabulary slices of width vs, in units of one value of the contraction
// length on a round of tiles: a launch runs tile_rounds(tiles) rounds whose
// contraction length is d (logit tiles), the slice width (grad_hidden) or the
// block's rows (grad_W); each slice adds a fixed cost for its launches. The
// sizes are those of the loops in fkl_backward.
double backward_cost(int64_t N, int64_t Vpad, int64_t d, int64_t rc, int64_t vs) {
  constexpr double kSliceCost = 1000.0;
  const int64_t dt = fkl::ceil_div(d, 256);
  double c = 0.0;
  for (int64_t r0 = 0; r0 < N; r0 += rc) {
    const int64_t nr = N - r0 < rc ? N - r0 : rc;
    const int64_t rt = fkl::ceil_div(nr, 256);
    for (int64_t v0 = 0; v0 < Vpad; v0 += vs) {
      const int64_t vw = Vpad - v0 < vs ? Vpad - v0 : vs;
      const int64_t vt = fkl::ceil_div(vw, 256);
      c += double(tile_rounds(rt * vt)) * d + double(tile_rounds(rt * dt)) * vw +
           double(tile_rounds(vt * dt)) * nr + kSliceCost;
    }
  }
  return c;
}

// Row blocks are multiples of 256 rows (or all N), slice widths multiples of
// 32 elements; among the shapes within the budget the one with the least
// predicted cost is chosen.
void plan_backward_blocks(int64_t N, int64_t Vpad, int64_t d, int64_t chunk_cap, int64_t eb,
                          int64_t* rows, int64_t* width) {
  constexpr int64_t kGran = 32;
  int64_t budget = chunk_cap * Vpad;
  // rows * pitch * eb must stay below kMaxBlockBytes with up to 63 pad elements per row
  if (budget > kMaxBlockBytes / eb - 64 * N) budget = kMaxBlockBytes / eb - 64 * N;
  // grad_W reads the block's hidden rows through 32-bit offsets as well
  const int64_t max_rows = kMaxBlockBytes / (d * eb);
  if (budget >= N * Vpad && N <= max_rows) {  // one block covers everything
    *rows = N;
    *width = Vpad;
    return;
  }
  double best = 1e300;
  *rows = 1;
  *width = Vpad;
  const int64_t max_blocks = fkl::ceil_div(N, 256);
  for (int64_t nb = 1; nb <= max_blocks; ++nb) {
    const int64_t rc = nb == 1 ? N : fkl::round_up(fkl::ceil_div(N, nb), 256);
    if (rc > N || rc * kGran > budget || rc > max_rows) continue;
    if (nb > 1 && fkl::ceil_div(N, rc) != nb) continue;  // same blocking as a smaller nb
    const int64_t vs_max = budget / rc;
    const int64_t vm = vs_max >= Vpad ? Vpad : vs_max / kGran * kGran;
    const int64_t ns0 = fkl::ceil_div(Vpad, vm);
    for (int64_t ns = ns0; ns < ns0 + 3; ++ns) {
      const int64_t vs = fkl::round_up(fkl::ceil_div(Vpad, ns), kGran);
      if (vs > vm) continue;
      const double cost = backward_cost(N, Vpad, d, rc, vs);
      if (cost < best) {
        best = cost;
        *rows = rc;
        *width = vs;
      }
    }
  }
  if (best == 1e300) {  // tiny budget: as many rows as fit, whole vocabulary
    int64_t r = budget / Vpad > 0 ? (budget / Vpad < N ? budget / Vpad : N) : 1;
    if (r > max_rows) r = max_rows;
    *rows = r;
    *width = Vpad;
  }
}

// Parts the grad_hidden contraction over a slice of width vs is cut into, for
// row blocks of rc rows: the count (1 .. 4) with the fewest predicted rounds x
// contraction length (tile_rounds), e.g. 2 when one block's 256 x 256 tiles
// alone take 1.5 rounds of the chip.
int64_t grad_hidden_splits(int64_t rc, int64_t vs, int64_t d) {
  const int64_t tiles = fkl::ceil_div(rc, 256) * fkl::ceil_div(d, 256);
  int64_t best = 1;
  double best_cost = 1e300;
  for (int64_t sp = 1; sp <= 4; ++sp) {
    const int64_t kc = fkl::round_up(fkl::ceil_div(vs, sp), 64);
    if (sp > 1 && kc * (sp - 1) >= vs) break;  // a part would be empty
    const double c = double(tile_rounds(tiles * sp)) * double(kc) * (1.0 + 0.02 * double(sp - 1));
    if (c < best_cost) {
      best_cost = c;
      best = sp;
    }
  }
  return best;
}

Plan make_plan(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int32_t dtype) {
  using namespace fkl;
  Plan p{};
  const int64_t eb = dtype == FKL_BF16 ? 2 : 4;
  p.chunk_cap = chunk < N ? chunk : N;
  if (p.chunk_cap < 1) p.chunk_cap = 1;
  p.Vpad = round_up(V, 8);
  p.nslots = ceil_div(V, kSliceVocab);
  p.slot_cap = lse_slots(V);
  plan_backward_blocks(N > 0 ? N : 1, p.Vpad, d, p.chunk_cap, eb, &p.bw_rows, &p.bw_width);
  p.bw_pitch = fkl::round_up(p.bw_width, 64);
  p.gh_splits = grad_hidden_splits(p.bw_rows, p.bw_width, d);
  p.pair_log2 = pair_bucket_log2(V);
  const bool pairs = p.pair_log2 >= 0;
  p.n_vb = pairs ? ceil_div(V, int64_t(1) << p.pair_log2) : 0;
  p.n_rt = pairs ? ceil_div(N, 256) : 0;
  p.pair_cap = 256 * (int64_t(K) + 1);
  const size_t pstart_bytes = static_cast<size_t>(p.n_rt) * (p.n_vb + 1) * 4;
  const size_t pentry_bytes = static_cast<size_t>(p.n_rt) * p.pair_cap * 4;

  size_t off = 0;
  p.f_part = off;
  off = align_up(off + static_cast<size_t>(p.slot_cap) * p.chunk_cap * 8);
  p.f_part_ce = off;  // temperature-1 partials (cross-entropy term at T != 1)
  off = align_up(off + static_cast<size_t>(p.slot_cap) * p.chunk_cap * 8);
  p.f_rowloss = off;
  off = align_up(off + static_cast<size_t>(N) * 4);
  p.f_topkz = off;
  off = align_up(off + static_cast<size_t>(N) * K * 4);
  p.f_zy = off;  // z at the labels
  off = align_up(off + static_cast<size_t>(N) * 4);
  p.f_pstart = off;
  off = align_up(off + pstart_bytes);
  p.f_pentry = off;
  off = align_up(off + pentry_bytes);
  p.f_flag = off;
  off = align_up(off + 4);
  p.f_total = off;

  const size_t rows = static_cast<size_t>(p.bw_rows);
  off = 0;
  p.b_G = off;
  off = align_up(off + rows * p.bw_pitch * eb);
  p.b_ghacc = off;
  off = align_up(off + rows * d * 4 * static_cast<size_t>(p.gh_splits));
  p.b_pcoef = off;
  off = align_up(off + rows * K * 4);
  p.b_acoef = off;
  off = align_up(off + rows * 4);
  p.b_lse2 = off;
  off = align_up(off + rows * 4);
  p.b_zk = off;
  off = align_up(off + rows * K * 4);
  p.b_bcoef = off;
  off = align_up(off + rows * 4);
  p.b_lse12 = off;
  off = align_up(off + rows * 4);
  p.b_ycoef = off;
  off = align_up(off + rows * 4);
  p.b_zy = off;
  off = align_up(off + rows * 4);
  p.b_tcoef = off;
  off = align_up(off + rows * 4);
  p.b_pstart = off;
  off = align_up(off + pstart_bytes);
  p.b_pentry = off;
  off = align_up(off + pentry_bytes);
  p.b_sub = off;  // exact-entry constants, K + 1 per row
  off = align_up(off + (pairs ? rows * (K + 1) * 4 : 0));
  p.b_tmul = off;
  off = align_up(off + (pairs ? rows * (K + 1) * 4 : 0));
  p.b_flag = off;
  off = align_up(off + 4);
  p.b_total = off;
  return p;
}

// Kept logits: each row padded to a multiple of 64 elements (128-byte lines in bf16).
int64_t keep_pitch(int64_t V) { return fkl::round_up(V, 64); }
size_t keep_bytes(int64_t N, int64_t V, int32_t dtype) {
  return static_cast<size_t>(N) * static_cast<size_t>(keep_pitch(V)) * (dtype == FKL_BF16 ? 2 : 4);
}

// The gradient products read 256-row tiles of the kept rows through 32-bit
// buffer offsets.
int32_t check_keep(int64_t V, int32_t dtype) {
  const int64_t eb = dtype == FKL_BF16 ? 2 : 4;
  if (256 * keep_pitch(V) * eb > kMaxBlockBytes)
    return fail(FKL_E_UNSUPPORTED, "vocabulary too large to keep the logits (V = %lld)",
                (long long)V);
  return FKL_OK;
}

// Workspace of fkl_backward_keep: per-row teacher coefficients, z at the ids
// and the fp32 grad_hidden accumulator, for all N rows.
struct KeepPlan {
  size_t pcoef, acoef, lse2, zk, ghacc, bcoef, lse12, ycoef, zy, tcoef, flag, total;
};
KeepPlan make_keep_plan(int64_t N, int64_t d, int32_t K) {
  KeepPlan q{};
  const size_t n = static_cast<size_t>(N);
  size_t off = 0;
  q.pcoef = off;
  off = align_up(off + n * K * 4);
  q.acoef = off;
  off = align_up(off + n * 4);
  q.lse2 = off;
  off = align_up(off + n * 4);
  q.zk = off;
  off = align_up(off + n * K * 4);
  q.ghacc = off;
  off = align_up(off + n * d * 4);
  q.bcoef = off;
  off = align_up(off + n * 4);
  q.lse12 = off;
  off = align_up(off + n * 4);
  q.ycoef = off;
  off = align_up(off + n * 4);
  q.zy = off;
  off = align_up(off + n * 4);
  q.tcoef = off;
  off = align_up(off + n * 4);
  q.flag = off;
  off = align_up(off + 4);
  q.total = off;
  return q;
}

// Loss options: their pointers' alignment, alpha, and (backward) lse1 when
// the cross-entropy term has its own softmax.
int32_t check_options(const fkl_loss_options* o, float T, bool backward) {
  if (!o) return FKL_OK;
  if (!std::isfinite(o->alpha)) return fail(FKL_E_ARG, "alpha must be finite");
  if (!aligned(o->row_weight, 4) || !aligned(o->labels, 4) || !aligned(o->lse1, 4) ||
      !aligned(o->teacher_lse, 4))
    return fail(FKL_E_ARG, "row_weight, labels, lse1 and teacher_lse must be 4-byte aligned");
  if (backward && o->labels && T != 1.0f && !o->lse1)
    return fail(FKL_E_ARG, "lse1 (from the forward) is required with labels when T != 1");
  return FKL_OK;
}

// fkl_forward and fkl_forward_keep: the chunk loop, with the logits kept in
// `logits` (N rows of keep_pitch(V) elements) when it is non-null.
// ---- the static scratch of fkl_forward_noalloc
//
// A file-scope device array stands in for the workspace argument, for callers
// that cannot allocate. In host code the name `scratch` is only a stand-in:
// the array's device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed to kernels. Every call on a device shares its copy.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch, looked up on its first use.
// A non-null stream must belong to the current device.
int32_t static_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FKL_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(FKL_E_UNSUPPORTED, "device index %d beyond %d", dev, kMaxScratchDevices);
  if (s) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return fail(FKL_E_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(FKL_E_ARG, "the stream belongs to device %d, the current device is %d",
                  static_cast<int>(sdev), dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FKL_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FKL_OK;
}

// With use_static, the workspace arguments are ignored and the current
// device's static scratch is used instead (looked up after every argument
// check, so a rejected call touches no device).
int32_t forward_impl(const void* hidden, const void* weight, const int32_t* topk_idx,
                     const float* topk_logit, float T, int64_t chunk, int64_t N, int64_t d,
                     int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                     const fkl_loss_options* o, float* loss, float* lse, float* row_loss,
                     float* topk_z, void* logits, size_t logits_bytes, void* workspace,
                     size_t workspace_bytes, void* stream, bool use_static = false) {
  int32_t r = check_shapes(N, d, V, K, chunk, dtype);
  if (r) return r;
  if (!std::isfinite(T) || !(T > 0.0f)) return fail(FKL_E_ARG, "T must be finite and > 0");
  if ((flags & ~FKL_FLAG_VALIDATE_IDX) != 0) return fail(FKL_E_ARG, "unknown forward flag bits");
  if (use_static) {
    workspace = nullptr;
    workspace_bytes = kStaticScratchBytes;
  }
  if (!loss || !weight || (!workspace && !use_static)) return fail(FKL_E_ARG, "null pointer argument");
  if (N > 0 && (!hidden || !topk_idx || !topk_logit || !lse))
    return fail(FKL_E_ARG, "null pointer argument");
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16))
    return fail(FKL_E_ARG, "hidden, weight and workspace must be 16-byte aligned");
  if (!aligned(topk_idx, 4) || !aligned(topk_logit, 4) || !aligned(loss, 4) || !aligned(lse, 4) ||
      !aligned(row_loss, 4) || !aligned(topk_z, 4))
    return fail(FKL_E_ARG, "fp32/int32 arrays must be 4-byte aligned");
  r = check_options(o, T, false);
  if (r) return r;
  const int64_t zpitch = keep_pitch(V);
  if (logits) {
    r = check_keep(V, dtype);
    if (r) return r;
    if (!aligned(logits, 16)) return fail(FKL_E_ARG, "logits must be 16-byte aligned");
    const size_t need = keep_bytes(N, V, dtype);
    if (logits_bytes < need)
      return fail(FKL_E_WORKSPACE, "kept logits need %zu bytes, got %zu", need, logits_bytes);
  }
  const Plan p = make_plan(N, d, V, K, chunk, dtype);
  if (workspace_bytes < p.f_total)
    return fail(FKL_E_WORKSPACE, "forward workspace needs %zu bytes, %s %zu", p.f_total,
                use_static ? "the static scratch holds" : "got", workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_static) {
    r = static_scratch(s, &workspace);
    if (r) return r;
  }
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  (void)hipGetLastError();

  if (N == 0) {
    fkl::launch_fill_f32(loss, 1, 0.0f, s);
    return hip_check("forward (empty batch)");
  }
  const int32_t* labels = o ? o->labels : nullptr;
  if (flags & FKL_FLAG_VALIDATE_IDX) {
    r = validate_ids(topk_idx, N, K, V, reinterpret_cast<int32_t*>(ws + p.f_flag), s, labels);
    if (r) return r;
  }
  float2* part = reinterpret_cast<float2*>(ws + p.f_part);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + p.f_rowloss);
  float* zk = topk_z ? topk_z : reinterpret_cast<float*>(ws + p.f_topkz);
  const float c2 = 1.4426950408889634f / T;
  // a second set of partials at temperature 1 when T != 1 and something needs
  // that softmax: the cross-entropy term, or the caller's lse1 output
  const bool two_sm = (labels || (o && o->lse1)) && T != 1.0f;
  fkl::MergeOpts mo{};
  mo.part_ce = two_sm ? reinterpret_cast<float2*>(ws + p.f_part_ce) : nullptr;
  mo.labels = labels;
  mo.row_weight = o ? o->row_weight : nullptr;
  mo.a_kl = labels ? o->alpha : 1.0f;
  mo.a_ce = labels ? 1.0f - o->alpha : 0.0f;
  mo.lse1 = o ? o->lse1 : nullptr;
  mo.teacher_lse = o ? o->teacher_lse : nullptr;

  float* zy = reinterpret_cast<float*>(ws + p.f_zy);
  if (labels) mo.zy = zy;
  // z at the teacher ids (and labels): taken from the logit tiles through the
  // pair index, or gathered by separate dot products for vocabularies too
  // wide to bucket
  fkl::PairIndex pi{};
  if (p.pair_log2 >= 0) {
    int32_t* pstart = reinterpret_cast<int32_t*>(ws + p.f_pstart);
    uint32_t* pentry = reinterpret_cast<uint32_t*>(ws + p.f_pentry);
    fkl::launch_pair_index(topk_idx, labels, N, K, V, p.pair_log2, p.n_vb, pstart, pentry,
                           p.pair_cap, zk, zy, s);
    pi = fkl::PairIndex{pstart, pentry, p.n_vb, p.pair_cap, p.pair_log2, K};
  } else {
    fkl::launch_gather_dot(dtype, weight, hidden, topk_idx, d, 0, N, K, zk, s);
    if (labels) fkl::launch_gather_dot(dtype, weight, hidden, labels, d, 0, N, 1, zy, s);
  }
  for (int64_t row0 = 0; row0 < N; row0 += p.chunk_cap) {
    const int64_t nrows = (N - row0) < p.chunk_cap ? (N - row0) : p.chunk_cap;
    fkl::launch_logits_lse(dtype, weight, hidden, d, V, row0, nrows, c2, part, p.chunk_cap,
                           const_cast<float2*>(mo.part_ce), logits, zpitch,
                           p.pair_log2 >= 0 ? &pi : nullptr, zk, zy, s);
    fkl::launch_merge_loss(part, p.chunk_cap, p.nslots, zk, topk_logit, row0, nrows, K, T, lse, rl,
                           mo, s);
  }
  fkl::launch_reduce_loss(rl, N, loss, s);
  return hip_check("forward launch");
}

}  // namespace

extern "C" {

int32_t fkl_abi_version(void) { return FKL_ABI_VERSION; }

const char* fkl_status_string(int32_t status) {
  switch (status) {
    case FKL_OK: return "ok";
    case FKL_E_ARG: return "invalid argument";
    case FKL_E_UNSUPPORTED: return "unsupported configuration";
    case FKL_E_WORKSPACE: return "workspace too small";
    case FKL_E_HIP: return "HIP runtime error";
    case FKL_E_INDEX: return "invalid teacher id";
    default: return "unknown status";
  }
}

const char* fkl_last_error(void) { return g_last_error; }

int32_t fkl_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                           int32_t dtype, size_t* fwd_bytes, size_t* bwd_bytes) {
  g_last_error[0] = 0;
  const int32_t r = check_shapes(N, d, V, K, chunk, dtype);
  if (r) return r;
  const Plan p = make_plan(N, d, V, K, chunk, dtype);
  if (fwd_bytes) *fwd_bytes = p.f_total;
  if (bwd_bytes) *bwd_bytes = p.b_total;
  return FKL_OK;
}

int32_t fkl_forward(const void* hidden, const void* weight, const int32_t* topk_idx,
                    const float* topk_logit, float T, int64_t chunk, int64_t N, int64_t d,
                    int64_t V, int32_t K, int32_t dtype, uint32_t flags, float* loss, float* lse,
                    float* row_loss, float* topk_z, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_last_error[0] = 0;
  return forward_impl(hidden, weight, topk_idx, topk_logit, T, chunk, N, d, V, K, dtype, flags,
                      nullptr, loss, lse, row_loss, topk_z, nullptr, 0, workspace,
                      workspace_bytes, stream);
}

int32_t fkl_forward_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                       const float* topk_logit, float T, int64_t chunk, int64_t N, int64_t d,
                       int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                       const fkl_loss_options* opts, float* loss, float* lse, float* row_loss,
                       float* topk_z, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return forward_impl(hidden, weight, topk_idx, topk_logit, T, chunk, N, d, V, K, dtype, flags,
                      opts, loss, lse, row_loss, topk_z, nullptr, 0, workspace, workspace_bytes,
                      stream);
}

int32_t fkl_forward_keep(const void* hidden, const void* weight, const int32_t* topk_idx,
                         const float* topk_logit, float T, int64_t chunk, int64_t N, int64_t d,
                         int64_t V, int32_t K, int32_t dtype, uint32_t flags, float* loss,
                         float* lse, float* row_loss, float* topk_z, void* logits,
                         size_t logits_bytes, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_last_error[0] = 0;
  if (!logits && N > 0) return fail(FKL_E_ARG, "null pointer argument (logits)");
  return forward_impl(hidden, weight, topk_idx, topk_logit, T, chunk, N, d, V, K, dtype, flags,
                      nullptr, loss, lse, row_loss, topk_z, logits, logits_bytes, workspace,
                      workspace_bytes, stream);
}

int32_t fkl_forward_keep_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                            const float* topk_logit, float T, int64_t chunk, int64_t N,
                            int64_t d, int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                            const fkl_loss_options* opts, float* loss, float* lse,
                            float* row_loss, float* topk_z, void* logits, size_t logits_bytes,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!logits && N > 0) return fail(FKL_E_ARG, "null pointer argument (logits)");
  return forward_impl(hidden, weight, topk_idx, topk_logit, T, chunk, N, d, V, K, dtype, flags,
                      opts, loss, lse, row_loss, topk_z, logits, logits_bytes, workspace,
                      workspace_bytes, stream);
}

int32_t fkl_forward_noalloc(const void* hidden, const void* weight, const int32_t* topk_idx,
                            const float* topk_logit, float T, int64_t chunk, int64_t N,
                            int64_t d, int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                            float* loss, float* lse, float* row_loss, float* topk_z,
                            void* stream) {
  g_last_error[0] = 0;
  return forward_impl(hidden, weight, topk_idx, topk_logit, T, chunk, N, d, V, K, dtype, flags,
                      nullptr, loss, lse, row_loss, topk_z, nullptr, 0, nullptr, 0, stream,
                      /*use_static=*/true);
}

static int32_t backward_impl(const void* hidden, const void* weight, const int32_t* topk_idx,
                             const float* topk_logit, const float* lse, const float* topk_z,
                             const float* grad_loss, float T, int64_t chunk, int64_t N,
                             int64_t d, int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                             const fkl_loss_options* o, void* grad_hidden, float* grad_weight,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int32_t r = check_shapes(N, d, V, K, chunk, dtype);
  if (r) return r;
  if (!std::isfinite(T) || !(T > 0.0f)) return fail(FKL_E_ARG, "T must be finite and > 0");
  if ((flags & ~(FKL_FLAG_VALIDATE_IDX | FKL_FLAG_ACCUMULATE_GRAD_W)) != 0)
    return fail(FKL_E_ARG, "unknown backward flag bits");
  if (!weight || !grad_weight || !workspace) return fail(FKL_E_ARG, "null pointer argument");
  if (N > 0 && (!hidden || !topk_idx || !topk_logit || !lse || !grad_hidden))
    return fail(FKL_E_ARG, "null pointer argument");
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16) ||
      !aligned(grad_hidden, 16) || !aligned(grad_weight, 16))
    return fail(FKL_E_ARG, "hidden, weight, gradients and workspace must be 16-byte aligned");
  if (!aligned(topk_idx, 4) || !aligned(topk_logit, 4) || !aligned(lse, 4) || !aligned(topk_z, 4) ||
      !aligned(grad_loss, 4))
    return fail(FKL_E_ARG, "fp32/int32 arrays must be 4-byte aligned");
  r = check_options(o, T, true);
  if (r) return r;
  const Plan p = make_plan(N, d, V, K, chunk, dtype);
  if (workspace_bytes < p.b_total)
    return fail(FKL_E_WORKSPACE, "backward workspace needs %zu bytes, got %zu", p.b_total,
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const bool accumulate = (flags & FKL_FLAG_ACCUMULATE_GRAD_W) != 0;
  (void)hipGetLastError();

  if (N == 0) {
    if (!accumulate) fkl::launch_fill_f32(grad_weight, V * d, 0.0f, s);
    return hip_check("backward (empty batch)");
  }
  const int32_t* labels = o ? o->labels : nullptr;
  const float* row_weight = o ? o->row_weight : nullptr;
  const bool two_sm = labels && T != 1.0f;
  const float a_kl = labels ? o->alpha : 1.0f, a_ce = labels ? 1.0f - o->alpha : 0.0f;
  if (flags & FKL_FLAG_VALIDATE_IDX) {
    r = validate_ids(topk_idx, N, K, V, reinterpret_cast<int32_t*>(ws + p.b_flag), s, labels);
    if (r) return r;
  }
  void* G = ws + p.b_G;
  float* bcoef = reinterpret_cast<float*>(ws + p.b_bcoef);
  float* lse12 = reinterpret_cast<float*>(ws + p.b_lse12);
  float* ycoef = reinterpret_cast<float*>(ws + p.b_ycoef);
  float* zy = reinterpret_cast<float*>(ws + p.b_zy);
  const float* tlse = o ? o->teacher_lse : nullptr;
  float* tcoef = reinterpret_cast<float*>(ws + p.b_tcoef);
  float* ghacc = reinterpret_cast<float*>(ws + p.b_ghacc);
  float* pcoef = reinterpret_cast<float*>(ws + p.b_pcoef);
  float* acoef = reinterpret_cast<float*>(ws + p.b_acoef);
  float* lse2 = reinterpret_cast<float*>(ws + p.b_lse2);
  float* zk_ws = reinterpret_cast<float*>(ws + p.b_zk);
  const float c2 = 1.4426950408889634f / T;
  const int64_t eb = dtype == FKL_BF16 ? 2 : 4;
  // the exact G entries at the teacher ids and labels: written by the logit
  // tiles through the pair index, or by the separate fixup kernel for
  // vocabularies too wide to bucket
  const bool pairs = p.pair_log2 >= 0;
  fkl::PairIndex pi{};
  float* sub = reinterpret_cast<float*>(ws + p.b_sub);
  float* tmul = reinterpret_cast<float*>(ws + p.b_tmul);
  if (pairs) {
    int32_t* pstart = reinterpret_cast<int32_t*>(ws + p.b_pstart);
    uint32_t* pentry = reinterpret_cast<uint32_t*>(ws + p.b_pentry);
    fkl::launch_pair_index(topk_idx, labels, N, K, V, p.pair_log2, p.n_vb, pstart, pentry,
                           p.pair_cap, nullptr, nullptr, s);
    pi = fkl::PairIndex{pstart, pentry, p.n_vb, p.pair_cap, p.pair_log2, K};
  }

  for (int64_t row0 = 0; row0 < N; row0 += p.bw_rows) {
    const int64_t nrows = (N - row0) < p.bw_rows ? (N - row0) : p.bw_rows;
    const float* zk;
    if (topk_z) {
      zk = topk_z + row0 * K;
    } else {
      // recompute z at the ids for this block into the workspace (rows 0..nrows)
      fkl::launch_gather_dot(dtype, weight, static_cast<const unsigned char*>(hidden) + row0 * d * eb,
                             topk_idx + row0 * K, d, 0, nrows, K, zk_ws, s);
      zk = zk_ws;
    }
    if (labels)  // z at the labels of this block (rows 0..nrows)
      fkl::launch_gather_dot(dtype, weight, static_cast<const unsigned char*>(hidden) + row0 * d * eb,
                             labels + row0, d, 0, nrows, 1, zy, s);
    fkl::launch_bwd_prep(topk_logit, lse, grad_loss, row0, nrows, K, T, row_weight, labels, a_kl,
                         a_ce, o ? o->lse1 : nullptr, two_sm, tlse, zk, pcoef, acoef, lse2,
                         two_sm ? bcoef : nullptr, two_sm ? lse12 : nullptr,
                         labels ? ycoef : nullptr, tlse ? tcoef : nullptr, topk_idx + row0 * K,
                         pairs ? sub : nullptr, pairs ? tmul : nullptr, s);
    fkl::RowCoef rc{pcoef, acoef, lse2, two_sm ? bcoef : nullptr, two_sm ? lse12 : nullptr,
                    labels ? ycoef : nullptr, labels ? labels + row0 : nullptr,
                    labels ? zy : nullptr, tlse ? tcoef : nullptr};
    const fkl::PairPatch pp{pi, zk, zy, sub, tmul};  // zk, zy: the block's rows
    for (int64_t v0 = 0; v0 < p.Vpad; v0 += p.bw_width) {
      const int64_t Vw = (p.Vpad - v0) < p.bw_width ? (p.Vpad - v0) : p.bw_width;
      const int64_t Vlim = (V - v0) < Vw ? (V - v0) : Vw;
      fkl::launch_gprod(dtype, weight, hidden, d, V, v0, Vw, p.bw_pitch, row0, nrows, c2, rc, G,
                        pairs ? &pp : nullptr, s);
      if (!pairs)
        fkl::launch_fixup(dtype, G, p.bw_pitch, v0, Vw, topk_idx, zk, rc, row0, nrows, K, c2, s);
      fkl::launch_grad_hidden(dtype, G, p.bw_pitch, weight, d, v0, Vw, Vlim, nrows, v0 > 0, ghacc,
                              p.gh_splits, s);
      fkl::launch_grad_w(dtype, G, p.bw_pitch, hidden, d, v0, Vw, Vlim, row0, nrows,
                         accumulate || row0 > 0, grad_weight, s);
    }
    fkl::launch_reduce_grad_hidden(dtype, ghacc, p.gh_splits, nrows, d, grad_hidden, row0, s);
  }
  return hip_check("backward launch");
}

int32_t fkl_backward(const void* hidden, const void* weight, const int32_t* topk_idx,
                     const float* topk_logit, const float* lse, const float* topk_z,
                     const float* grad_loss, float T, int64_t chunk, int64_t N, int64_t d,
                     int64_t V, int32_t K, int32_t dtype, uint32_t flags, void* grad_hidden,
                     float* grad_weight, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return backward_impl(hidden, weight, topk_idx, topk_logit, lse, topk_z, grad_loss, T, chunk, N,
                       d, V, K, dtype, flags, nullptr, grad_hidden, grad_weight, workspace,
                       workspace_bytes, stream);
}

int32_t fkl_backward_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                        const float* topk_logit, const float* lse, const float* topk_z,
                        const float* grad_loss, float T, int64_t chunk, int64_t N, int64_t d,
                        int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                        const fkl_loss_options* opts, void* grad_hidden, float* grad_weight,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return backward_impl(hidden, weight, topk_idx, topk_logit, lse, topk_z, grad_loss, T, chunk, N,
                       d, V, K, dtype, flags, opts, grad_hidden, grad_weight, workspace,
                       workspace_bytes, stream);
}

int32_t fkl_keep_sizes(int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype,
                       size_t* logits_bytes, size_t* bwd_bytes) {
  g_last_error[0] = 0;
  int32_t r = check_shapes(N, d, V, K, 1, dtype);
  if (r) return r;
  r = check_keep(V, dtype);
  if (r) return r;
  if (logits_bytes) *logits_bytes = keep_bytes(N, V, dtype);
  if (bwd_bytes) *bwd_bytes = make_keep_plan(N, d, K).total;
  return FKL_OK;
}

static int32_t backward_keep_impl(const void* hidden, const void* weight,
                                  const int32_t* topk_idx, const float* topk_logit,
                                  const float* lse, const float* topk_z, const float* grad_loss,
                                  float T, int64_t N, int64_t d, int64_t V, int32_t K,
                                  int32_t dtype, uint32_t flags, const fkl_loss_options* o,
                                  void* logits, size_t logits_bytes, void* grad_hidden,
                                  float* grad_weight, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int32_t r = check_shapes(N, d, V, K, 1, dtype);
  if (r) return r;
  r = check_keep(V, dtype);
  if (r) return r;
  if (!std::isfinite(T) || !(T > 0.0f)) return fail(FKL_E_ARG, "T must be finite and > 0");
  if ((flags & ~(FKL_FLAG_VALIDATE_IDX | FKL_FLAG_ACCUMULATE_GRAD_W)) != 0)
    return fail(FKL_E_ARG, "unknown backward flag bits");
  if (!weight || !grad_weight || !workspace) return fail(FKL_E_ARG, "null pointer argument");
  if (N > 0 && (!hidden || !topk_idx || !topk_logit || !lse || !grad_hidden || !logits))
    return fail(FKL_E_ARG, "null pointer argument");
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16) ||
      !aligned(grad_hidden, 16) || !aligned(grad_weight, 16) || !aligned(logits, 16))
    return fail(FKL_E_ARG,
                "hidden, weight, logits, gradients and workspace must be 16-byte aligned");
  if (!aligned(topk_idx, 4) || !aligned(topk_logit, 4) || !aligned(lse, 4) || !aligned(topk_z, 4) ||
      !aligned(grad_loss, 4))
    return fail(FKL_E_ARG, "fp32/int32 arrays must be 4-byte aligned");
  r = check_options(o, T, true);
  if (r) return r;
  const size_t need = keep_bytes(N, V, dtype);
  if (logits_bytes < need)
    return fail(FKL_E_WORKSPACE, "kept logits need %zu bytes, got %zu", need, logits_bytes);
  const KeepPlan q = make_keep_plan(N, d, K);
  if (workspace_bytes < q.total)
    return fail(FKL_E_WORKSPACE, "backward workspace needs %zu bytes, got %zu", q.total,
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const bool accumulate = (flags & FKL_FLAG_ACCUMULATE_GRAD_W) != 0;
  (void)hipGetLastError();

  if (N == 0) {
    if (!accumulate) fkl::launch_fill_f32(grad_weight, V * d, 0.0f, s);
    return hip_check("backward (empty batch)");
  }
  const int32_t* labels = o ? o->labels : nullptr;
  const bool two_sm = labels && T != 1.0f;
  const float a_kl = labels ? o->alpha : 1.0f, a_ce = labels ? 1.0f - o->alpha : 0.0f;
  if (flags & FKL_FLAG_VALIDATE_IDX) {
    r = validate_ids(topk_idx, N, K, V, reinterpret_cast<int32_t*>(ws + q.flag), s, labels);
    if (r) return r;
  }
  float* pcoef = reinterpret_cast<float*>(ws + q.pcoef);
  float* acoef = reinterpret_cast<float*>(ws + q.acoef);
  float* lse2 = reinterpret_cast<float*>(ws + q.lse2);
  float* ghacc = reinterpret_cast<float*>(ws + q.ghacc);
  const float c2 = 1.4426950408889634f / T;
  const int64_t eb = dtype == FKL_BF16 ? 2 : 4;
  const int64_t zpitch = keep_pitch(V);
  const int64_t zld = zpitch * eb;

  const float* zk = topk_z;
  if (!zk) {
    float* zk_ws = reinterpret_cast<float*>(ws + q.zk);
    fkl::launch_gather_dot(dtype, weight, hidden, topk_idx, d, 0, N, K, zk_ws, s);
    zk = zk_ws;
  }
  float* bcoef = reinterpret_cast<float*>(ws + q.bcoef);
  float* lse12 = reinterpret_cast<float*>(ws + q.lse12);
  float* ycoef = reinterpret_cast<float*>(ws + q.ycoef);
  float* zy = reinterpret_cast<float*>(ws + q.zy);
  const float* tlse = o ? o->teacher_lse : nullptr;
  float* tcoef = reinterpret_cast<float*>(ws + q.tcoef);
  if (labels) fkl::launch_gather_dot(dtype, weight, hidden, labels, d, 0, N, 1, zy, s);
  fkl::launch_bwd_prep(topk_logit, lse, grad_loss, 0, N, K, T, o ? o->row_weight : nullptr, labels,
                       a_kl, a_ce, o ? o->lse1 : nullptr, two_sm, tlse, zk, pcoef, acoef, lse2,
                       two_sm ? bcoef : nullptr, two_sm ? lse12 : nullptr,
                       labels ? ycoef : nullptr, tlse ? tcoef : nullptr, topk_idx, nullptr,
                       nullptr, s);
  const fkl::RowCoef rc{pcoef, acoef, lse2, two_sm ? bcoef : nullptr, two_sm ? lse12 : nullptr,
                        labels ? ycoef : nullptr, labels, labels ? zy : nullptr,
                        tlse ? tcoef : nullptr};
  fkl::launch_g_from_z(dtype, logits, zpitch, V, topk_idx, zk, rc, N, K, c2, s);
  // grad_hidden over all rows in one launch (tiles of 256 rows reach 256 * zld bytes)
  fkl::launch_grad_hidden(dtype, logits, zpitch, weight, d, 0, zpitch, V, N, false, ghacc, 1, s);
  fkl::launch_reduce_grad_hidden(dtype, ghacc, 1, N, d, grad_hidden, 0, s);
  // grad_W over row blocks whose rows stay within the 32-bit offsets of both
  // operands (the kept rows and the hidden rows)
  const int64_t rmax = kMaxBlockBytes / (zld > d * eb ? zld : d * eb);
  const int64_t nb = fkl::ceil_div(N, rmax);
  int64_t rb = fkl::round_up(fkl::ceil_div(N, nb), 64);
  if (rb > rmax) rb = fkl::ceil_div(N, nb);
  const unsigned char* zb = static_cast<const unsigned char*>(logits);
  for (int64_t row0 = 0; row0 < N; row0 += rb) {
    const int64_t nrows = (N - row0) < rb ? (N - row0) : rb;
    fkl::launch_grad_w(dtype, zb + row0 * zld, zpitch, hidden, d, 0, zpitch, V, row0, nrows,
                       accumulate || row0 > 0, grad_weight, s);
  }
  return hip_check("backward launch");
}

int32_t fkl_backward_keep(const void* hidden, const void* weight, const int32_t* topk_idx,
                          const float* topk_logit, const float* lse, const float* topk_z,
                          const float* grad_loss, float T, int64_t N, int64_t d, int64_t V,
                          int32_t K, int32_t dtype, uint32_t flags, void* logits,
                          size_t logits_bytes, void* grad_hidden, float* grad_weight,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return backward_keep_impl(hidden, weight, topk_idx, topk_logit, lse, topk_z, grad_loss, T, N, d,
                            V, K, dtype, flags, nullptr, logits, logits_bytes, grad_hidden,
                            grad_weight, workspace, workspace_bytes, stream);
}

int32_t fkl_backward_keep_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                             const float* topk_logit, const float* lse, const float* topk_z,
                             const float* grad_loss, float T, int64_t N, int64_t d, int64_t V,
                             int32_t K, int32_t dtype, uint32_t flags,
                             const fkl_loss_options* opts, void* logits, size_t logits_bytes,
                             void* grad_hidden, float* grad_weight, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return backward_keep_impl(hidden, weight, topk_idx, topk_logit, lse, topk_z, grad_loss, T, N, d,
                            V, K, dtype, flags, opts, logits, logits_bytes, grad_hidden,
                            grad_weight, workspace, workspace_bytes, stream);
}

int32_t fkl_timing_enable(int32_t on) { return fkl::timing_set(on != 0) ? 1 : 0; }

int32_t fkl_timing_reset(void) {
  fkl::timing_reset();
  return FKL_OK;
}

int32_t fkl_timing_read(int32_t kernel, int64_t* launches, double* total_ms) {
  g_last_error[0] = 0;
  if (!fkl::timing_read(kernel, launches, total_ms))
    return fail(FKL_E_ARG, "unknown kernel id %d", kernel);
  return FKL_OK;
}

int32_t fkl_kernel_count(void) { return fkl::KID_COUNT; }

const char* fkl_kernel_name(int32_t kernel) { return fkl::kernel_name(kernel); }

}  // extern "C"
