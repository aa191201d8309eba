// C ABI of the student-renormalised top-K loss: argument validation,
// workspace planning and the launches. Declarations, argument meanings,
// layouts and error behaviour are in include/fkl.h.
#include <hip/hip_runtime.h>

#include <cmath>

#include "api_common.hpp"
#include "fkl.h"
#include "kernels.hpp"

using namespace fkl_api;

namespace {

// Sizes of the pair sort: blocks of rows whose per-id counters take at most
// 256 MiB in all (and at least 16 rows each), chunks of kRenormSeg sorted
// pairs; rows per block of the hot ids' dense product.
fkl::RenormSortPlan sort_plan(int64_t N, int64_t d, int32_t K, int64_t V, int64_t eb) {
  fkl::RenormSortPlan q{};
  const int64_t nn = N > 0 ? N : 1;
  int64_t max_nb = (int64_t(256) << 20) / (V * 4);
  if (max_nb < 1) max_nb = 1;
  int64_t nb = fkl::ceil_div(nn, 16);
  if (nb > max_nb) nb = max_nb;
  q.rows_per_block = fkl::ceil_div(nn, nb);
  q.nb = fkl::ceil_div(nn, q.rows_per_block);
  const int64_t NK = N * K;
  q.seg = fkl::kRenormSeg;
  q.nchunks = NK > 0 ? fkl::ceil_div(NK, q.seg) : 0;
  q.nslices = fkl::ceil_div(d, fkl::kRenormSliceCols);
  // The dense product's output is hot_max x d. An id costs the product a full
  // column, 2 N d flops (~0.17 us at 32K x 3072), and the sorted walk one
  // d-wide row read per pair (~1.2 ns): the break-even is ~140 pairs, which on
  // Zipf ids of a 128K vocabulary the ~2000 most frequent ids reach. So at most
  // 2048 ids, and no more than one round of 256 x 256 tiles on the 256 CUs
  // (the product's time is set by its contraction over rows up to one round).
  const int64_t d_tiles = fkl::ceil_div(d, 256);
  q.hot_max = (256 / d_tiles) * 256;
  if (q.hot_max < 256) q.hot_max = 256;
  if (q.hot_max > fkl::kRenormHotCap) q.hot_max = fkl::kRenormHotCap;
  // row blocks of the product: 256 MiB of hot coefficients at most, equal sizes
  const int64_t max_rows = (int64_t(256) << 20) / (q.hot_max * eb);
  const int64_t nblk = fkl::ceil_div(nn, max_rows);
  q.hot_rows = fkl::ceil_div(nn, nblk);
  // its 256 x 256 tiles form groups of 32, one group per XCD: split the rows
  // so that the groups' copies fill the 8 XCDs (at least 1024 rows a split)
  const int64_t groups = fkl::ceil_div(q.hot_max / 256, 8) * fkl::ceil_div(d_tiles, 4);
  q.hot_splits = groups >= 8 ? 1 : 8 / groups;
  const int64_t by_rows = q.hot_rows / 1024 > 0 ? q.hot_rows / 1024 : 1;
  if (q.hot_splits > by_rows) q.hot_splits = by_rows;
  return q;
}

struct RenormPlan {
  fkl::RenormSortPlan sort;
  // forward workspace
  size_t f_zk, f_rowloss, f_flag, f_total;
  // backward workspace
  size_t b_coef, b_zk, b_hist, b_total_ids, b_start, b_srow, b_sid, b_scoef, b_hs, b_partial,
      b_slot, b_hot_ids, b_info, b_tsum, b_hot_c, b_hot_prod, b_flag, b_total;
};

RenormPlan make_renorm_plan(int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype) {
  RenormPlan p{};
  const int64_t eb = dtype == FKL_BF16 ? 2 : 4;
  p.sort = sort_plan(N, d, K, V, eb);
  const size_t NK = static_cast<size_t>(N) * K;
  size_t off = 0;
  p.f_zk = off;
  off = align_up(off + NK * 4);
  p.f_rowloss = off;
  off = align_up(off + static_cast<size_t>(N) * 4);
  p.f_flag = off;
  off = align_up(off + 4);
  p.f_total = off;
  off = 0;
  p.b_coef = off;
  off = align_up(off + NK * 4);
  p.b_zk = off;
  off = align_up(off + NK * 4);
  p.b_hist = off;
  off = align_up(off + static_cast<size_t>(p.sort.nb) * V * 4);
  p.b_total_ids = off;
  off = align_up(off + static_cast<size_t>(V) * 4);
  p.b_start = off;
  off = align_up(off + static_cast<size_t>(V + 1) * 4);
  p.b_srow = off;  // each padded by a quad for the walk's 16-byte loads
  off = align_up(off + NK * 4 + 16);
  p.b_sid = off;
  off = align_up(off + NK * 4 + 16);
  p.b_scoef = off;
  off = align_up(off + NK * 4 + 16);
  p.b_hs = off;
  off = align_up(off + static_cast<size_t>(N) * p.sort.nslices * fkl::kRenormSliceCols * eb);
  p.b_partial = off;
  off = align_up(off + static_cast<size_t>(2 * p.sort.nchunks) * d * 4);
  p.b_slot = off;
  off = align_up(off + static_cast<size_t>(V) * 4);
  p.b_hot_ids = off;
  off = align_up(off + static_cast<size_t>(p.sort.hot_max) * 4);
  p.b_info = off;
  off = align_up(off + 16);
  p.b_tsum = off;
  off = align_up(off + static_cast<size_t>(fkl::ceil_div(V, 8192)) * 2 * 4);
  p.b_hot_c = off;
  off = align_up(off + static_cast<size_t>(p.sort.hot_rows) * p.sort.hot_max * eb);
  p.b_hot_prod = off;
  off = align_up(off + static_cast<size_t>(p.sort.hot_splits) * p.sort.hot_max * d * 4);
  p.b_flag = off;
  off = align_up(off + 4);
  p.b_total = off;
  return p;
}

int32_t check_renorm(int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype) {
  int32_t r = check_shapes(N, d, V, K, 1, dtype);
  if (r) return r;
  if (K > fkl::kRenormMaxK)
    return fail(FKL_E_UNSUPPORTED, "K > %d is not supported here (got %d)", fkl::kRenormMaxK, K);
  if (d > fkl::kRenormMaxD)
    return fail(FKL_E_UNSUPPORTED, "d > %lld is not supported here (got %lld)",
                (long long)fkl::kRenormMaxD, (long long)d);
  if (N * static_cast<int64_t>(K) >= (int64_t(1) << 31))
    return fail(FKL_E_UNSUPPORTED, "N * K must stay below 2^31");
  return FKL_OK;
}

int32_t check_common(const void* hidden, const void* weight, const int32_t* idx,
                     const float* logit, int64_t N, float T, const float* row_weight,
                     const void* workspace) {
  if (!std::isfinite(T) || !(T > 0.0f)) return fail(FKL_E_ARG, "T must be finite and > 0");
  if (!weight || !workspace) return fail(FKL_E_ARG, "null pointer argument");
  if (N > 0 && (!hidden || !idx || !logit)) return fail(FKL_E_ARG, "null pointer argument");
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16))
    return fail(FKL_E_ARG, "hidden, weight and workspace must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(logit, 4) || !aligned(row_weight, 4))
    return fail(FKL_E_ARG, "fp32/int32 arrays must be 4-byte aligned");
  return FKL_OK;
}

}  // namespace

extern "C" int32_t fkl_renorm_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K,
                                             int32_t dtype, size_t* fwd_bytes,
                                             size_t* bwd_bytes) {
  g_last_error[0] = 0;
  const int32_t r = check_renorm(N, d, V, K, dtype);
  if (r) return r;
  const RenormPlan p = make_renorm_plan(N, d, V, K, dtype);
  if (fwd_bytes) *fwd_bytes = p.f_total;
  if (bwd_bytes) *bwd_bytes = p.b_total;
  return FKL_OK;
}

extern "C" int32_t fkl_renorm_forward(const void* hidden, const void* weight,
                                      const int32_t* topk_idx, const float* topk_logit, float T,
                                      int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype,
                                      uint32_t flags, const float* row_weight, float* loss,
                                      float* row_loss, float* topk_z, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  int32_t r = check_renorm(N, d, V, K, dtype);
  if (r) return r;
  r = check_common(hidden, weight, topk_idx, topk_logit, N, T, row_weight, workspace);
  if (r) return r;
  if ((flags & ~FKL_FLAG_VALIDATE_IDX) != 0) return fail(FKL_E_ARG, "unknown forward flag bits");
  if (!loss) return fail(FKL_E_ARG, "null pointer argument");
  if (!aligned(loss, 4) || !aligned(row_loss, 4) || !aligned(topk_z, 4))
    return fail(FKL_E_ARG, "fp32/int32 arrays must be 4-byte aligned");
  const RenormPlan p = make_renorm_plan(N, d, V, K, dtype);
  if (workspace_bytes < p.f_total)
    return fail(FKL_E_WORKSPACE, "forward workspace needs %zu bytes, got %zu", p.f_total,
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  (void)hipGetLastError();
  if (N == 0) {
    fkl::launch_fill_f32(loss, 1, 0.0f, s);
    return hip_check("renormalised forward (empty batch)");
  }
  if (flags & FKL_FLAG_VALIDATE_IDX) {
    r = validate_ids(topk_idx, N, K, V, reinterpret_cast<int32_t*>(ws + p.f_flag), s);
    if (r) return r;
  }
  float* zk = topk_z ? topk_z : reinterpret_cast<float*>(ws + p.f_zk);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + p.f_rowloss);
  fkl::launch_gather_dot(dtype, weight, hidden, topk_idx, d, 0, N, K, zk, s);
  fkl::launch_renorm_rows(false, zk, topk_logit, row_weight, nullptr, N, K, T, rl, nullptr, s);
  fkl::launch_reduce_loss(rl, N, loss, s);
  return hip_check("renormalised forward launch");
}

extern "C" int32_t fkl_renorm_backward(const void* hidden, const void* weight,
                                       const int32_t* topk_idx, const float* topk_logit,
                                       const float* topk_z, const float* grad_loss, float T,
                                       int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype,
                                       uint32_t flags, const float* row_weight, void* grad_hidden,
                                       float* grad_weight, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  int32_t r = check_renorm(N, d, V, K, dtype);
  if (r) return r;
  r = check_common(hidden, weight, topk_idx, topk_logit, N, T, row_weight, workspace);
  if (r) return r;
  if ((flags & ~(FKL_FLAG_ACCUMULATE_GRAD_W | FKL_FLAG_VALIDATE_IDX)) != 0)
    return fail(FKL_E_ARG, "unknown backward flag bits");
  if (!grad_weight || (N > 0 && !grad_hidden)) return fail(FKL_E_ARG, "null pointer argument");
  if (!aligned(grad_hidden, 16) || !aligned(grad_weight, 16))
    return fail(FKL_E_ARG, "grad_hidden and grad_weight must be 16-byte aligned");
  if (!aligned(topk_z, 4) || !aligned(grad_loss, 4))
    return fail(FKL_E_ARG, "fp32/int32 arrays must be 4-byte aligned");
  const RenormPlan p = make_renorm_plan(N, d, V, K, dtype);
  if (workspace_bytes < p.b_total)
    return fail(FKL_E_WORKSPACE, "backward workspace needs %zu bytes, got %zu", p.b_total,
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  (void)hipGetLastError();
  if (N > 0 && (flags & FKL_FLAG_VALIDATE_IDX)) {
    r = validate_ids(topk_idx, N, K, V, reinterpret_cast<int32_t*>(ws + p.b_flag), s);
    if (r) return r;
  }
  float* coef = reinterpret_cast<float*>(ws + p.b_coef);
  if (N > 0) {
    const float* zk = topk_z;
    if (!zk) {
      float* z = reinterpret_cast<float*>(ws + p.b_zk);
      fkl::launch_gather_dot(dtype, weight, hidden, topk_idx, d, 0, N, K, z, s);
      zk = z;
    }
    fkl::launch_renorm_rows(true, zk, topk_logit, row_weight, grad_loss, N, K, T, nullptr, coef,
                            s);
    fkl::launch_renorm_grad_h(dtype, weight, topk_idx, coef, N, K, d, grad_hidden, s);
  }
  fkl::RenormBuffers b{};
  b.hist = reinterpret_cast<int32_t*>(ws + p.b_hist);
  b.total = reinterpret_cast<int32_t*>(ws + p.b_total_ids);
  b.start = reinterpret_cast<int32_t*>(ws + p.b_start);
  b.srow = reinterpret_cast<int32_t*>(ws + p.b_srow);
  b.sid = reinterpret_cast<int32_t*>(ws + p.b_sid);
  b.scoef = reinterpret_cast<float*>(ws + p.b_scoef);
  b.hs = ws + p.b_hs;
  b.slot = reinterpret_cast<int32_t*>(ws + p.b_slot);
  b.hot_ids = reinterpret_cast<int32_t*>(ws + p.b_hot_ids);
  b.info = reinterpret_cast<int32_t*>(ws + p.b_info);
  b.tsum = reinterpret_cast<int32_t*>(ws + p.b_tsum);
  b.partial = reinterpret_cast<float*>(ws + p.b_partial);
  b.hot_c = ws + p.b_hot_c;
  b.hot_prod = reinterpret_cast<float*>(ws + p.b_hot_prod);
  fkl::launch_renorm_grad_w(dtype, hidden, topk_idx, coef, N, K, d, V, p.sort, b,
                            (flags & FKL_FLAG_ACCUMULATE_GRAD_W) != 0, grad_weight, s);
  return hip_check("renormalised backward launch");
}
