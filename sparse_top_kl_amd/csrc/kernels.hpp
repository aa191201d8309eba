// Host-side launchers for the loss kernels (internal to libfkl).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkl {

// Options of the loss beyond the plain KL (forward side), per chunk of rows:
// per-row weights, hard labels (< 0: none) with z at the label, the mixing
// weights of the KL and cross-entropy terms, and the temperature-1 partials
// (present when labels are given and T != 1, else lse1 = lse).
struct MergeOpts {
  const float2* part_ce;     // [slot][row] partials at temperature 1, or null
  const float* zy;           // [rows] z at the label, or null (no labels)
  const int32_t* labels;     // [rows] or null
  const float* row_weight;   // [rows] or null (weight 1)
  float a_kl, a_ce;          // weights of the KL and cross-entropy terms
  float* lse1;               // [rows] out: ln sum exp(z) at temperature 1, or null
  const float* teacher_lse;  // [rows] teacher's full-vocabulary lse at T (tail bucket), or null
};

// Per-row coefficients of the logit gradient (backward), rows of one block:
//   dense G = acoef * 2^(z*c2 - lse2) [+ bcoef * 2^(z*log2(e) - lse1_2)]
//   at the teacher ids minus pcoef_k plus (tail bucket) tcoef * 2^(z*c2 - lse2)
//   per cached copy of the id, at the label minus ycoef.
struct RowCoef {
  const float* pcoef;      // [rows][K]
  const float* acoef;      // [rows]
  const float* lse2;       // [rows]
  const float* bcoef;      // [rows] or null (one softmax)
  const float* lse1_2;     // [rows] or null
  const float* ycoef;      // [rows] or null (no labels)
  const int32_t* labels;   // [rows] or null
  const float* zy;         // [rows] z at the label, or null
  const float* tcoef;      // [rows] or null (no tail bucket)
};

// Teacher-id pairs of the batch, bucketed so that a logit tile finds the
// pairs it holds in one contiguous range: for each tile of 256 rows (global
// row / 256) the pairs sorted by vocabulary bucket (id >> bw_log2), with
// start[t][b] .. start[t][b + 1] the bucket's entries in the tile's block of
// `cap` entries. An entry packs the pair's entry index k (bits 0-12; k = K is
// the row's label when labels are indexed), its row within the tile (bits
// 13-20) and the id's low 11 bits (21-31), which fix the id inside any window
// of fewer than 2048 ids. Order inside a bucket is unspecified (each pair has
// its own output).
struct PairIndex {
  const int32_t* start;   // [n_rt][n_vb + 1]
  const uint32_t* entry;  // [n_rt][cap]
  int64_t n_vb;           // vocabulary buckets
  int64_t cap;            // entries per row tile: 256 * Kp
  int32_t bw_log2;        // bucket width 2^bw_log2 (32 .. 512)
  int32_t K;              // teacher entries per row (pair K is the label)
};
constexpr int kPairMaxBuckets = 16384;  // buckets one row tile sorts in LDS
// Bucket width (log2) for a vocabulary of V ids: the smallest power of two
// >= 32 with at most kPairMaxBuckets buckets; -1 if V needs buckets wider than 512.
inline int pair_bucket_log2(int64_t V) {
  for (int b = 5; b <= 9; ++b)
    if (((V + (int64_t(1) << b) - 1) >> b) <= kPairMaxBuckets) return b;
  return -1;
}

// Builds the pair index of rows [0, N) (ids [N][K], optional labels [N]; a
// label < 0 or an id outside [0, V) is no pair: its z output is set to 0 in
// zk [N][K] / zy [N] instead). One workgroup per row tile.
void launch_pair_index(const int32_t* idx, const int32_t* labels, int64_t N, int K, int64_t V,
                       int bw_log2, int64_t n_vb, int32_t* start, uint32_t* entry, int64_t cap,
                       float* zk, float* zy, hipStream_t s);

// Rows of a (vocab-slice, token) partial: running max and sum of 2^(z*c2).
constexpr int kSliceVocab = 128;  // vocabulary entries per partial slot

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// Number of partial slots per token (one per 128-wide vocabulary slice).
inline int64_t lse_slots(int64_t V) { return ceil_div(V, 256) * 2; }

// Forward, per chunk: partial (max, sum) of 2^(z * c2) per (vocab slice, token).
// With Z non-null the chunk's logits are also kept: Z[row0 + r][v] (pitch zpitch
// elements of the dtype) = z rounded to the dtype for v < V, zero for V <= v < zpitch.
// With part_ce non-null, partials at temperature 1 are written there too.
// With pi non-null the tile also writes z at the teacher-id pairs of its rows
// and vocabulary: zk[r][k] (global row r) and, for label pairs, zy[r].
void launch_logits_lse(int dtype, const void* W, const void* H, int64_t d, int64_t V,
                       int64_t row0, int64_t nrows, float c2, float2* part, int64_t part_ld,
                       float2* part_ce, void* Z, int64_t zpitch, const PairIndex* pi, float* zk,
                       float* zy, hipStream_t s);
// z at the teacher ids for rows [row0, row0 + nrows) (an id < 0 gives 0).
void launch_gather_dot(int dtype, const void* W, const void* H, const int32_t* idx, int64_t d,
                       int64_t row0, int64_t nrows, int K, float* zk, hipStream_t s);
// Merge partials into lse, teacher softmax and per-row loss for one chunk.
// (opts pointers are indexed by absolute row.)
void launch_merge_loss(const float2* part, int64_t part_ld, int64_t nslots, const float* zk,
                       const float* logit, int64_t row0, int64_t nrows, int K, float T,
                       float* lse, float* row_loss, const MergeOpts& opts, hipStream_t s);
// loss = sum of row_loss in a fixed order (fp64 accumulation).
void launch_reduce_loss(const float* row_loss, int64_t N, float* loss, hipStream_t s);

// Backward, per chunk.
// Coefficients of rows [row0, row0 + nrows) into the block arrays (row 0 =
// row0): row_weight, labels and lse1 are indexed by absolute row; bcoef,
// lse1_2 and ycoef may be null (not needed); two_sm selects the separate
// temperature-1 softmax of the cross-entropy term.
// With teacher_lse (absolute rows) the tail bucket's coefficients need zk
// (block rows) and go to tcoef.
// With sub / tmul non-null (pitch K + 1 per row) also the per-pair constants of
// the exact entries (PairPatch); idx starts at the block's first row.
void launch_bwd_prep(const float* logit, const float* lse, const float* grad_loss, int64_t row0,
                     int64_t nrows, int K, float T, const float* row_weight,
                     const int32_t* labels, float a_kl, float a_ce, const float* lse1,
                     bool two_sm, const float* teacher_lse, const float* zk, float* pcoef,
                     float* acoef, float* lse2, float* bcoef, float* lse1_2, float* ycoef,
                     float* tcoef, const int32_t* idx, float* sub, float* tmul, hipStream_t s);
// Exact entries of G at the teacher-id and label pairs (backward): the entry
// of pair (r, k) is dense(z) - sub[k] + tmul[k] 2^(z c2 - lse2) with z the
// gathered logit; sub and tmul are [rows][K + 1] (entry K is the label's, NaN
// in sub when the label is also a teacher id, whose entries then write it).
// zk [rows][K], zy [rows], sub and tmul start at the block's first row.
struct PairPatch {
  PairIndex pi;
  const float* zk;
  const float* zy;
  const float* sub;
  const float* tmul;
};
// Recompute the logit block rows [row0, row0 + nrows) x vocabulary [v0, v0 + Vw) into
// the dense part of G (pitch gpitch elements); with pp non-null, then the exact
// entries at the pairs inside the tile.
void launch_gprod(int dtype, const void* W, const void* H, int64_t d, int64_t V, int64_t v0,
                  int64_t Vw, int64_t gpitch, int64_t row0, int64_t nrows, float c2,
                  const RowCoef& rc, void* G, const PairPatch* pp, hipStream_t s);
// Exact G entries at the teacher ids and the label that fall inside the slice.
void launch_fixup(int dtype, void* G, int64_t gpitch, int64_t v0, int64_t Vw, const int32_t* idx,
                  const float* zk, const RowCoef& rc, int64_t row0, int64_t nrows, int K,
                  float c2, hipStream_t s);
// Kept logits -> logit gradient in place, rows [0, nrows) of Z (pitch zpitch elements),
// teacher-id entries included; idx, zk, pcoef, acoef and lse2 start at row 0 of Z.
void launch_g_from_z(int dtype, void* Z, int64_t zpitch, int64_t V, const int32_t* idx,
                     const float* zk, const RowCoef& rc, int64_t nrows, int K, float c2,
                     hipStream_t s);
// acc[nrows][d] (+)= G_block . W[v0 : v0 + Vw]  (Vlim entries of the slice lie below V);
// with splits > 1 the slice's columns are cut in `splits` parts contracted into
// `splits` copies of acc (stride nrows * d), to be summed by the reduction.
void launch_grad_hidden(int dtype, const void* G, int64_t gpitch, const void* W, int64_t d,
                        int64_t v0, int64_t Vw, int64_t Vlim, int64_t nrows, bool accumulate,
                        float* acc, int64_t splits, hipStream_t s);
void launch_reduce_grad_hidden(int dtype, const float* part, int64_t splits, int64_t nrows,
                               int64_t d, void* grad_hidden, int64_t row0, hipStream_t s);
// grad_W[v0 : v0 + Vlim] (+)= G_block^T . H[row0 : row0 + nrows].
void launch_grad_w(int dtype, const void* G, int64_t gpitch, const void* H, int64_t d,
                   int64_t v0, int64_t Vw, int64_t Vlim, int64_t row0, int64_t nrows,
                   bool accumulate, float* grad_w, hipStream_t s);
// The same product with its rows split in `splits` equal parts contracted in
// parallel, split i into out + i * out_split_stride (rows [0, Vlim) of each).
void launch_grad_w_split(int dtype, const void* G, int64_t gpitch, const void* H, int64_t d,
                         int64_t Vw, int64_t Vlim, int64_t row0, int64_t nrows, int64_t splits,
                         bool accumulate, float* out, int64_t out_split_stride, hipStream_t s);

// Teacher top-K cache, per chunk of rows [row0, row0 + nrows): the chunk's
// fp32 logits LT[v][r] (pitch lt_ld floats) and per (row, 128-vocab slice)
// maxima smax[r][slot] (pitch sm_ld) ...
// With part non-null also the LSE partials at c2 = log2(e)/T ([slot][lt_ld]).
void launch_teacher_logits(int dtype, const void* W, const void* H, int64_t d, int64_t V,
                           int64_t row0, int64_t nrows, float* LT, int64_t lt_ld,
                           uint32_t* smax, int64_t sm_ld, float c2, float2* part,
                           hipStream_t s);
// out[r] = natural-log log-sum-exp of row r's slice partials.
void launch_merge_lse_rows(const float2* part, int64_t part_ld, int64_t nslots, int64_t nrows,
                           float* out, hipStream_t s);
// ... then per row the K largest (ids, values) sorted, ties to the lower id;
// theta [nrows], cand [nrows][topk_capacity()] and count [nrows] are scratch.
void launch_topk_select(const float* LT, int64_t lt_ld, int64_t V, const uint32_t* smax,
                        int64_t sm_ld, int64_t nslots, int64_t nrows, int K, uint32_t* theta,
                        uint64_t* cand, uint32_t* count, int32_t* out_idx, float* out_val,
                        hipStream_t s);
int topk_capacity();

// Utilities.
void launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
void launch_validate_idx(const int32_t* idx, int64_t N, int K, int64_t V, bool allow_negative,
                         int32_t* flag, hipStream_t s);

// ---- student-renormalised loss (renorm.hip)
constexpr int kRenormMaxK = 1024;  // cached entries per row
constexpr int64_t kRenormMaxD = 8192;  // hidden size (eight columns per thread, 1024 threads)
constexpr int kRenormMaxSeg = 2048;    // sorted pairs per grad_W chunk (at most)
// pairs per chunk: 64 shares of 30 with the shares' pieces fit four
// 256-thread workgroups in a CU's 160 KiB of LDS
constexpr int kRenormSeg = 1920;
constexpr int kRenormSliceCols = 64;   // grad_W columns per slice of the sorted walk

// grad_W of the renormalised loss: a stable counting sort of the N * K (row,
// entry) pairs by id in nb blocks of rows_per_block rows, then sums over
// chunks of seg sorted pairs, slice by slice of kRenormSliceCols columns.
constexpr int32_t kRenormHotCap = 2048;  // ids summed by the dense product (at most)
constexpr int32_t kRenormHotMin = 64;    // pairs an id needs to be one of them

struct RenormSortPlan {
  int64_t nb, rows_per_block, seg, nchunks;
  int64_t nslices;   // ceil(d / kRenormSliceCols)
  int64_t hot_max;   // ids the dense product can take: one round of 256 x 256 tiles
  int64_t hot_rows;  // rows per dense-product block
  int64_t hot_splits;  // row splits of the product, each into its own copy of the output
};
// Workspace arrays of launch_renorm_grad_w.
struct RenormBuffers {
  int32_t* hist;        // [nb * V] per-block id counters
  int32_t* total;       // [V] pairs per id
  int32_t* start;       // [V + 1] cold bucket starts
  int32_t* srow;        // [N * K] sorted cold pairs: row,
  int32_t* sid;         //   id
  float* scoef;         //   and coefficient
  unsigned char* hs;    // [nslices][N][kRenormSliceCols] hidden rows, slice-major
  int32_t* slot;        // [V] hot slot or -1
  int32_t* hot_ids;     // [hot_max]
  int32_t* info;        // [4] number of hot ids, tau
  int32_t* tsum;        // [2 * ceil(V / 8192)] hot ids and cold pairs per tile of ids
  float* partial;       // [2 * nchunks * d] chunk partials
  unsigned char* hot_c; // [hot_rows * hot_max] coefficients, input dtype
  float* hot_prod;      // [hot_splits * hot_max * d] C^T H, one copy per split
};

// Forward (coef_mode false): row_loss[r] = w_r T^2 KL over the row's cached
// entries. Backward (coef_mode true): coef[r][k] = dloss/dz at entry k.
void launch_renorm_rows(bool coef_mode, const float* zk, const float* logit,
                        const float* row_weight, const float* grad_loss, int64_t N, int K,
                        float T, float* row_loss, float* coef, hipStream_t s);
// grad_hidden[r] = sum_k coef[r][k] W[idx[r][k]] in the input dtype.
void launch_renorm_grad_h(int dtype, const void* W, const int32_t* idx, const float* coef,
                          int64_t N, int K, int64_t d, void* gh, hipStream_t s);
// grad_W[v] (=, or += with acc_out) sum over pairs with id v of coef * H[row].
void launch_renorm_grad_w(int dtype, const void* H, const int32_t* idx, const float* coef,
                          int64_t N, int K, int64_t d, int64_t V, const RenormSortPlan& q,
                          const RenormBuffers& b, bool acc_out, float* gw, hipStream_t s);

}  // namespace fkl
