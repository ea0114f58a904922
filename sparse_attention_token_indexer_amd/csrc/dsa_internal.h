// Internal (host-side) interfaces between the C-ABI layer and the kernel
// translation units.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

enum ItemMode { MODE_RANGE = 0, MODE_POOLED = 1, MODE_LIST = 2, MODE_BLOCKS = 3 };

// Arguments of one score-and-select pass.  One workgroup scores `chunk` items of
// one query; items are mapped to key rows by `mode`:
//   RANGE   item u = token u of the query's sequence, u = 0..pos
//   POOLED  item b = pooled block b, b = 0..ceil((pos+1)/block)-1; the partial
//           last block (if any) is read from `partial` instead of `pooled`
//   LIST    item i = token list[t][i] (entries < 0 or > pos are skipped)
//   BLOCKS  item i = token list[t][i / block] * block + i % block (same rule)
struct SelArgs {
  const void* q;               // [nq, n_heads, D] bf16 bits or f32
  const float* w;              // [nq, n_heads]
  const void* keys;            // [n_seq, l_max, D]
  const uint16_t* pooled;      // [n_seq, m_max, D] bf16 (POOLED)
  const uint16_t* partial;     // [nq, D] bf16 (POOLED), may be null
  const int32_t* q_seq;        // [nq] or null (all 0)
  const int32_t* q_pos;        // [nq]
  const int32_t* heads;        // [nq, heads_stride] given heads, or null = all
  const float* route_part;     // [nq, route_splits, n_heads] router sums, or null
  int route_splits;            // (route_part given: heads are the top h_use by importance)
  int32_t* out_heads;          // [nq, h_use] routed heads or null (route_part given)
  float* out_importance;       // [nq, n_heads] router importance or null
  const int32_t* list;         // LIST / BLOCKS
  int nq, n_heads, h_use, heads_stride, head_dim, n_seq;
  int64_t l_max, m_max;
  int block, list_len, top_k, chunk, n_chunks;
  int f32;                     // inputs are float32
  int mode;
  int store_all;               // short pass: every item's (key, id) to cand, no emission
                               // (selected by the short-pass select kernel)
  // workspace
  uint2* cand;                 // [nq, n_chunks, chunk]
  uint32_t* cand_cnt;          // [nq, n_chunks]
  uint32_t* ghist;             // [nq, 4096]   (zeroed before the pass)
  // outputs
  int32_t* out_idx;            // [nq, top_k]
  float* out_score;            // [nq, top_k] or null
  // certified screening pass (RANGE mode over the screened heads): per query
  // {N+, N-, M} of the heads left out; the selection key of every item is its
  // lower bound, its upper bound goes to ub[t * ub_stride + item]
  const float* cert;           // [nq, 4] or null
  float* ub;                   // [nq, ub_stride]
  int64_t ub_stride;
  const int32_t* list_count;   // LIST: [nq] entries of each query's list, or null: list_len
};

// Certified exact top-k (bounds of the heads left out of a screening pass):
// the screened heads of every query, the bounds, and the survivors.
constexpr int kCertMaxHeads = 16;      // screened heads (the 16-row MFMA scorer)
// relative error margin of the bounds (fp32 rounding of the screened score,
// of the norms and of the full score is far below it)
constexpr float kCertRel = 1.0f / 4096.0f;
struct CertArgs {
  const uint16_t* q;           // [nq, n_heads, head_dim] bf16
  const float* w;              // [nq, n_heads]
  const int32_t* q_seq;        // [nq] or null
  const int32_t* q_pos;        // [nq]
  int nq, n_heads, head_dim, n_seq, h, top_k;
  int64_t l_max;
  int32_t* heads;              // [nq, h] screened heads (largest |w_j| ||q_j||, ties: lower j)
  float* cert;                 // [nq, 4] {N+, N-, M, 0}
  const int32_t* lb_idx;       // [nq, top_k] the screening pass's selection by lower bound
  const float* lb_score;       // [nq, top_k] its lower bounds
  const float* ub;             // [nq, l_max] upper bounds
  int32_t* list;               // [nq, l_max] survivors (first cnt[t] entries)
  uint32_t* cnt;               // [nq] survivor counts (zeroed before the call)
  int32_t* out_survivors;      // [nq] copy of cnt, or null
};
hipError_t launch_certify_heads(const CertArgs& a, hipStream_t stream);
hipError_t launch_certify_compact(const CertArgs& a, hipStream_t stream);
hipError_t launch_certify_counts(const CertArgs& a, hipStream_t stream);   // cnt -> out_survivors

// A selection pass is the score-and-emit kernel followed by the merge kernel,
// launched in that order on one stream.
hipError_t launch_score_emit(const SelArgs& a, hipStream_t stream);
hipError_t launch_merge(const SelArgs& a, hipStream_t stream);
// Short passes (at most kShortItems items per query): exact top-k of one
// query's (key, id) pairs in one workgroup.
constexpr int kShortItems = 16384;
hipError_t launch_select_short(const SelArgs& a, hipStream_t stream);
constexpr int kMaxChunks = 8192;        // chunks per query in one pass
constexpr int kMergeListCap = 12288;    // tie-bin entries resolved in LDS
size_t score_select_lds_bytes(int chunk, int f32, int head_dim);

// Clears `zero_words` 32-bit words at `zero` and, if `partial` is given, pools
// the partial last block of every query whose prefix does not end on a block
// boundary (mean over its valid tokens, rounded once to bf16).
struct PrepArgs {
  uint32_t* zero;
  size_t zero_words;
  const uint16_t* keys;        // [n_seq, l_max, D] bf16
  const int32_t* q_seq;
  const int32_t* q_pos;
  int nq, n_seq, head_dim, block;
  int64_t l_max;
  uint16_t* partial;           // [nq, D] or null
  int32_t* status;             // [nq] per-query status words cleared with the region, or null
};
hipError_t launch_prepare(const PrepArgs& a, hipStream_t stream);

hipError_t launch_mean_pool(const uint16_t* k, int n_seq, int64_t l_max, int head_dim, int block,
                            uint16_t* out, hipStream_t stream);

// MISA router: per-head importance from pooled keys and top-h head selection.
// The router kernel writes, per query and slice of pooled blocks, the per-head
// sums of max(0, q_j . kbar_b); the routed scoring pass adds the slices in slice
// order, weights by |w_j| and ranks the heads itself (route_heads below).
struct RouteArgs {
  const uint16_t* q;           // [nq, n_heads, D]
  const uint16_t* pooled;      // [n_seq, m_max, D]
  const uint16_t* partial;     // [nq, D] (by query) or [l_max, D] (by position), or null
  int partial_by_pos;          // partial holds the in-block prefix mean of every position
  const int32_t* q_seq;
  const int32_t* q_pos;
  int nq, n_heads, head_dim, n_seq, block, splits, blocks_per_split;
  int64_t l_max, m_max;
  float* part;                 // [nq, splits, n_heads] workspace
};
// out[p] = mean of the keys from the start of p's block to p, sequence 0, every
// position p < l_max (the pooled key of a prefix that ends inside a block),
// accumulated in float64 and rounded once to bf16 like the block means.
hipError_t launch_pool_prefix(const uint16_t* k, int64_t l_max, int head_dim, int block,
                              uint16_t* out, hipStream_t stream);
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

// Prefill-shaped dense pass: all queries on sequence 0, grouped by 8 rows.
struct PrefillArgs {
  const uint16_t* q;           // [nq, n_heads, D] bf16
  const float* w;              // [nq, n_heads]
  const uint16_t* keys;        // [1, l_max, D] bf16
  const int32_t* q_seq;        // [nq] or null
  const int32_t* q_pos;        // [nq]
  int nq, n_heads, head_dim, top_k;
  int64_t l_max;
  int64_t row_stride;          // floats per score row (l_max rounded up to 128)
  float* scores;               // [nq, row_stride] workspace (only u <= pos written)
  int32_t* rowmeta;            // [nq, 4] workspace: threshold bin, count above, count in bin
  int bin_bits;                // first-level histogram bits (dense: 12 up to 65535 keys per
                               // row, 11 beyond; routed: 10)
  int key_chunk;               // > 0 splits every row's keys into chunks of this many (a
                               // multiple of 128), one workgroup per (row group, chunk), and
                               // the select counts the rows itself (12-bit bins, parthist)
  const int32_t* heads;        // routed pass: [nq, heads_stride] head ids (first h_use used)
  int heads_stride, h_use;
  float* spare_row;            // [row_stride] scratch row taking the stores of rows that are
                               // not scored
  uint32_t* rowctl;            // key_chunk > 0: [nq, kRowCtlWords] the select's counters per
                               // row
  uint32_t* parthist;          // key_chunk > 0: [nq, row_parts, kBins / 2] each part's 12-bit
                               // histogram (16-bit counts)
  int row_parts;               // parts of kRowPartKeys keys per row (l_max rounded up)
  uint2* ties;                 // key_chunk > 0: [nq, kRowTieCap] entries of each row's
                               // threshold bin
  int32_t* out_idx;
  float* out_score;
};
// Select of rows whose keys were split over workgroups: every row in parts of
// kRowPartKeys keys, one workgroup each, in four kernels (count, threshold,
// emission, finish) whose boundaries carry the data between workgroups; per
// row kRowCtlWords words: [emitted entries, threshold bin entries, threshold
// bin, count above it, count in it] and padding, written by the threshold
// kernel.
constexpr int kRowPartKeys = 8192;
constexpr int kRowCtlWords = 8;
constexpr int kRowTieCap = 2048;
enum : int { RH_EMIT = 0, RH_TIES, RH_BSTAR, RH_ABOVE, RH_NB };
hipError_t launch_prefill_score(const PrefillArgs& a, hipStream_t stream);
// MISA on the prefill shape: rows scored with their h_use <= 8 routed heads,
// four rows per 32-row MFMA tile; 10-bit per-row histograms.
constexpr int kRoutedMaxHeads = 8;
hipError_t launch_prefill_routed_score(const PrefillArgs& a, hipStream_t stream);
// Top-h heads of every query from the router's per-slice sums (heads written
// to heads[t * heads_stride + rank], optionally out_heads / out_importance).
struct RouteHeadsArgs {
  const float* part;           // [nq, splits, n_heads]
  const float* w;              // [nq, n_heads]
  const int32_t* q_seq;
  const int32_t* q_pos;
  int nq, n_heads, splits, h_use, heads_stride, n_seq;
  int64_t l_max;
  int32_t* heads;              // [nq, heads_stride]
  int32_t* out_heads;          // [nq, h_use] or null
  float* out_importance;       // [nq, n_heads] or null
};
hipError_t launch_route_heads(const RouteHeadsArgs& a, hipStream_t stream);
hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t stream);

hipError_t launch_iou(const int32_t* a, const int32_t* b, int nq, int k, float* out,
                      hipStream_t stream);

}  // namespace dsa
