// Host-side model of every kernel launch of libdsa_indexer, for the bounds
// audit (tests/test_audit_cpu.py).  This file replaces the kernel translation
// units: the C-ABI layer (api.hip, compiled for the host only) plans the
// workspace and fills the launch arguments exactly as in the library, and each
// dsa::launch_* below, instead of launching, walks the kernel's grid on the
// host and derives from the kernel's index arithmetic the byte range of every
// global-memory pointer it reads or writes.  Each range must lie inside one
// buffer that the driver registered (inputs, outputs, the workspace at its
// planned size).  It also checks the grid covers the work (no item, chunk or
// block left without a workgroup), which the kernels assume.
//
// Values that kernels read from device memory are modelled as follows: q_seq
// and q_pos come from host copies the driver registers; values that an earlier
// kernel of the call produced (candidate lists, kept blocks, routed heads) are
// bounded by the consuming kernel's own checks, which the model restates.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <string>
#include <vector>

#include "../../sparse_attention_token_indexer_amd/csrc/dsa_hisa.h"
#include "../../sparse_attention_token_indexer_amd/csrc/dsa_internal.h"
#include "../../sparse_attention_token_indexer_amd/csrc/dsa_mla.h"

namespace {

struct Region {
  uintptr_t base;
  size_t bytes;
  std::string name;
};

std::vector<Region> g_regions;
std::map<uintptr_t, std::vector<int32_t>> g_ints;
std::vector<std::string> g_viol;
std::map<std::string, int64_t> g_launches;
std::string g_kernel;

void violation(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (g_viol.size() < 200) g_viol.push_back(g_kernel + ": " + buf);
}

// bytes [lo, hi) past p are accessed
void touch(const void* p, int64_t lo, int64_t hi, const char* what) {
  if (hi <= lo) return;
  if (!p) {
    violation("%s: NULL pointer accessed at [%lld, %lld)", what, (long long)lo, (long long)hi);
    return;
  }
  if (lo < 0) {
    violation("%s: negative offset %lld", what, (long long)lo);
    return;
  }
  const uintptr_t a = (uintptr_t)p + (uintptr_t)lo, b = (uintptr_t)p + (uintptr_t)hi;
  for (const Region& r : g_regions)
    if (a >= r.base && a < r.base + r.bytes) {
      if (b > r.base + r.bytes)
        violation("%s: [%llu, %llu) past the end of %s (%zu bytes)", what,
                  (unsigned long long)(a - r.base), (unsigned long long)(b - r.base),
                  r.name.c_str(), r.bytes);
      return;
    }
  violation("%s: address %#llx (+%lld) in no registered buffer", what, (unsigned long long)p,
            (long long)lo);
}

template <class T>
void touch_elems(const T* p, int64_t lo, int64_t hi, const char* what) {
  touch(p, lo * (int64_t)sizeof(T), hi * (int64_t)sizeof(T), what);
}

// a device int32 the kernel reads (its value from the registered host copy)
int32_t dev_int(const int32_t* p, int64_t i, const char* what) {
  touch_elems(p, i, i + 1, what);
  for (auto& kv : g_ints) {
    const uintptr_t b = kv.first;
    if ((uintptr_t)p >= b && (uintptr_t)p < b + kv.second.size() * 4) {
      const int64_t j = (int64_t)(((uintptr_t)p - b) / 4) + i;
      if (j >= 0 && j < (int64_t)kv.second.size()) return kv.second[(size_t)j];
    }
  }
  violation("%s: value at %#llx[%lld] has no registered host copy", what, (unsigned long long)p,
            (long long)i);
  return -1;
}

void begin(const char* k) {
  g_kernel = k;
  ++g_launches[k];
}

struct QRow {
  int seq;
  int64_t pos;
  bool ok;
};

QRow qrow(const int32_t* q_seq, const int32_t* q_pos, int t, int n_seq, int64_t l_max) {
  QRow r;
  r.seq = q_seq ? dev_int(q_seq, t, "q_seq") : 0;
  r.pos = dev_int(q_pos, t, "q_pos");
  r.ok = r.seq >= 0 && r.seq < n_seq && r.pos >= 0 && r.pos < l_max;
  return r;
}

// Scorer::init: the head rows of q and the weights of the heads in use (head
// ids < n_heads: all heads, or routed heads chosen among them)
void scorer_init(const void* q, size_t eb, const float* w, int t, int n_heads, int D, int h_use,
                 const int32_t* heads_given, int heads_stride) {
  touch(q, (int64_t)t * n_heads * D * eb, (int64_t)(t + 1) * n_heads * D * eb, "q rows");
  touch_elems(w, (int64_t)t * n_heads, (int64_t)(t + 1) * n_heads, "w");
  if (heads_given)
    touch_elems(heads_given, (int64_t)t * heads_stride, (int64_t)t * heads_stride + h_use, "heads");
  if (h_use > n_heads) violation("h_use %d > n_heads %d", h_use, n_heads);
}

// key rows [r0, r1] (inclusive) of sequence seq
void key_rows(const void* keys, size_t row_bytes, int seq, int64_t l_max, int64_t r0, int64_t r1,
              const char* what) {
  if (r1 < r0) return;
  if (r0 < 0 || r1 >= l_max) violation("%s: row %lld..%lld outside [0, %lld)", what,
                                       (long long)r0, (long long)r1, (long long)l_max);
  touch(keys, ((int64_t)seq * l_max + r0) * (int64_t)row_bytes,
        ((int64_t)seq * l_max + r1 + 1) * (int64_t)row_bytes, what);
}

int64_t n_items_of(const dsa::SelArgs& a, const QRow& r) {
  if (!r.ok) return 0;
  switch (a.mode) {
    case dsa::MODE_RANGE: return r.pos + 1;
    case dsa::MODE_POOLED: return (r.pos + a.block) / a.block;
    case dsa::MODE_LIST: return a.list_len;   // (a per-query count is clamped to list_len)
    default: return (int64_t)a.list_len * a.block;
  }
}

// the key rows that items [i0, i0 + n) of a query can address (item_of)
void items_rows(const dsa::SelArgs& a, int t, const QRow& r, int64_t i0, int64_t n) {
  const size_t eb = a.f32 ? 4 : 2;
  const size_t rb = eb * a.head_dim;
  switch (a.mode) {
    case dsa::MODE_RANGE:
      key_rows(a.keys, rb, r.seq, a.l_max, i0, i0 + n - 1, "key rows (range)");
      if (i0 + n - 1 > r.pos) violation("range item %lld past pos %lld", (long long)(i0 + n - 1), (long long)r.pos);
      break;
    case dsa::MODE_POOLED: {
      const int64_t last = i0 + n - 1;
      const bool part = a.partial && last == n_items_of(a, r) - 1 && ((r.pos + 1) % a.block) != 0;
      if (a.m_max < (r.pos + a.block) / a.block) violation("m_max %lld below the query's blocks", (long long)a.m_max);
      touch(a.pooled, ((int64_t)r.seq * a.m_max + i0) * (int64_t)rb,
            ((int64_t)r.seq * a.m_max + (part ? last : last + 1)) * (int64_t)rb, "pooled rows");
      if (part) touch(a.partial, (int64_t)t * rb, (int64_t)(t + 1) * rb, "partial row");
      break;
    }
    case dsa::MODE_LIST:
      touch_elems(a.list, (int64_t)t * a.list_len + i0, (int64_t)t * a.list_len + i0 + n, "list");
      // entries outside [0, pos] are replaced by row 0
      key_rows(a.keys, rb, r.seq, a.l_max, 0, r.pos, "key rows (list)");
      break;
    default:
      touch_elems(a.list, (int64_t)t * a.list_len + i0 / a.block,
                  (int64_t)t * a.list_len + (i0 + n - 1) / a.block + 1, "block list");
      key_rows(a.keys, rb, r.seq, a.l_max, 0, r.pos, "key rows (blocks)");
      break;
  }
}

}  // namespace

namespace dsa {

size_t score_select_lds_bytes(int chunk, int f32, int head_dim) {
  size_t b = (size_t)chunk * 4 + 4096 * 4 + 64 * 4;
  if (f32) b += (size_t)(64 * head_dim + 64) * 4;
  return b;
}

hipError_t launch_score_emit(const SelArgs& a, hipStream_t) {
  begin(a.store_all ? "k_score_emit(store_all)" : "k_score_emit");
  if (a.n_chunks > kMaxChunks) return hipErrorInvalidValue;
  if (a.f32 && a.mode != MODE_RANGE) return hipErrorInvalidValue;
  if (a.cert && (a.f32 || a.mode != MODE_RANGE || a.h_use < 1 || a.h_use > kCertMaxHeads || !a.ub ||
                 a.ub_stride < a.l_max))
    return hipErrorInvalidValue;
  const size_t eb = a.f32 ? 4 : 2;
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    const int64_t n_items = n_items_of(a, r);
    if (n_items == 0) {
      if (a.route_part) {
        if (a.out_heads) touch_elems(a.out_heads, (int64_t)t * a.h_use, (int64_t)(t + 1) * a.h_use, "out_heads");
        if (a.out_importance) touch_elems(a.out_importance, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "out_importance");
      }
      continue;
    }
    const int64_t n_chunks_t = (n_items + a.chunk - 1) / a.chunk;
    if (n_chunks_t > a.n_chunks)
      violation("query %d needs %lld chunks, the grid has %d", t, (long long)n_chunks_t, a.n_chunks);
    if (a.route_part) {
      touch_elems(a.route_part, (int64_t)t * a.route_splits * a.n_heads,
                  (int64_t)(t + 1) * a.route_splits * a.n_heads, "route_part");
      if (a.out_heads) touch_elems(a.out_heads, (int64_t)t * a.h_use, (int64_t)(t + 1) * a.h_use, "out_heads");
      if (a.out_importance) touch_elems(a.out_importance, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "out_importance");
    }
    if (a.mode == MODE_LIST && a.list_count)
      touch_elems(a.list_count, t, t + 1, "list count");
    scorer_init(a.q, eb, a.w, t, a.n_heads, a.head_dim, a.h_use, a.route_part ? nullptr : a.heads,
                a.heads_stride);
    if (a.cert) touch_elems(a.cert, (int64_t)t * 4, (int64_t)t * 4 + 3, "bounds");
    for (int c = 0; c < std::min<int64_t>(n_chunks_t, a.n_chunks); ++c) {
      const int64_t i0 = (int64_t)c * a.chunk;
      const int64_t n_c = std::min<int64_t>(n_items - i0, a.chunk);
      items_rows(a, t, r, i0, n_c);
      if (a.cert) touch_elems(a.ub, (int64_t)t * a.ub_stride + i0, (int64_t)t * a.ub_stride + i0 + n_c,
                              "upper bounds");
      const int64_t seg = ((int64_t)t * a.n_chunks + c) * a.chunk;
      touch_elems(a.cand, seg, seg + n_c, "candidate segment");
      if (!a.store_all) {
        touch_elems(a.ghist, (int64_t)t * 4096, (int64_t)(t + 1) * 4096, "global histogram");
        touch_elems(a.cand_cnt, (int64_t)t * a.n_chunks + c, (int64_t)t * a.n_chunks + c + 1, "segment count");
      }
    }
  }
  return hipSuccess;
}

hipError_t launch_merge(const SelArgs& a, hipStream_t) {
  begin("k_merge");
  if (a.n_chunks > kMaxChunks) return hipErrorInvalidValue;
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    const int64_t n_items = n_items_of(a, r);
    const int64_t n_chunks_t = (n_items + a.chunk - 1) / a.chunk;
    if (n_chunks_t > a.n_chunks) violation("query %d: %lld chunks > %d", t, (long long)n_chunks_t, a.n_chunks);
    touch_elems(a.ghist, (int64_t)t * 4096, (int64_t)(t + 1) * 4096, "global histogram");
    touch_elems(a.cand_cnt, (int64_t)t * a.n_chunks, (int64_t)t * a.n_chunks + n_chunks_t, "segment counts");
    // every count is clamped to the segment capacity
    touch_elems(a.cand, (int64_t)t * a.n_chunks * a.chunk,
                (int64_t)t * a.n_chunks * a.chunk + n_chunks_t * a.chunk, "candidates");
    touch_elems(a.out_idx, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_idx");
    if (a.out_score) touch_elems(a.out_score, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_score");
  }
  return hipSuccess;
}

hipError_t launch_certify_heads(const CertArgs& a, hipStream_t) {
  begin("k_certify_heads");
  if (a.nq < 1 || a.n_heads < 1 || a.n_heads > 64 || a.h < 1 || a.h > a.n_heads ||
      (a.head_dim != 64 && a.head_dim != 128))
    return hipErrorInvalidValue;
  for (int t = 0; t < a.nq; ++t) {
    touch_elems(a.q, (int64_t)t * a.n_heads * a.head_dim, (int64_t)(t + 1) * a.n_heads * a.head_dim,
                "q rows");
    touch_elems(a.w, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "w");
    touch_elems(a.heads, (int64_t)t * a.h, (int64_t)(t + 1) * a.h, "screened heads");
    touch_elems(a.cert, (int64_t)t * 4, (int64_t)t * 4 + 4, "bounds");
  }
  return hipSuccess;
}

hipError_t launch_certify_compact(const CertArgs& a, hipStream_t) {
  begin("k_certify_compact");
  if (a.nq < 1 || a.top_k < 1 || a.l_max < 1) return hipErrorInvalidValue;
  if ((a.l_max + 4095) / 4096 > 65535) return hipErrorInvalidValue;
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    if (!r.ok) continue;
    touch_elems(a.lb_idx, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "screening selection");
    touch_elems(a.lb_score, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "lower bounds");
    touch_elems(a.ub, (int64_t)t * a.l_max, (int64_t)t * a.l_max + r.pos + 1, "upper bounds");
    touch_elems(a.cnt, t, t + 1, "survivor count");
    // at most every key of the prefix survives
    touch_elems(a.list, (int64_t)t * a.l_max, (int64_t)t * a.l_max + r.pos + 1, "survivor list");
  }
  return hipSuccess;
}

hipError_t launch_certify_counts(const CertArgs& a, hipStream_t) {
  begin("k_certify_counts");
  if (a.nq < 1 || !a.out_survivors) return hipErrorInvalidValue;
  touch_elems(a.cnt, 0, a.nq, "survivor counts");
  touch_elems(a.out_survivors, 0, a.nq, "out_survivors");
  return hipSuccess;
}

hipError_t launch_select_short(const SelArgs& a, hipStream_t) {
  begin("k_select_short");
  if ((int64_t)a.n_chunks * a.chunk < 1) return hipErrorInvalidValue;
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    const int64_t n_items = n_items_of(a, r);
    const int64_t n = std::min<int64_t>(n_items, kShortItems);
    if (n_items > kShortItems) violation("query %d: %lld items in a short pass", t, (long long)n_items);
    if (n > (int64_t)a.n_chunks * a.chunk)
      violation("query %d: %lld items, %lld stored slots", t, (long long)n, (long long)a.n_chunks * a.chunk);
    touch_elems(a.cand, (int64_t)t * a.n_chunks * a.chunk, (int64_t)t * a.n_chunks * a.chunk + n, "stored pairs");
    touch_elems(a.out_idx, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_idx");
    if (a.out_score) touch_elems(a.out_score, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_score");
  }
  return hipSuccess;
}

hipError_t launch_prepare(const PrepArgs& a, hipStream_t) {
  begin("k_prepare");
  touch_elems(a.zero, 0, (int64_t)a.zero_words, "zeroed region");
  if (a.status) touch_elems(a.status, 0, a.nq, "status");
  if (a.partial)
    for (int t = 0; t < a.nq; ++t) {
      const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
      if (!r.ok) continue;
      const int64_t n = (r.pos + 1) % a.block;
      if (n == 0) continue;
      key_rows(a.keys, (size_t)a.head_dim * 2, r.seq, a.l_max, r.pos + 1 - n, r.pos, "partial block keys");
      touch_elems(a.partial, (int64_t)t * a.head_dim, (int64_t)(t + 1) * a.head_dim, "partial");
    }
  return hipSuccess;
}

hipError_t launch_mean_pool(const uint16_t* k, int n_seq, int64_t l_max, int head_dim, int block,
                            uint16_t* out, hipStream_t) {
  begin("k_mean_pool");
  const int64_t m_max = (l_max + block - 1) / block;
  if (n_seq > 0 && l_max > 0) {
    touch_elems(k, 0, (int64_t)n_seq * l_max * head_dim, "keys");
    touch_elems(out, 0, (int64_t)n_seq * m_max * head_dim, "pooled out");
  }
  return hipSuccess;
}

hipError_t launch_pool_prefix(const uint16_t* k, int64_t l_max, int head_dim, int block,
                              uint16_t* out, hipStream_t) {
  begin("k_pool_prefix");
  (void)block;
  touch_elems(k, 0, l_max * head_dim, "keys (sequence 0)");
  touch_elems(out, 0, l_max * head_dim, "prefix-pooled out");
  return hipSuccess;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t) {
  const bool prefill = a.splits == 1 && a.n_seq == 1 && a.partial_by_pos;
  begin(prefill ? "k_route_prefill" : a.splits == 1 ? "k_route_rows" : "k_route");
  const int D = a.head_dim;
  int64_t maxfull_all = 0;
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    if (prefill) {
      const bool ok = r.ok && r.seq == 0;
      if (ok) {
        touch_elems(a.q, (int64_t)t * a.n_heads * D, (int64_t)(t + 1) * a.n_heads * D, "q rows");
        maxfull_all = std::max<int64_t>(maxfull_all, (r.pos + 1) / a.block);
        if ((r.pos + 1) % a.block) touch_elems(a.partial, r.pos * D, (r.pos + 1) * D, "prefix-pooled row");
      } else {
        touch_elems(a.q, 0, (int64_t)a.n_heads * D, "q rows (stand-in)");
      }
      touch_elems(a.part, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "router sums");
      continue;
    }
    const int64_t M = r.ok ? (r.pos + a.block) / a.block : 0;
    if ((int64_t)a.splits * a.blocks_per_split < M)
      violation("query %d: %lld blocks, %d slices of %d", t, (long long)M, a.splits, a.blocks_per_split);
    const bool part = a.partial && r.ok && ((r.pos + 1) % a.block) != 0;
    if (M > 0) {
      touch_elems(a.q, (int64_t)t * a.n_heads * D, (int64_t)(t + 1) * a.n_heads * D, "q rows");
      if (a.m_max < M) violation("m_max %lld below %lld blocks", (long long)a.m_max, (long long)M);
      touch_elems(a.pooled, (int64_t)r.seq * a.m_max * D, ((int64_t)r.seq * a.m_max + (part ? M - 1 : M)) * D,
                  "pooled rows");
      if (part) {
        const int64_t pr = a.partial_by_pos ? r.pos : t;
        touch_elems(a.partial, pr * D, (pr + 1) * D, "partial row");
      }
    }
    touch_elems(a.part, (int64_t)t * a.splits * a.n_heads, (int64_t)(t + 1) * a.splits * a.n_heads,
                "router sums");
  }
  if (prefill && maxfull_all > 0) {
    if (maxfull_all > a.m_max) violation("pooled rows %lld > m_max %lld", (long long)maxfull_all, (long long)a.m_max);
    touch_elems(a.pooled, 0, maxfull_all * D, "pooled rows (sequence 0)");
  }
  return hipSuccess;
}

hipError_t launch_route_heads(const RouteHeadsArgs& a, hipStream_t) {
  begin("k_route_heads");
  if (a.n_heads > 64 || a.h_use > a.heads_stride) return hipErrorInvalidValue;
  for (int t = 0; t < a.nq; ++t) {
    (void)qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    touch_elems(a.part, (int64_t)t * a.splits * a.n_heads, (int64_t)(t + 1) * a.splits * a.n_heads, "router sums");
    touch_elems(a.w, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "w");
    if (a.out_importance) touch_elems(a.out_importance, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "out_importance");
    touch_elems(a.heads, (int64_t)t * a.heads_stride, (int64_t)t * a.heads_stride + a.h_use, "heads");
    if (a.out_heads) touch_elems(a.out_heads, (int64_t)t * a.h_use, (int64_t)(t + 1) * a.h_use, "out_heads");
  }
  return hipSuccess;
}

namespace {
// shared by the dense and routed prefill scorers: rows of one sequence in
// workgroups of `rows` rows; keys of a group clamp to its largest position
void prefill_scorer(const PrefillArgs& a, int rows, bool routed) {
  const int D = a.head_dim;
  const int64_t rb = (int64_t)D * 2;
  if (a.row_stride % 128 != 0 || a.row_stride < a.l_max || !a.spare_row) {
    violation("row stride %lld", (long long)a.row_stride);
    return;
  }
  touch_elems(a.spare_row, 0, a.row_stride, "spare row");
  const int groups = (a.nq + rows - 1) / rows;
  for (int grp = 0; grp < groups; ++grp) {
    int64_t maxpos = -1;
    std::vector<int64_t> pos(rows, -1);
    for (int i = 0; i < rows; ++i) {
      const int t = grp * rows + i;
      if (t >= a.nq) continue;
      const QRow r = qrow(a.q_seq, a.q_pos, t, 1, a.l_max);
      if (r.ok && r.seq == 0) pos[i] = r.pos;
      maxpos = std::max(maxpos, pos[i]);
    }
    if (maxpos < 0) continue;
    if (maxpos > 65535 && a.key_chunk == 0 && (routed || a.bin_bits == 12))
      violation("16-bit LDS row histograms with position %lld", (long long)maxpos);
    if (a.key_chunk < 0 || a.key_chunk % 128) violation("key chunk %d", a.key_chunk);
    const int64_t n_stages = maxpos / 128 + 1;
    touch(a.keys, 0, (maxpos + 1) * rb, "keys (sequence 0, clamped to the group's last position)");
    for (int i = 0; i < rows; ++i) {
      const int t = grp * rows + i;
      if (pos[i] < 0) continue;
      if (routed) {
        touch_elems(a.heads, (int64_t)t * a.heads_stride, (int64_t)t * a.heads_stride + a.h_use, "heads");
        touch_elems(a.q, (int64_t)t * a.n_heads * D, (int64_t)(t + 1) * a.n_heads * D, "q rows (routed heads)");
      } else {
        touch_elems(a.q, (int64_t)t * a.n_heads * D, (int64_t)(t + 1) * a.n_heads * D, "q rows");
      }
      touch_elems(a.w, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "w");
      // stores span whole stages of the group
      if (n_stages * 128 > a.row_stride) violation("stage stores past the row stride");
      // (split key chunks store whole stages inside [0, n_stages * 128) too)
      touch_elems(a.scores, (int64_t)t * a.row_stride, (int64_t)t * a.row_stride + n_stages * 128, "score row");
      if (a.key_chunk == 0) touch_elems(a.rowmeta, (int64_t)t * 4, (int64_t)t * 4 + 3, "row metadata");
    }
  }
}
}  // namespace

hipError_t launch_prefill_score(const PrefillArgs& a, hipStream_t) {
  begin("k_prefill_score");
  if (a.nq <= 0) return hipSuccess;
  if (a.row_stride % 128 != 0 || a.row_stride < a.l_max || !a.spare_row) return hipErrorInvalidValue;
  if (a.l_max >= (int64_t)1 << 30 || (a.bin_bits == 12 && a.l_max > 65535 && a.key_chunk == 0) ||
      (a.bin_bits != 12 && a.bin_bits != 11) || a.key_chunk < 0 || a.key_chunk % 128 ||
      (a.key_chunk > 0 && a.bin_bits != 12))
    return hipErrorInvalidValue;
  prefill_scorer(a, 8, false);
  return hipSuccess;
}

hipError_t launch_prefill_routed_score(const PrefillArgs& a, hipStream_t) {
  begin("k_prefill_routed_score");
  if (a.nq <= 0) return hipSuccess;
  const bool split = a.key_chunk > 0;
  if (a.h_use < 1 || a.h_use > kRoutedMaxHeads || a.key_chunk < 0 || a.key_chunk % 128 ||
      a.bin_bits != (split ? 12 : 10) || (!split && a.l_max > 65535) || a.l_max >= (int64_t)1 << 30)
    return hipErrorInvalidValue;
  if (a.row_stride % 128 != 0 || a.row_stride < a.l_max || !a.spare_row) return hipErrorInvalidValue;
  prefill_scorer(a, 32, true);
  return hipSuccess;
}

hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t) {
  begin("k_prefill_select");
  if (a.nq <= 0) return hipSuccess;
  if (a.key_chunk > 0) {
    // k_rows_count and k_rows_emit: grid (parts, rows), a part reads its
    // 16-byte pieces below n (the last one whole); the count stores the part's
    // histogram, the emission writes the output row and the tie buffer.
    // k_rows_threshold and k_rows_finish: one workgroup per row, on the row's
    // select words, part histograms, tie buffer and output row; the finish
    // reads the whole stored row when the tie bin overflows the buffer
    g_kernel = "k_rows_count / k_rows_threshold / k_rows_emit / k_rows_finish";
    const int64_t parts = (a.l_max + kRowPartKeys - 1) / kRowPartKeys;
    if (a.bin_bits != 12 || !a.rowctl || !a.parthist || !a.ties || a.row_parts < parts ||
        a.nq > 65535 || parts > 65535)
      return hipErrorInvalidValue;
    for (int t = 0; t < a.nq; ++t) {
      const QRow r = qrow(a.q_seq, a.q_pos, t, 1, a.l_max);
      touch_elems(a.out_idx, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_idx");
      if (a.out_score) touch_elems(a.out_score, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_score");
      if (!(r.ok && r.seq == 0)) continue;
      const int64_t n = r.pos + 1;
      touch_elems(a.rowctl, (int64_t)t * kRowCtlWords, (int64_t)(t + 1) * kRowCtlWords, "row select counters");
      const int64_t row_parts = (n + kRowPartKeys - 1) / kRowPartKeys;
      if (row_parts > parts) violation("row %d has %lld parts of %lld", t, (long long)row_parts, (long long)parts);
      // each part stores (and the threshold kernel reads) 2048 words of the row's
      if (n > a.top_k)
        touch_elems(a.parthist, (int64_t)t * a.row_parts * 2048,
                    ((int64_t)t * a.row_parts + row_parts) * 2048, "part histograms");
      const int64_t hi = 4 * ((n + 3) / 4);
      if (hi > a.row_stride) violation("row %d reads %lld floats of a %lld stride", t, (long long)hi, (long long)a.row_stride);
      touch_elems(a.scores, (int64_t)t * a.row_stride, (int64_t)t * a.row_stride + hi, "score row");
      touch_elems(a.ties, (int64_t)t * kRowTieCap, (int64_t)(t + 1) * kRowTieCap, "tie buffer");
    }
    return hipSuccess;
  }
  if (a.bin_bits != 12 && a.bin_bits != 11 && a.bin_bits != 10) return hipErrorInvalidValue;
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, 1, a.l_max);
    touch_elems(a.out_idx, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_idx");
    if (a.out_score) touch_elems(a.out_score, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_score");
    if (!(r.ok && r.seq == 0)) continue;
    const int64_t n = r.pos + 1;
    // 16-byte pieces, the last one clamped: up to 4 * ceil(n / 4) floats
    const int64_t hi = n <= a.top_k ? n : 4 * ((n + 3) / 4);
    if (hi > a.row_stride) violation("row %d reads %lld floats of a %lld stride", t, (long long)hi, (long long)a.row_stride);
    touch_elems(a.scores, (int64_t)t * a.row_stride, (int64_t)t * a.row_stride + hi, "score row");
    if (n > a.top_k && a.key_chunk == 0) touch_elems(a.rowmeta, (int64_t)t * 4, (int64_t)t * 4 + 3, "row metadata");
  }
  return hipSuccess;
}

hipError_t launch_iou(const int32_t* A, const int32_t* B, int nq, int k, float* out, hipStream_t) {
  begin("k_iou");
  if (k > 8192) return hipErrorInvalidValue;
  if (nq == 0) return hipSuccess;
  touch_elems(A, 0, (int64_t)nq * k, "a");
  touch_elems(B, 0, (int64_t)nq * k, "b");
  touch_elems(out, 0, nq, "out_iou");
  return hipSuccess;
}

hipError_t launch_hisa(const HisaArgs& a, hipStream_t) {
  begin("k_hisa");
  const int gmax = a.split ? std::max(a.groups1, a.groups2) : a.groups;
  const int gmin = a.split ? std::min(a.groups1, a.groups2) : a.groups;
  if (gmin < 1 || gmax > kHisaMaxGroups || a.ch1 < 32 || a.ch2 < 32 ||
      (a.split && (int64_t)a.nq * (a.groups1 + a.groups2) > 0x7FFFFFFF) ||
      a.ch1 > kHisaMaxChunk || a.ch2 > kHisaMaxChunk || a.ch1 % 32 || a.ch2 % 32 ||
      a.sblk_n < a.ch2 / a.block + 2 || a.nq < 1 || a.nq > 65535 || a.m_blocks < 1 ||
      a.m_blocks > kHisaMaxBlocks || (int64_t)a.m_blocks * a.block > kHisaRegKeys)
    return hipErrorInvalidValue;
  if (a.h_use < 1 || a.h_use > a.n_heads || (a.heads && a.heads_stride < a.h_use))
    return hipErrorInvalidValue;
  if (a.route_part && (a.heads || a.route_splits < 1 || a.n_heads > 64)) return hipErrorInvalidValue;
  const int D = a.head_dim;
  const int g1 = a.split ? a.groups1 : a.groups, g2 = a.split ? a.groups2 : a.groups;
  // LDS holds one workgroup's block ids: at most ch2 / block + 2 blocks per token-pass item
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    if (!r.ok) {
      touch_elems(a.blocks, (int64_t)t * a.m_blocks, (int64_t)(t + 1) * a.m_blocks, "kept blocks");
      if (a.out_block_score) touch_elems(a.out_block_score, (int64_t)t * a.m_blocks, (int64_t)(t + 1) * a.m_blocks, "block scores");
      if (a.route_part) {
        if (a.out_heads) touch_elems(a.out_heads, (int64_t)t * a.h_use, (int64_t)(t + 1) * a.h_use, "out_heads");
        if (a.out_importance) touch_elems(a.out_importance, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "out_importance");
      }
      continue;
    }
    const int64_t M = (r.pos + a.block) / a.block;
    const int64_t m1 = std::min<int64_t>(a.m_blocks, M);
    const int64_t n1 = (M + a.ch1 - 1) / a.ch1;
    const int64_t items2 = m1 * a.block;
    const int64_t n2 = (items2 + a.ch2 - 1) / a.ch2;
    // every pooled block and token item has a workgroup, and the block pass's
    // arrival count reaches n1 (else the token pass would wait in vain)
    if (n1 > g1) violation("query %d: %lld block-pass workgroups needed, %d launched", t, (long long)n1, g1);
    if (n2 > g2) violation("query %d: %lld token-pass workgroups needed, %d launched", t, (long long)n2, g2);
    if (a.m_max < M) violation("m_max %lld below %lld blocks", (long long)a.m_max, (long long)M);
    touch_elems(a.sync, (int64_t)t * kHisaSyncWords, (int64_t)(t + 1) * kHisaSyncWords, "sync words");
    touch_elems(a.bflag, (int64_t)t * a.m_blocks, (int64_t)t * a.m_blocks + m1, "kept-block flags");
    if (a.route_part) {
      touch_elems(a.route_part, (int64_t)t * a.route_splits * a.n_heads,
                  (int64_t)(t + 1) * a.route_splits * a.n_heads, "route_part");
      if (a.out_heads) touch_elems(a.out_heads, (int64_t)t * a.h_use, (int64_t)(t + 1) * a.h_use, "out_heads");
      if (a.out_importance) touch_elems(a.out_importance, (int64_t)t * a.n_heads, (int64_t)(t + 1) * a.n_heads, "out_importance");
    }
    scorer_init(a.q, 2, a.w, t, a.n_heads, D, a.h_use, a.heads, a.heads_stride);
    // block pass
    const bool part = ((r.pos + 1) % a.block) != 0;
    for (int64_t g = 0; g < std::min<int64_t>(n1, g1); ++g) {
      const int64_t i0 = g * a.ch1, nc = std::min<int64_t>(M - i0, a.ch1);
      const int64_t last = i0 + nc - 1;
      const bool pl = part && last == M - 1;
      touch_elems(a.pooled, ((int64_t)r.seq * a.m_max + i0) * D,
                  ((int64_t)r.seq * a.m_max + (pl ? last : last + 1)) * D, "pooled rows");
      if (pl) touch_elems(a.partial, (int64_t)t * D, (int64_t)(t + 1) * D, "partial row");
      touch_elems(a.cand1, ((int64_t)t * g1 + g) * a.ch1, ((int64_t)t * g1 + g) * a.ch1 + nc, "block candidates");
      touch_elems(a.cnt1, (int64_t)t * g1 + g, (int64_t)t * g1 + g + 1, "block candidate count");
    }
    // the selecting workgroup: counts, the first S entries of every segment,
    // then each segment up to its (clamped) count
    touch_elems(a.cnt1, (int64_t)t * g1, (int64_t)t * g1 + std::min<int64_t>(n1, g1), "block candidate counts");
    touch_elems(a.cand1, (int64_t)t * g1 * a.ch1, (int64_t)t * g1 * a.ch1 + std::min<int64_t>(n1, g1) * a.ch1,
                "block candidates (selection)");
    {
      const int S = std::min<int>(std::min<int>((int)kHisaCandCap / (int)n1, a.ch1), 128);
      const int U = (int)kHisaCandCap / 256;
      for (int tid = 0; tid < 256; ++tid)
        for (int u = 0; u < U; ++u) {
          const int f = tid + u * 256, sg = S > 0 ? f / S : 0;
          if (sg < n1) {
            const int64_t e = (int64_t)t * g1 * a.ch1 + (int64_t)sg * a.ch1 + (f - sg * S);
            if (f - sg * S >= a.ch1) violation("up-front read past a segment");
            touch_elems(a.cand1, e, e + 1, "block candidates (up-front read)");
          }
        }
    }
    touch_elems(a.blocks, (int64_t)t * a.m_blocks, (int64_t)(t + 1) * a.m_blocks, "kept blocks");
    if (a.out_block_score) touch_elems(a.out_block_score, (int64_t)t * a.m_blocks, (int64_t)(t + 1) * a.m_blocks, "block scores");
    // token pass
    for (int64_t g = 0; g < std::min<int64_t>(n2, g2); ++g) {
      const int64_t j0 = g * a.ch2, nc2 = std::min<int64_t>(items2 - j0, a.ch2);
      const int64_t li0 = j0 / a.block, li1 = (j0 + nc2 - 1) / a.block;
      if (li1 - li0 + 1 > a.sblk_n) violation("token item %lld spans %lld blocks, %d LDS slots", (long long)g, (long long)(li1 - li0 + 1), a.sblk_n);
      touch_elems(a.bflag, (int64_t)t * a.m_blocks + li0, (int64_t)t * a.m_blocks + li1 + 1, "kept-block flags (wait)");
      // kept block b < M, token u = b * block + r checked against pos
      key_rows(a.keys, (size_t)D * 2, r.seq, a.l_max, 0, r.pos, "key rows (kept blocks)");
      touch_elems(a.keys2, (int64_t)t * g2 * a.ch2 + j0, (int64_t)t * g2 * a.ch2 + j0 + nc2, "token keys");
    }
  }
  // k_hisa_topk: every query's first round of loads (token keys up to
  // m_blocks * block, the m_blocks kept blocks, its row and timeout word)
  // comes before the row is checked
  g_kernel = "k_hisa_topk";
  const int64_t G2 = a.split ? a.groups2 : a.groups;
  const int64_t items_max = (int64_t)a.m_blocks * a.block;
  if (items_max > G2 * a.ch2) violation("%lld token keys per query, %lld slots", (long long)items_max, (long long)(G2 * a.ch2));
  if (items_max > kHisaRegKeys) violation("%lld token keys > LDS entries", (long long)items_max);
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    touch_elems(a.keys2, (int64_t)t * G2 * a.ch2, (int64_t)t * G2 * a.ch2 + items_max, "token keys");
    touch_elems(a.blocks, (int64_t)t * a.m_blocks, (int64_t)(t + 1) * a.m_blocks, "kept blocks");
    touch_elems(a.sync, (int64_t)t * kHisaSyncWords + kHisaSyncTimeout,
                (int64_t)t * kHisaSyncWords + kHisaSyncTimeout + 1, "timeout word");
    if (a.out_status) touch_elems(a.out_status, t, t + 1, "out_status");
    touch_elems(a.out_idx, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_idx");
    if (a.out_score) touch_elems(a.out_score, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "out_score");
    (void)r;
  }
  return hipSuccess;
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t) {
  begin("k_sparse_mla");
  if (a.nq < 1 || a.top_k < 1 || a.top_k > kMlaMaxTopK || a.n_heads < 32 || a.n_heads > 128 ||
      a.n_heads % 32 || a.splits < 1 || a.splits > kMlaMaxSplits || a.tiles_per_split < 1 ||
      a.tiles_per_split > kMlaMaxTiles ||
      (int64_t)a.splits * a.tiles_per_split * kMlaTile < a.top_k ||
      (int64_t)a.nq * a.splits > 0x3FFFFFF ||
      mla_lds_bytes(a.n_heads, a.tiles_per_split) > 160 * 1024 ||
      (a.splits > 1 && (!a.part_o || !a.part_ml)))
    return hipErrorInvalidValue;
  for (int t = 0; t < a.nq; ++t) {
    const QRow r = qrow(a.q_seq, a.q_pos, t, a.n_seq, a.l_max);
    touch_elems(a.idx, (int64_t)t * a.top_k, (int64_t)(t + 1) * a.top_k, "index list");
    touch_elems(a.q, (int64_t)t * a.n_heads * kMlaDqk, (int64_t)(t + 1) * a.n_heads * kMlaDqk, "q rows");
    // listed rows outside [0, pos] are skipped; row 0 of the sequence stands in
    const int seq = r.ok ? r.seq : 0;
    touch_elems(a.kv, (int64_t)seq * a.l_max * kMlaDqk,
                ((int64_t)seq * a.l_max + (r.ok ? r.pos + 1 : 1)) * kMlaDqk, "latent rows");
    if (a.splits == 1) {
      touch_elems(a.out, (int64_t)t * a.n_heads * kMlaDv, (int64_t)(t + 1) * a.n_heads * kMlaDv, "out");
    } else {
      touch_elems(a.part_o, (int64_t)t * a.splits * a.n_heads * kMlaDv,
                  (int64_t)(t + 1) * a.splits * a.n_heads * kMlaDv, "slice outputs");
      touch_elems(a.part_ml, (int64_t)t * a.splits * a.n_heads, (int64_t)(t + 1) * a.splits * a.n_heads,
                  "slice (max, sum)");
    }
  }
  if (a.splits > 1) {
    g_kernel = "k_mla_combine";
    touch_elems(a.part_o, 0, (int64_t)a.nq * a.splits * a.n_heads * kMlaDv, "slice outputs");
    touch_elems(a.part_ml, 0, (int64_t)a.nq * a.splits * a.n_heads, "slice (max, sum)");
    touch_elems(a.out, 0, (int64_t)a.nq * a.n_heads * kMlaDv, "out");
  }
  return hipSuccess;
}

}  // namespace dsa

extern "C" {

void audit_reset(void) {
  g_regions.clear();
  g_ints.clear();
  g_viol.clear();
  g_launches.clear();
}

void audit_region(uintptr_t base, size_t bytes, const char* name) {
  g_regions.push_back({base, bytes, name ? name : "?"});
}

void audit_ints(uintptr_t base, const int32_t* vals, int64_t n) {
  g_ints[base] = std::vector<int32_t>(vals, vals + n);
}

// number of violations; the first ones, newline-separated, into buf
int audit_report(char* buf, size_t n) {
  std::string s;
  for (const auto& v : g_viol) s += v + "\n";
  if (n) {
    const size_t m = std::min(n - 1, s.size());
    std::copy(s.begin(), s.begin() + m, buf);
    buf[m] = 0;
  }
  return (int)g_viol.size();
}

// launches per modelled kernel: "name=count;..." into buf
void audit_launches(char* buf, size_t n) {
  std::string s;
  for (const auto& kv : g_launches) s += kv.first + "=" + std::to_string(kv.second) + ";";
  const size_t m = n ? std::min(n - 1, s.size()) : 0;
  if (n) {
    std::copy(s.begin(), s.begin() + m, buf);
    buf[m] = 0;
  }
}

}  // extern "C"
