// C-ABI layer: argument validation, workspace planning and kernel dispatch.
// Declarations and the contract of every entry point are in include/dsa_indexer.h.
#include "../../include/dsa_indexer.h"

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "dsa_hisa.h"
#include "dsa_internal.h"
#include "dsa_mla.h"

namespace {

thread_local std::string g_err;
// bound of the HISA token pass's wait for its query's block selection
std::atomic<uint64_t> g_hisa_spin{dsa::kHisaSpinTicks};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool debug_sync() {
  static const int on = [] {
    const char* e = getenv("DSA_DEBUG");
    return e && e[0] && e[0] != '0' ? 1 : 0;
  }();
  return on != 0;
}

int hip_status(hipError_t e, const char* what, hipStream_t stream) {
  if (e != hipSuccess) return fail(DSA_EHIP, "%s: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(DSA_EHIP, "%s (DSA_DEBUG sync): %s", what, hipGetErrorString(e));
  }
  return DSA_OK;
}

// ---- kernel timing (measurement support, see dsa_kernel_timing in the header)
struct TimingRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<hipEvent_t> g_event_pool;
std::vector<TimingRec> g_recs;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(int kind, hipStream_t stream, F&& launch) {
  if (!g_timing) return launch();
  std::lock_guard<std::mutex> lk(g_tmu);
  hipEvent_t a = pooled_event(), b = pooled_event();
  if (a) (void)hipEventRecord(a, stream);
  hipError_t e = launch();
  if (b) (void)hipEventRecord(b, stream);
  if (a && b) g_recs.push_back({kind, a, b});
  return e;
}

int score_kind(int mode) {
  switch (mode) {
    case dsa::MODE_RANGE: return DSA_KERNEL_SCORE_TOKENS;
    case dsa::MODE_POOLED: return DSA_KERNEL_SCORE_POOLED;
    case dsa::MODE_LIST: return DSA_KERNEL_SCORE_LIST;
    default: return DSA_KERNEL_SCORE_BLOCKS;
  }
}

template <class F>
hipError_t timed_pool(hipStream_t stream, F&& f) {
  return timed(DSA_KERNEL_POOL, stream, f);
}

// Most items one query can have in a pass.
int64_t pass_items_max(const dsa::SelArgs& a) {
  switch (a.mode) {
    case dsa::MODE_RANGE: return a.l_max;
    case dsa::MODE_POOLED: return a.m_max;
    case dsa::MODE_LIST: return a.list_len;
    default: return (int64_t)a.list_len * a.block;
  }
}

// One selection pass: the score-and-emit kernel, then the merge kernel; or, for
// a short pass (every query has at most kShortItems items), the scoring kernel
// storing every item's (key, id) and the one-workgroup-per-query select.
hipError_t run_score_select(dsa::SelArgs a, hipStream_t stream) {
  a.store_all = pass_items_max(a) <= dsa::kShortItems ? 1 : 0;
  hipError_t e = timed(score_kind(a.mode), stream, [&] { return dsa::launch_score_emit(a, stream); });
  if (e != hipSuccess) return e;
  if (a.store_all)
    return timed(DSA_KERNEL_MERGE, stream, [&] { return dsa::launch_select_short(a, stream); });
  return timed(DSA_KERNEL_MERGE, stream, [&] { return dsa::launch_merge(a, stream); });
}

constexpr int kBins = 4096;
// Chunks of up to 8192 items.  (One round of 16384-item chunks over 64
// queries x 128K keys, which leaves a single selection phase per call,
// measured slower than two rounds of 8192.)
constexpr int kMaxChunk = 8192;
constexpr int kMinChunk = 256;
constexpr int64_t kTargetWorkgroups = 512;   // >= 2 per compute unit on MI355X
constexpr int64_t kComputeUnits = 256;       // MI355X
constexpr size_t kMaxLds = 64 * 1024;
constexpr int64_t kMaxItems = (int64_t)kMaxChunk * dsa::kMaxChunks;   // per query and pass
constexpr int kMaxTopK = 1 << 20;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Arena {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  }
};

struct StagePlan {
  int chunk = 0, n_chunks = 0;
  size_t ghist = 0, cand = 0, cnt = 0;
};

// largest power-of-two chunk (<= the LDS limit) that still gives about
// kTargetWorkgroups workgroups over the call
int choose_chunk(int64_t n_items, int64_t nq, int f32, int head_dim) {
  int chunk = kMaxChunk;
  while (chunk > kMinChunk &&
         dsa::score_select_lds_bytes(chunk, f32, head_dim) > kMaxLds)
    chunk >>= 1;
  while (chunk > kMinChunk && nq * cdiv(n_items, chunk) < kTargetWorkgroups) chunk >>= 1;
  // the merge keeps one offset per chunk in LDS (n_items is at most
  // kMaxChunk * kMaxChunks, checked with the arguments)
  while (cdiv(n_items, chunk) > dsa::kMaxChunks && chunk < kMaxChunk) chunk <<= 1;
  return chunk;
}

void plan_zero(Arena& A, StagePlan& s, int64_t nq) {
  s.ghist = A.take((size_t)nq * kBins * 4);
}

void plan_cand(Arena& A, StagePlan& s, int64_t nq, int64_t n_items, int f32, int head_dim) {
  s.chunk = choose_chunk(n_items, nq, f32, head_dim);
  s.n_chunks = (int)cdiv(n_items, s.chunk);
  s.cand = A.take((size_t)nq * s.n_chunks * s.chunk * 8);
  s.cnt = A.take((size_t)nq * s.n_chunks * 4);
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

dsa::SelArgs stage_args(const StagePlan& s, void* ws) {
  dsa::SelArgs a{};
  a.chunk = s.chunk;
  a.n_chunks = s.n_chunks;
  a.cand = at<uint2>(ws, s.cand);
  a.cand_cnt = at<uint32_t>(ws, s.cnt);
  a.ghist = at<uint32_t>(ws, s.ghist);
  return a;
}

int check_common(const void* q, const float* w, const void* k, int32_t dtype, const int32_t* q_pos,
                 int32_t nq, int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                 int32_t top_k, const int32_t* out_idx) {
  if (nq < 0) return fail(DSA_EINVAL, "nq must be >= 0 (got %d)", nq);
  if (dtype != DSA_DTYPE_BF16 && dtype != DSA_DTYPE_F32)
    return fail(DSA_EINVAL, "dtype must be DSA_DTYPE_BF16 or DSA_DTYPE_F32 (got %d)", dtype);
  if (n_heads < 1 || n_heads > 64) return fail(DSA_EUNSUPPORTED, "n_heads must be in [1, 64] (got %d)", n_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(DSA_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (n_seq < 1) return fail(DSA_EINVAL, "n_seq must be >= 1 (got %d)", n_seq);
  if (l_max < 1 || l_max > 0x7FFFFFFF) return fail(DSA_EINVAL, "l_max must be in [1, 2^31) (got %lld)", (long long)l_max);
  if (l_max > kMaxItems)
    return fail(DSA_EUNSUPPORTED, "l_max above %lld is not supported (got %lld)",
                (long long)kMaxItems, (long long)l_max);
  if (top_k < 1 || top_k > kMaxTopK) return fail(DSA_EINVAL, "top_k must be in [1, %d] (got %d)", kMaxTopK, top_k);
  if (nq == 0) return DSA_OK;
  if (!q || !w || !k || !q_pos || !out_idx)
    return fail(DSA_EINVAL, "q, w, k, q_pos and out_idx must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(DSA_EINVAL, "q and k must be 16-byte aligned");
  if (!aligned(w, 4) || !aligned(q_pos, 4) || !aligned(out_idx, 4))
    return fail(DSA_EINVAL, "w, q_pos and out_idx must be 4-byte aligned");
  return DSA_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (have < need)
    return fail(DSA_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", have, need);
  if (need && (!ws || !aligned(ws, 256))) return fail(DSA_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  return DSA_OK;
}

// ---------------------------------------------------------------- dense ----

// Prefill-shaped calls (many queries on one sequence: a prefill, a chunk of
// one, or decode queries sharing one cache) run the query-grouped kernels.
// Rows of up to 65535 keys count their scores in 12-bit bins of 16-bit
// counters, longer rows in 11-bit bins of 32-bit counters.
bool use_prefill(int32_t dtype, int64_t nq, int n_seq, int64_t l_max) {
  return dtype == DSA_DTYPE_BF16 && n_seq == 1 && nq >= 64 && l_max < ((int64_t)1 << 30);
}
int prefill_bin_bits(int64_t l_max) { return l_max <= 65535 ? 12 : 11; }

// Keys per workgroup when the row groups (8 rows each, 32 for the routed
// scorer) are too few to fill the chip: enough chunks for about 512
// workgroups, each at least 1024 keys; 0 = no split.
int prefill_key_chunk(int64_t nq, int64_t l_max, int rows_per_group = 8) {
  const int64_t groups = (nq + rows_per_group - 1) / rows_per_group;
  if (groups >= 256) return 0;
  int64_t chunks = std::min<int64_t>((512 + groups - 1) / groups, (l_max + 1023) / 1024);
  if (chunks <= 1) return 0;
  return (int)((((l_max + chunks - 1) / chunks) + 127) / 128 * 128);
}

// (key-split rows: each row's counters, its parts' histograms and its
// threshold-bin buffer, for the select)
int row_parts(int64_t l_max) { return (int)((l_max + dsa::kRowPartKeys - 1) / dsa::kRowPartKeys); }
struct RowSelectPlan {
  size_t ctl = 0, parthist = 0, ties = 0;
};
RowSelectPlan plan_row_select(Arena& A, int64_t nq, int64_t l_max) {
  RowSelectPlan r;
  r.ctl = A.take((size_t)nq * dsa::kRowCtlWords * 4);
  r.parthist = A.take((size_t)nq * row_parts(l_max) * (kBins / 2) * 4);
  r.ties = A.take((size_t)nq * dsa::kRowTieCap * 8);
  return r;
}
void set_row_select(dsa::PrefillArgs& pa, const RowSelectPlan& r, void* ws) {
  pa.rowctl = at<uint32_t>(ws, r.ctl);
  pa.parthist = at<uint32_t>(ws, r.parthist);
  pa.row_parts = row_parts(pa.l_max);
  pa.ties = at<uint2>(ws, r.ties);
}

struct PrefillPlan {
  size_t scores = 0, rowmeta = 0, total = 0;
  RowSelectPlan rs;
};

// score rows span whole 128-key stages (the scorers store every key of a
// row's last stage); one spare row takes the stores of rows that are not scored
int64_t prefill_row_stride(int64_t l_max) { return (l_max + 127) & ~(int64_t)127; }

PrefillPlan plan_prefill(int64_t nq, int64_t l_max) {
  PrefillPlan p;
  Arena A;
  p.scores = A.take((size_t)(nq + 1) * prefill_row_stride(l_max) * 4);
  p.rowmeta = A.take((size_t)nq * 16);
  if (prefill_key_chunk(nq, l_max) > 0) p.rs = plan_row_select(A, nq, l_max);
  p.total = A.off;
  return p;
}

struct DensePlan {
  StagePlan s;
  size_t zero_bytes = 0, total = 0;
};

DensePlan plan_dense(int64_t nq, int head_dim, int64_t l_max, int f32) {
  DensePlan p;
  Arena A;
  plan_zero(A, p.s, nq);
  p.zero_bytes = A.off;
  plan_cand(A, p.s, nq, l_max, f32, head_dim);
  p.total = A.off;
  return p;
}

// workspace of the dense call (prefill-shaped or decode-shaped)
size_t dense_workspace(int32_t nq, int32_t head_dim, int32_t n_seq, int64_t l_max, int32_t dtype) {
  if (use_prefill(dtype, nq, n_seq, l_max)) return plan_prefill(nq, l_max).total;
  return plan_dense(nq, head_dim, l_max, dtype == DSA_DTYPE_F32).total;
}

// ----------------------------------------------------------------- MISA ----

struct MisaPlan {
  StagePlan s0, s1;
  size_t zero_bytes = 0, part = 0, cand_list = 0, partial = 0, pooled = 0;
  size_t total = 0;
  int splits = 1, bps = 1;
  int64_t m_max = 0;
};

MisaPlan plan_misa(int64_t nq, int n_heads, int head_dim, int n_seq, int64_t l_max, int block, int h,
                   int k_prime, bool pooled_given) {
  MisaPlan p;
  Arena A;
  p.m_max = cdiv(l_max, block);
  plan_zero(A, p.s0, nq);
  if (k_prime > 0) plan_zero(A, p.s1, nq);
  p.zero_bytes = A.off;
  // router: about kTargetWorkgroups workgroups, at least 64 blocks each
  int64_t bps = 64;
  while (bps < p.m_max && nq * cdiv(p.m_max, bps) > kTargetWorkgroups) bps *= 2;
  p.bps = (int)bps;
  p.splits = (int)cdiv(p.m_max, bps);
  p.part = A.take((size_t)nq * p.splits * n_heads * 4);
  (void)h;
  plan_cand(A, p.s0, nq, l_max, 0, head_dim);
  if (k_prime > 0) {
    p.cand_list = A.take((size_t)nq * k_prime * 4);
    plan_cand(A, p.s1, nq, k_prime, 0, head_dim);
  }
  p.partial = A.take((size_t)nq * head_dim * 2);
  if (!pooled_given) p.pooled = A.take((size_t)n_seq * p.m_max * head_dim * 2);
  p.total = A.off;
  return p;
}

// ----------------------------------------------------------------- HISA ----

struct HisaPlan {
  StagePlan s0, s1;
  size_t zero_bytes = 0, blocks = 0, partial = 0, pooled = 0, total = 0;
  int64_t m_max = 0;
};

HisaPlan plan_hisa(int64_t nq, int head_dim, int n_seq, int64_t l_max, int block, int m,
                   bool pooled_given) {
  HisaPlan p;
  Arena A;
  p.m_max = cdiv(l_max, block);
  plan_zero(A, p.s0, nq);
  plan_zero(A, p.s1, nq);
  p.zero_bytes = A.off;
  plan_cand(A, p.s0, nq, p.m_max, 0, head_dim);
  p.blocks = A.take((size_t)nq * m * 4);
  plan_cand(A, p.s1, nq, (int64_t)m * block, 0, head_dim);
  p.partial = A.take((size_t)nq * head_dim * 2);
  if (!pooled_given) p.pooled = A.take((size_t)n_seq * p.m_max * head_dim * 2);
  p.total = A.off;
  return p;
}

// HISA kernels.  When one grid of G workgroups per query (about
// kTargetWorkgroups in all) fits the chip at once, every workgroup takes part
// in both passes: ch1 pooled blocks, then ch2 token items.  Otherwise (many
// queries: prefill rows) the grid is split into block-pass items, all
// dispatched first, and token-pass items, so that no workgroup waits for a
// selection while occupying a slot that block-pass work still needs.  Chunks
// are at most kHisaMaxChunk and multiples of the 32-item tile.  The sync
// words and the kept-block flags come first: the prepare kernel clears them.
struct HisaFusedPlan {
  bool ok = false;
  int split = 0, groups = 0, groups1 = 0, groups2 = 0, ch1 = 0, ch2 = 0, sblk_n = 0;
  int64_t m_max = 0;
  size_t zero_bytes = 0, sync = 0, bflag = 0, cand1 = 0, cnt1 = 0, keys2 = 0, blocks = 0;
  size_t partial = 0, pooled = 0, total = 0;
};

// workgroups per query for `items` items: about kTargetWorkgroups over the
// call, more when a chunk would exceed kHisaMaxChunk
int64_t hisa_groups(int64_t nq, int64_t items) {
  int64_t g = cdiv(kTargetWorkgroups, nq);
  if (g > dsa::kHisaMaxGroups) g = dsa::kHisaMaxGroups;
  while (g < dsa::kHisaMaxGroups && cdiv(items, g) > dsa::kHisaMaxChunk) g *= 2;
  return g > dsa::kHisaMaxGroups ? dsa::kHisaMaxGroups : g;
}

int hisa_chunk(int64_t items, int64_t g) { return (int)(cdiv(cdiv(items, g), 32) * 32); }

HisaFusedPlan plan_hisa_fused(int64_t nq, int head_dim, int n_seq, int64_t l_max, int block, int m,
                              bool pooled_given) {
  HisaFusedPlan p;
  p.m_max = cdiv(l_max, block);
  const int64_t items = (int64_t)m * block;
  const int64_t g = std::max(hisa_groups(nq, p.m_max), hisa_groups(nq, items));
  p.split = nq * g > kTargetWorkgroups ? 1 : 0;
  int64_t g1 = g, g2 = g;
  if (p.split) {
    g1 = hisa_groups(nq, p.m_max);
    g2 = hisa_groups(nq, items);
  }
  p.ok = nq <= 65535 && m <= dsa::kHisaMaxBlocks && items <= dsa::kHisaRegKeys &&
         cdiv(p.m_max, g1) <= dsa::kHisaMaxChunk && cdiv(items, g2) <= dsa::kHisaMaxChunk;
  p.groups = (int)g;
  p.groups1 = (int)g1;
  p.groups2 = (int)g2;
  p.ch1 = hisa_chunk(p.m_max, g1);
  p.ch2 = hisa_chunk(items, g2);
  p.sblk_n = p.ch2 / block + 2;
  Arena A;
  p.sync = A.take((size_t)nq * dsa::kHisaSyncWords * 4);
  p.bflag = A.take((size_t)nq * m * 4);
  p.zero_bytes = A.off;
  p.cand1 = A.take((size_t)nq * g1 * p.ch1 * 8);
  p.cnt1 = A.take((size_t)nq * g1 * 4);
  p.keys2 = A.take((size_t)nq * g2 * p.ch2 * 4);
  p.blocks = A.take((size_t)nq * m * 4);
  p.partial = A.take((size_t)nq * head_dim * 2);
  if (!pooled_given) p.pooled = A.take((size_t)n_seq * p.m_max * head_dim * 2);
  p.total = A.off;
  return p;
}

int run_prepare(void* ws, size_t zero_bytes, const void* k, const int32_t* q_seq,
                const int32_t* q_pos, int nq, int n_seq, int head_dim, int block, int64_t l_max,
                uint16_t* partial, hipStream_t stream, int32_t* status = nullptr) {
  dsa::PrepArgs pa{};
  pa.zero = at<uint32_t>(ws, 0);
  pa.zero_words = zero_bytes / 4;
  pa.keys = reinterpret_cast<const uint16_t*>(k);
  pa.q_seq = q_seq;
  pa.q_pos = q_pos;
  pa.nq = nq;
  pa.n_seq = n_seq;
  pa.head_dim = head_dim;
  pa.block = block;
  pa.l_max = l_max;
  pa.partial = partial;
  pa.status = status;
  return hip_status(timed(DSA_KERNEL_PREPARE, stream, [&] { return dsa::launch_prepare(pa, stream); }),
                    "prepare kernel", stream);
}

// The HISA kernels' common set-up: pooled keys (the caller's, or pooled into
// the workspace) and the prepare kernel (sync words, kept-block flags,
// partial last blocks).
int hisa_setup(const HisaFusedPlan& f, const void* k, const void* k_pooled, const int32_t* q_seq,
               const int32_t* q_pos, int nq, int n_seq, int head_dim, int64_t l_max, int block,
               void* workspace, hipStream_t stream, const uint16_t** pooled_out,
               uint16_t** partial_out) {
  int st;
  const uint16_t* pooled = reinterpret_cast<const uint16_t*>(k_pooled);
  if (!pooled) {
    uint16_t* dst = at<uint16_t>(workspace, f.pooled);
    st = hip_status(timed_pool(stream, [&] { return dsa::launch_mean_pool(reinterpret_cast<const uint16_t*>(k), n_seq, l_max,
                                          head_dim, block, dst, stream); }),
                    "mean-pool kernel", stream);
    if (st) return st;
    pooled = dst;
  }
  uint16_t* partial = at<uint16_t>(workspace, f.partial);
  if ((st = run_prepare(workspace, f.zero_bytes, k, q_seq, q_pos, nq, n_seq, head_dim, block,
                        l_max, partial, stream)))
    return st;
  *pooled_out = pooled;
  *partial_out = partial;
  return DSA_OK;
}

// MISA routing of the HISA kernels: the router's per-slice head sums, from
// which k_hisa keeps the h_use most important heads, and where it reports them.
struct HisaRoute {
  const float* part = nullptr;   // [nq, splits, n_heads], or null: all n_heads
  int splits = 0, h_use = 0;
  int32_t* out_heads = nullptr;
  float* out_importance = nullptr;
};

// k_hisa and k_hisa_topk over the plan, over all n_heads or the routed ones.
int run_hisa_kernels(const HisaFusedPlan& f, const void* q, const float* w, const void* k,
                     const uint16_t* pooled, const uint16_t* partial, const int32_t* q_seq,
                     const int32_t* q_pos, const HisaRoute& route, int nq, int n_heads,
                     int head_dim, int n_seq, int64_t l_max, int block, int m_blocks, int top_k,
                     int32_t* out_idx, float* out_score, int32_t* out_blocks,
                     float* out_block_score, int32_t* out_status, void* workspace,
                     hipStream_t stream) {
  dsa::HisaArgs h{};
  h.q = reinterpret_cast<const uint16_t*>(q);
  h.w = w;
  h.keys = reinterpret_cast<const uint16_t*>(k);
  h.pooled = pooled;
  h.partial = partial;
  h.q_seq = q_seq;
  h.q_pos = q_pos;
  h.heads = nullptr;
  h.heads_stride = 0;
  h.h_use = route.part ? route.h_use : n_heads;
  h.route_part = route.part;
  h.route_splits = route.splits;
  h.out_heads = route.out_heads;
  h.out_importance = route.out_importance;
  h.nq = nq;
  h.n_heads = n_heads;
  h.head_dim = head_dim;
  h.n_seq = n_seq;
  h.block = block;
  h.m_blocks = m_blocks;
  h.top_k = top_k;
  h.l_max = l_max;
  h.m_max = f.m_max;
  h.groups = f.groups;
  h.split = f.split;
  h.groups1 = f.groups1;
  h.groups2 = f.groups2;
  h.ch1 = f.ch1;
  h.ch2 = f.ch2;
  h.sblk_n = f.sblk_n;
  h.sync = at<uint32_t>(workspace, f.sync);
  h.bflag = at<int32_t>(workspace, f.bflag);
  h.cand1 = at<uint2>(workspace, f.cand1);
  h.cnt1 = at<uint32_t>(workspace, f.cnt1);
  h.keys2 = at<uint32_t>(workspace, f.keys2);
  h.blocks = out_blocks ? out_blocks : at<int32_t>(workspace, f.blocks);
  h.out_idx = out_idx;
  h.out_score = out_score;
  h.out_block_score = out_block_score;
  h.out_status = out_status;
  h.spin_ticks = g_hisa_spin.load(std::memory_order_relaxed);
  int st = hip_status(timed(DSA_KERNEL_HISA, stream, [&] { return dsa::launch_hisa(h, stream); }),
                      "HISA kernel", stream);
  if (st || !debug_sync()) return st;
  // DSA_DEBUG: the call has completed; report queries whose token pass gave up
  // its wait (their rows hold padding only)
  std::vector<uint32_t> sy((size_t)nq * dsa::kHisaSyncWords);
  hipError_t e = hipMemcpyAsync(sy.data(), h.sync, sy.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(DSA_EHIP, "HISA status read (DSA_DEBUG): %s", hipGetErrorString(e));
  int n_to = 0, first = -1;
  for (int t = 0; t < nq; ++t)
    if (sy[(size_t)t * dsa::kHisaSyncWords + dsa::kHisaSyncTimeout]) {
      if (first < 0) first = t;
      ++n_to;
    }
  if (n_to)
    return fail(DSA_ETIMEOUT, "HISA: %d queries (first: %d) timed out waiting for their block "
                "selection; their rows hold padding only", n_to, first);
  return DSA_OK;
}

// MISA∘HISA: the HISA plan, then the router's per-slice sums.
struct MisaHisaPlan {
  HisaFusedPlan h;
  size_t part = 0, total = 0;
  int splits = 1, bps = 1;
};

MisaHisaPlan plan_misa_hisa(int64_t nq, int n_heads, int head_dim, int n_seq, int64_t l_max,
                            int block, int m, bool pooled_given) {
  MisaHisaPlan p;
  p.h = plan_hisa_fused(nq, head_dim, n_seq, l_max, block, m, pooled_given);
  int64_t bps = 64;
  while (bps < p.h.m_max && nq * cdiv(p.h.m_max, bps) > kTargetWorkgroups) bps *= 2;
  p.bps = (int)bps;
  p.splits = (int)cdiv(p.h.m_max, bps);
  Arena A;
  A.off = p.h.total;
  p.part = A.take((size_t)nq * p.splits * n_heads * 4);
  p.total = A.off;
  return p;
}

void fill_common(dsa::SelArgs& a, const void* q, const float* w, const void* k,
                 const int32_t* q_seq, const int32_t* q_pos, int nq, int n_heads, int head_dim,
                 int n_seq, int64_t l_max) {
  a.q = q;
  a.w = w;
  a.keys = k;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.nq = nq;
  a.n_heads = n_heads;
  a.h_use = n_heads;
  a.head_dim = head_dim;
  a.n_seq = n_seq;
  a.l_max = l_max;
}

}  // namespace

// MISA on the prefill shape (one sequence, many bf16 rows, h <= 8, k' = 0): the
// router, the head selection, the packed routed scoring and the row select.
// (the routed scorer's per-row histograms have 16-bit counters: rows of up to
// 65535 keys, unless the keys are split and the select counts the rows)
bool use_misa_prefill(int32_t dtype, int64_t nq, int n_seq, int64_t l_max, int h, int k_prime) {
  return use_prefill(dtype, nq, n_seq, l_max) && k_prime == 0 && h <= dsa::kRoutedMaxHeads &&
         (l_max <= 65535 || prefill_key_chunk(nq, l_max, 32) > 0);
}

struct MisaPrefillPlan {
  size_t part = 0, heads = 0, prefix = 0, pooled = 0, scores = 0, rowmeta = 0, total = 0;
  RowSelectPlan rs;
  int splits = 1, bps = 1;
  int64_t m_max = 0, row_stride = 0;
};

MisaPrefillPlan plan_misa_prefill(int64_t nq, int n_heads, int head_dim, int n_seq, int64_t l_max,
                                  int block, bool pooled_given) {
  MisaPrefillPlan p;
  Arena A;
  p.m_max = cdiv(l_max, block);
  p.bps = (int)p.m_max;                         // one slice: a wave per query
  p.splits = 1;
  p.part = A.take((size_t)nq * n_heads * 4);
  p.heads = A.take((size_t)nq * dsa::kRoutedMaxHeads * 4);
  p.prefix = A.take((size_t)l_max * head_dim * 2);
  if (!pooled_given) p.pooled = A.take((size_t)n_seq * p.m_max * head_dim * 2);
  p.row_stride = prefill_row_stride(l_max);
  p.scores = A.take((size_t)(nq + 1) * p.row_stride * 4);
  p.rowmeta = A.take((size_t)nq * 16);
  if (prefill_key_chunk(nq, l_max, 32) > 0) p.rs = plan_row_select(A, nq, l_max);
  p.total = A.off;
  return p;
}

int misa_prefill(const void* q, const float* w, const void* k, const void* k_pooled,
                 const int32_t* q_seq, const int32_t* q_pos, int32_t nq, int32_t n_heads,
                 int32_t head_dim, int32_t n_seq, int64_t l_max, int32_t block, int32_t h,
                 int32_t top_k, int32_t* out_idx, float* out_score, int32_t* out_heads,
                 float* out_importance, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  MisaPrefillPlan p = plan_misa_prefill(nq, n_heads, head_dim, n_seq, l_max, block,
                                        k_pooled != nullptr);
  int st = check_ws(workspace, workspace_bytes, p.total);
  if (st) return st;
  const uint16_t* pooled = reinterpret_cast<const uint16_t*>(k_pooled);
  if (!pooled) {
    uint16_t* dst = at<uint16_t>(workspace, p.pooled);
    st = hip_status(timed_pool(stream, [&] { return dsa::launch_mean_pool(reinterpret_cast<const uint16_t*>(k), n_seq, l_max,
                                          head_dim, block, dst, stream); }),
                    "mean-pool kernel", stream);
    if (st) return st;
    pooled = dst;
  }
  // pooled keys of prefixes that end inside a block, by position
  uint16_t* prefix = at<uint16_t>(workspace, p.prefix);
  if ((st = hip_status(timed(DSA_KERNEL_PREPARE, stream, [&] {
                         return dsa::launch_pool_prefix(reinterpret_cast<const uint16_t*>(k), l_max,
                                                        head_dim, block, prefix, stream); }),
                       "prefix-pool kernel", stream)))
    return st;
  dsa::RouteArgs ra{};
  ra.q = reinterpret_cast<const uint16_t*>(q);
  ra.pooled = pooled;
  ra.partial = prefix;
  ra.partial_by_pos = 1;
  ra.q_seq = q_seq;
  ra.q_pos = q_pos;
  ra.nq = nq;
  ra.n_heads = n_heads;
  ra.head_dim = head_dim;
  ra.n_seq = n_seq;
  ra.block = block;
  ra.splits = p.splits;
  ra.blocks_per_split = p.bps;
  ra.l_max = l_max;
  ra.m_max = p.m_max;
  ra.part = at<float>(workspace, p.part);
  if ((st = hip_status(timed(DSA_KERNEL_ROUTE, stream, [&] { return dsa::launch_route(ra, stream); }),
                       "router kernel", stream))) return st;
  dsa::RouteHeadsArgs rh{};
  rh.part = ra.part;
  rh.w = w;
  rh.q_seq = q_seq;
  rh.q_pos = q_pos;
  rh.nq = nq;
  rh.n_heads = n_heads;
  rh.splits = p.splits;
  rh.h_use = h;
  rh.heads_stride = dsa::kRoutedMaxHeads;
  rh.n_seq = n_seq;
  rh.l_max = l_max;
  rh.heads = at<int32_t>(workspace, p.heads);
  rh.out_heads = out_heads;
  rh.out_importance = out_importance;
  if ((st = hip_status(timed(DSA_KERNEL_ROUTE_HEADS, stream,
                             [&] { return dsa::launch_route_heads(rh, stream); }),
                       "head selection kernel", stream))) return st;
  dsa::PrefillArgs pa{};
  pa.q = reinterpret_cast<const uint16_t*>(q);
  pa.w = w;
  pa.keys = reinterpret_cast<const uint16_t*>(k);
  pa.q_seq = q_seq;
  pa.q_pos = q_pos;
  pa.nq = nq;
  pa.n_heads = n_heads;
  pa.head_dim = head_dim;
  pa.top_k = top_k;
  pa.l_max = l_max;
  pa.row_stride = p.row_stride;
  pa.scores = at<float>(workspace, p.scores);
  pa.spare_row = pa.scores + (size_t)nq * p.row_stride;
  pa.rowmeta = at<int32_t>(workspace, p.rowmeta);
  pa.key_chunk = prefill_key_chunk(nq, l_max, 32);
  pa.bin_bits = pa.key_chunk ? 12 : 10;
  if (pa.key_chunk) set_row_select(pa, p.rs, workspace);
  pa.heads = rh.heads;
  pa.heads_stride = rh.heads_stride;
  pa.h_use = h;
  pa.out_idx = out_idx;
  pa.out_score = out_score;
  if ((st = hip_status(timed(DSA_KERNEL_PREFILL_ROUTED, stream,
                             [&] { return dsa::launch_prefill_routed_score(pa, stream); }),
                       "routed prefill scoring kernel", stream))) return st;
  return hip_status(timed(DSA_KERNEL_ROWSELECT, stream,
                          [&] { return dsa::launch_prefill_select(pa, stream); }),
                    "prefill select kernel", stream);
}

extern "C" {

const char* dsa_last_error(void) { return g_err.c_str(); }

int dsa_abi_version(void) { return 3; }

int dsa_hisa_wait_limit(int64_t ticks) {
  g_hisa_spin.store(ticks < 0 ? dsa::kHisaSpinTicks : (uint64_t)ticks, std::memory_order_relaxed);
  return DSA_OK;
}

int dsa_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  if (!g_timing) {
    for (auto& r : g_recs) {
      g_event_pool.push_back(r.a);
      g_event_pool.push_back(r.b);
    }
    g_recs.clear();
  }
  return DSA_OK;
}

int dsa_kernel_timing_read(int32_t kind, int64_t* launches, double* total_ms, double* min_ms,
                           double* max_ms) {
  if (kind < 0 || kind >= DSA_KERNEL_KINDS) return fail(DSA_EINVAL, "unknown kernel kind %d", kind);
  std::lock_guard<std::mutex> lk(g_tmu);
  int64_t n = 0;
  double tot = 0, lo = 0, hi = 0;
  std::vector<TimingRec> keep;
  for (auto& r : g_recs) {
    if (r.kind != kind) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
    if (e != hipSuccess) return fail(DSA_EHIP, "event timing: %s", hipGetErrorString(e));
    lo = n ? (ms < lo ? ms : lo) : ms;
    hi = n ? (ms > hi ? ms : hi) : ms;
    tot += ms;
    ++n;
  }
  g_recs.swap(keep);
  if (launches) *launches = n;
  if (total_ms) *total_ms = tot;
  if (min_ms) *min_ms = lo;
  if (max_ms) *max_ms = hi;
  return DSA_OK;
}

size_t indexer_score_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                         int32_t n_seq, int64_t l_max, int32_t top_k,
                                         int32_t dtype) {
  (void)n_heads; (void)top_k;
  if (nq <= 0 || l_max <= 0) return 0;
  return dense_workspace(nq, head_dim, n_seq, l_max, dtype);
}

}  // extern "C"

namespace {

// The dense call after argument validation: the prefill-shaped kernels, or
// the decode-shaped pass (clear, score-and-emit, merge), over `workspace`.
int dense_call(const void* q, const float* w, const void* k, int32_t dtype, const int32_t* q_seq,
               const int32_t* q_pos, int32_t nq, int32_t n_heads, int32_t head_dim,
               int32_t n_seq, int64_t l_max, int32_t top_k, int32_t* out_idx, float* out_score,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st;
  const int f32 = dtype == DSA_DTYPE_F32;
  if (use_prefill(dtype, nq, n_seq, l_max)) {
    PrefillPlan pp = plan_prefill(nq, l_max);
    if ((st = check_ws(workspace, workspace_bytes, pp.total))) return st;
    dsa::PrefillArgs pa{};
    pa.q = reinterpret_cast<const uint16_t*>(q);
    pa.w = w;
    pa.keys = reinterpret_cast<const uint16_t*>(k);
    pa.q_seq = q_seq;
    pa.q_pos = q_pos;
    pa.nq = nq;
    pa.n_heads = n_heads;
    pa.head_dim = head_dim;
    pa.top_k = top_k;
    pa.l_max = l_max;
    pa.row_stride = prefill_row_stride(l_max);
    pa.scores = at<float>(workspace, pp.scores);
    pa.spare_row = pa.scores + (size_t)nq * pa.row_stride;
    pa.rowmeta = at<int32_t>(workspace, pp.rowmeta);
    pa.key_chunk = prefill_key_chunk(nq, l_max);
    pa.bin_bits = pa.key_chunk ? 12 : prefill_bin_bits(l_max);   // first-level bins of the rows
    if (pa.key_chunk) set_row_select(pa, pp.rs, workspace);
    pa.out_idx = out_idx;
    pa.out_score = out_score;
    st = hip_status(timed(DSA_KERNEL_PREFILL, stream,
                          [&] { return dsa::launch_prefill_score(pa, stream); }),
                    "prefill score kernel", stream);
    if (st) return st;
    return hip_status(timed(DSA_KERNEL_ROWSELECT, stream,
                            [&] { return dsa::launch_prefill_select(pa, stream); }),
                      "prefill select kernel", stream);
  }
  DensePlan p = plan_dense(nq, head_dim, l_max, f32);
  if ((st = check_ws(workspace, workspace_bytes, p.total))) return st;
  if ((st = run_prepare(workspace, p.zero_bytes, k, q_seq, q_pos, nq, n_seq, head_dim, 1, l_max,
                        nullptr, stream)))
    return st;
  dsa::SelArgs a = stage_args(p.s, workspace);
  fill_common(a, q, w, k, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max);
  a.f32 = f32;
  a.mode = dsa::MODE_RANGE;
  a.top_k = top_k;
  a.out_idx = out_idx;
  a.out_score = out_score;
  return hip_status(run_score_select(a, stream), "score/select kernel", stream);
}

// ---- the entry point that allocates nothing: its workspace is this
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never uses the array's name as an address (on the host it is only
// a stand-in symbol): the device address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DSA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

int indexer_score_topk(const void* q, const float* w, const void* k, int32_t dtype,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t nq, int32_t n_heads,
                       int32_t head_dim, int32_t n_seq, int64_t l_max, int32_t top_k,
                       int32_t* out_idx, float* out_score, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  int st = check_common(q, w, k, dtype, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k, out_idx);
  if (st || nq == 0) return st;
  return dense_call(q, w, k, dtype, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k,
                    out_idx, out_score, workspace, workspace_bytes, stream);
}

int indexer_score_topk_noalloc(const void* q, const float* w, const void* k, int32_t dtype,
                               const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                               int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                               int32_t top_k, int32_t* out_idx, float* out_score,
                               hipStream_t stream) {
  int st = check_common(q, w, k, dtype, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k, out_idx);
  if (st || nq == 0) return st;
  const size_t need = dense_workspace(nq, head_dim, n_seq, l_max, dtype);
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_EUNSUPPORTED, "this call needs %zu bytes of scratch; the no-allocation entry "
                "point holds %zu (use indexer_score_topk with a workspace)", need,
                (size_t)DSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return dense_call(q, w, k, dtype, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k,
                    out_idx, out_score, ws, (size_t)DSA_NOALLOC_SCRATCH_BYTES, stream);
}

int indexer_mean_pool_keys(const void* k, int32_t dtype, int32_t n_seq, int64_t l_max,
                           int32_t head_dim, int32_t block, void* k_pooled, hipStream_t stream) {
  if (dtype != DSA_DTYPE_BF16) return fail(DSA_EUNSUPPORTED, "pooling supports bf16 keys only");
  if (head_dim != 64 && head_dim != 128)
    return fail(DSA_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (n_seq < 0 || l_max < 0 || l_max > 0x7FFFFFFF) return fail(DSA_EINVAL, "bad n_seq / l_max");
  if (block < 1) return fail(DSA_EINVAL, "block must be >= 1 (got %d)", block);
  if (n_seq == 0 || l_max == 0) return DSA_OK;
  if (!k || !k_pooled) return fail(DSA_EINVAL, "k and k_pooled must not be NULL");
  if (!aligned(k, 16) || !aligned(k_pooled, 16)) return fail(DSA_EINVAL, "k and k_pooled must be 16-byte aligned");
  return hip_status(timed_pool(stream, [&] { return dsa::launch_mean_pool(reinterpret_cast<const uint16_t*>(k), n_seq, l_max,
                                          head_dim, block, reinterpret_cast<uint16_t*>(k_pooled),
                                          stream); }),
                    "mean-pool kernel", stream);
}

size_t misa_route_score_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                            int32_t n_seq, int64_t l_max, int32_t block,
                                            int32_t n_active_heads, int32_t k_prime,
                                            int32_t top_k, int32_t pooled_given) {
  (void)top_k;
  if (nq <= 0 || l_max <= 0 || block <= 0 || n_active_heads <= 0) return 0;
  if (use_misa_prefill(DSA_DTYPE_BF16, nq, n_seq, l_max, n_active_heads, k_prime))
    return plan_misa_prefill(nq, n_heads, head_dim, n_seq, l_max, block, pooled_given != 0).total;
  return plan_misa(nq, n_heads, head_dim, n_seq, l_max, block, n_active_heads, k_prime,
                   pooled_given != 0).total;
}

int misa_route_score_topk(const void* q, const float* w, const void* k, const void* k_pooled,
                          int32_t dtype, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                          int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                          int32_t block, int32_t n_active_heads, int32_t k_prime, int32_t top_k,
                          int32_t* out_idx, float* out_score, int32_t* out_heads,
                          float* out_importance, int32_t* out_cand, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  int st = check_common(q, w, k, dtype, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k, out_idx);
  if (st) return st;
  if (dtype != DSA_DTYPE_BF16) return fail(DSA_EUNSUPPORTED, "MISA supports bf16 inputs only");
  if (block < 1) return fail(DSA_EINVAL, "block must be >= 1 (got %d)", block);
  if (n_active_heads < 1 || n_active_heads > n_heads)
    return fail(DSA_EINVAL, "n_active_heads must be in [1, n_heads] (got %d)", n_active_heads);
  if (k_prime != 0 && (k_prime < top_k || k_prime > kMaxTopK))
    return fail(DSA_EINVAL, "k_prime must be 0 or in [top_k, %d] (got %d)", kMaxTopK, k_prime);
  if (nq == 0) return DSA_OK;
  if (k_pooled && !aligned(k_pooled, 16)) return fail(DSA_EINVAL, "k_pooled must be 16-byte aligned");
  if (use_misa_prefill(dtype, nq, n_seq, l_max, n_active_heads, k_prime))
    return misa_prefill(q, w, k, k_pooled, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max, block,
                        n_active_heads, top_k, out_idx, out_score, out_heads, out_importance,
                        workspace, workspace_bytes, stream);
  MisaPlan p = plan_misa(nq, n_heads, head_dim, n_seq, l_max, block, n_active_heads, k_prime,
                         k_pooled != nullptr);
  if ((st = check_ws(workspace, workspace_bytes, p.total))) return st;
  const uint16_t* pooled = reinterpret_cast<const uint16_t*>(k_pooled);
  if (!pooled) {
    uint16_t* dst = at<uint16_t>(workspace, p.pooled);
    st = hip_status(timed_pool(stream, [&] { return dsa::launch_mean_pool(reinterpret_cast<const uint16_t*>(k), n_seq, l_max,
                                          head_dim, block, dst, stream); }),
                    "mean-pool kernel", stream);
    if (st) return st;
    pooled = dst;
  }
  uint16_t* partial = at<uint16_t>(workspace, p.partial);
  if ((st = run_prepare(workspace, p.zero_bytes, k, q_seq, q_pos, nq, n_seq, head_dim, block,
                        l_max, partial, stream)))
    return st;
  // router
  dsa::RouteArgs ra{};
  ra.q = reinterpret_cast<const uint16_t*>(q);
  ra.pooled = pooled;
  ra.partial = partial;
  ra.q_seq = q_seq;
  ra.q_pos = q_pos;
  ra.nq = nq;
  ra.n_heads = n_heads;
  ra.head_dim = head_dim;
  ra.n_seq = n_seq;
  ra.block = block;
  ra.splits = p.splits;
  ra.blocks_per_split = p.bps;
  ra.l_max = l_max;
  ra.m_max = p.m_max;
  ra.part = at<float>(workspace, p.part);
  if ((st = hip_status(timed(DSA_KERNEL_ROUTE, stream, [&] { return dsa::launch_route(ra, stream); }),
                       "router kernel", stream))) return st;
  // routed token pass
  dsa::SelArgs a = stage_args(p.s0, workspace);
  fill_common(a, q, w, k, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max);
  a.h_use = n_active_heads;
  a.route_part = ra.part;
  a.route_splits = ra.splits;
  a.out_heads = out_heads;
  a.out_importance = out_importance;
  a.mode = dsa::MODE_RANGE;
  if (k_prime == 0) {
    a.top_k = top_k;
    a.out_idx = out_idx;
    a.out_score = out_score;
    return hip_status(run_score_select(a, stream), "routed score/select kernel", stream);
  }
  int32_t* cand = out_cand ? out_cand : at<int32_t>(workspace, p.cand_list);
  a.top_k = k_prime;
  a.out_idx = cand;
  a.out_score = nullptr;
  if ((st = hip_status(run_score_select(a, stream), "routed score/select kernel", stream)))
    return st;
  // all-head rescoring of the k' candidates
  dsa::SelArgs b = stage_args(p.s1, workspace);
  fill_common(b, q, w, k, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max);
  b.mode = dsa::MODE_LIST;
  b.list = cand;
  b.list_len = k_prime;
  b.top_k = top_k;
  b.out_idx = out_idx;
  b.out_score = out_score;
  return hip_status(run_score_select(b, stream), "rescore/select kernel", stream);
}

size_t hisa_block_filter_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                             int32_t n_seq, int64_t l_max, int32_t block,
                                             int32_t m_blocks, int32_t top_k,
                                             int32_t pooled_given) {
  (void)n_heads; (void)top_k;
  if (nq <= 0 || l_max <= 0 || block <= 0 || m_blocks <= 0) return 0;
  HisaFusedPlan f = plan_hisa_fused(nq, head_dim, n_seq, l_max, block, m_blocks, pooled_given != 0);
  if (f.ok) return f.total;
  return plan_hisa(nq, head_dim, n_seq, l_max, block, m_blocks, pooled_given != 0).total;
}

int hisa_block_filter_topk(const void* q, const float* w, const void* k, const void* k_pooled,
                           int32_t dtype, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                           int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                           int32_t block, int32_t m_blocks, int32_t top_k, int32_t* out_idx,
                           float* out_score, int32_t* out_blocks, float* out_block_score,
                           int32_t* out_status, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  int st = check_common(q, w, k, dtype, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k, out_idx);
  if (st) return st;
  if (dtype != DSA_DTYPE_BF16) return fail(DSA_EUNSUPPORTED, "HISA supports bf16 inputs only");
  if (block < 1) return fail(DSA_EINVAL, "block must be >= 1 (got %d)", block);
  if (m_blocks < 1 || m_blocks > kMaxTopK) return fail(DSA_EINVAL, "m_blocks must be in [1, %d] (got %d)", kMaxTopK, m_blocks);
  if ((int64_t)m_blocks * block > 0x7FFFFFFF) return fail(DSA_EINVAL, "m_blocks * block too large");
  if (nq == 0) return DSA_OK;
  if (k_pooled && !aligned(k_pooled, 16)) return fail(DSA_EINVAL, "k_pooled must be 16-byte aligned");
  if (!aligned(out_status, 4)) return fail(DSA_EINVAL, "out_status must be 4-byte aligned");
  HisaFusedPlan f = plan_hisa_fused(nq, head_dim, n_seq, l_max, block, m_blocks, k_pooled != nullptr);
  if (f.ok) {
    if ((st = check_ws(workspace, workspace_bytes, f.total))) return st;
    const uint16_t* pooled = nullptr;
    uint16_t* partial = nullptr;
    if ((st = hisa_setup(f, k, k_pooled, q_seq, q_pos, nq, n_seq, head_dim, l_max, block, workspace,
                         stream, &pooled, &partial)))
      return st;
    return run_hisa_kernels(f, q, w, k, pooled, partial, q_seq, q_pos, HisaRoute{}, nq,
                            n_heads, head_dim, n_seq, l_max, block, m_blocks, top_k, out_idx,
                            out_score, out_blocks, out_block_score, out_status, workspace,
                            stream);
  }
  HisaPlan p = plan_hisa(nq, head_dim, n_seq, l_max, block, m_blocks, k_pooled != nullptr);
  if ((st = check_ws(workspace, workspace_bytes, p.total))) return st;
  const uint16_t* pooled = reinterpret_cast<const uint16_t*>(k_pooled);
  if (!pooled) {
    uint16_t* dst = at<uint16_t>(workspace, p.pooled);
    st = hip_status(timed_pool(stream, [&] { return dsa::launch_mean_pool(reinterpret_cast<const uint16_t*>(k), n_seq, l_max,
                                          head_dim, block, dst, stream); }),
                    "mean-pool kernel", stream);
    if (st) return st;
    pooled = dst;
  }
  uint16_t* partial = at<uint16_t>(workspace, p.partial);
  // (the passes of this path never wait: every query's status is 0)
  if ((st = run_prepare(workspace, p.zero_bytes, k, q_seq, q_pos, nq, n_seq, head_dim, block,
                        l_max, partial, stream, out_status)))
    return st;
  // stage 1: block scores over the pooled keys, top-m blocks
  int32_t* blocks = out_blocks ? out_blocks : at<int32_t>(workspace, p.blocks);
  dsa::SelArgs a = stage_args(p.s0, workspace);
  fill_common(a, q, w, k, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max);
  a.mode = dsa::MODE_POOLED;
  a.pooled = pooled;
  a.partial = partial;
  a.m_max = p.m_max;
  a.block = block;
  a.top_k = m_blocks;
  a.out_idx = blocks;
  a.out_score = out_block_score;
  if ((st = hip_status(run_score_select(a, stream), "block score/select kernel", stream)))
    return st;
  // stage 2: token refinement inside the surviving blocks
  dsa::SelArgs b = stage_args(p.s1, workspace);
  fill_common(b, q, w, k, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max);
  b.mode = dsa::MODE_BLOCKS;
  b.list = blocks;
  b.list_len = m_blocks;
  b.block = block;
  b.top_k = top_k;
  b.out_idx = out_idx;
  b.out_score = out_score;
  return hip_status(run_score_select(b, stream), "refine score/select kernel", stream);
}

size_t misa_hisa_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                     int32_t n_seq, int64_t l_max, int32_t block,
                                     int32_t n_active_heads, int32_t m_blocks, int32_t top_k,
                                     int32_t pooled_given) {
  (void)top_k;
  if (nq <= 0 || l_max <= 0 || block <= 0 || m_blocks <= 0 || n_active_heads <= 0 || n_heads <= 0)
    return 0;
  return plan_misa_hisa(nq, n_heads, head_dim, n_seq, l_max, block, m_blocks,
                        pooled_given != 0).total;
}

int misa_hisa_topk(const void* q, const float* w, const void* k, const void* k_pooled,
                   int32_t dtype, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                   int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max, int32_t block,
                   int32_t n_active_heads, int32_t m_blocks, int32_t top_k, int32_t* out_idx,
                   float* out_score, int32_t* out_heads, float* out_importance,
                   int32_t* out_blocks, float* out_block_score, int32_t* out_status,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_common(q, w, k, dtype, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k, out_idx);
  if (st) return st;
  if (dtype != DSA_DTYPE_BF16) return fail(DSA_EUNSUPPORTED, "MISA-HISA supports bf16 inputs only");
  if (block < 1) return fail(DSA_EINVAL, "block must be >= 1 (got %d)", block);
  if (n_active_heads < 1 || n_active_heads > n_heads)
    return fail(DSA_EINVAL, "n_active_heads must be in [1, n_heads] (got %d)", n_active_heads);
  if (m_blocks < 1) return fail(DSA_EINVAL, "m_blocks must be >= 1 (got %d)", m_blocks);
  if (nq == 0) return DSA_OK;
  if (k_pooled && !aligned(k_pooled, 16)) return fail(DSA_EINVAL, "k_pooled must be 16-byte aligned");
  if (!aligned(out_status, 4)) return fail(DSA_EINVAL, "out_status must be 4-byte aligned");
  MisaHisaPlan p = plan_misa_hisa(nq, n_heads, head_dim, n_seq, l_max, block, m_blocks,
                                  k_pooled != nullptr);
  if (!p.h.ok)
    return fail(DSA_EUNSUPPORTED, "MISA-HISA needs m_blocks <= %d, m_blocks * block <= %d, "
                "ceil(l_max / block) <= %d and nq <= 65535", dsa::kHisaMaxBlocks,
                dsa::kHisaRegKeys, dsa::kHisaMaxGroups * dsa::kHisaMaxChunk);
  if ((st = check_ws(workspace, workspace_bytes, p.total))) return st;
  const uint16_t* pooled = nullptr;
  uint16_t* partial = nullptr;
  if ((st = hisa_setup(p.h, k, k_pooled, q_seq, q_pos, nq, n_seq, head_dim, l_max, block,
                       workspace, stream, &pooled, &partial)))
    return st;
  // router: per-slice sums of max(0, q_j . kbar_b) over the pooled blocks
  dsa::RouteArgs ra{};
  ra.q = reinterpret_cast<const uint16_t*>(q);
  ra.pooled = pooled;
  ra.partial = partial;
  ra.q_seq = q_seq;
  ra.q_pos = q_pos;
  ra.nq = nq;
  ra.n_heads = n_heads;
  ra.head_dim = head_dim;
  ra.n_seq = n_seq;
  ra.block = block;
  ra.splits = p.splits;
  ra.blocks_per_split = p.bps;
  ra.l_max = l_max;
  ra.m_max = p.h.m_max;
  ra.part = at<float>(workspace, p.part);
  if ((st = hip_status(timed(DSA_KERNEL_ROUTE, stream, [&] { return dsa::launch_route(ra, stream); }),
                       "router kernel", stream))) return st;
  // HISA over the h most important heads, which k_hisa ranks from the sums
  HisaRoute route;
  route.part = ra.part;
  route.splits = p.splits;
  route.h_use = n_active_heads;
  route.out_heads = out_heads;
  route.out_importance = out_importance;
  return run_hisa_kernels(p.h, q, w, k, pooled, partial, q_seq, q_pos, route, nq, n_heads,
                          head_dim, n_seq, l_max, block, m_blocks, top_k, out_idx, out_score,
                          out_blocks, out_block_score, out_status, workspace, stream);
}

}  // extern "C"

// --------------------------------------------------- certified exact top-k ----

namespace {

// workspace of the certified call: two histograms and the survivor counts
// (cleared), the bounds, the screened heads, every key's upper bound, the
// screening selection, the survivor lists, and one set of candidate segments
// shared by the screening pass and the rescoring (they run one after the other)
struct CertPlan {
  StagePlan s0, s1;
  size_t zero_bytes = 0, cnt = 0, cert = 0, heads = 0, ub = 0, lb_idx = 0, lb_score = 0,
         list = 0, total = 0;
};

CertPlan plan_cert(int64_t nq, int head_dim, int64_t l_max, int h, int top_k) {
  CertPlan p;
  Arena A;
  plan_zero(A, p.s0, nq);
  plan_zero(A, p.s1, nq);
  p.cnt = A.take((size_t)nq * 4);
  p.zero_bytes = A.off;
  p.cert = A.take((size_t)nq * 16);
  p.heads = A.take((size_t)nq * h * 4);
  p.ub = A.take((size_t)nq * l_max * 4);
  p.lb_idx = A.take((size_t)nq * top_k * 4);
  p.lb_score = A.take((size_t)nq * top_k * 4);
  p.list = A.take((size_t)nq * l_max * 4);
  plan_cand(A, p.s0, nq, l_max, 0, head_dim);
  p.s1.chunk = p.s0.chunk;
  p.s1.n_chunks = p.s0.n_chunks;
  p.s1.cand = p.s0.cand;
  p.s1.cnt = p.s0.cnt;
  p.total = A.off;
  return p;
}

}  // namespace

extern "C" {

size_t indexer_certified_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                             int32_t n_seq, int64_t l_max,
                                             int32_t n_screen_heads, int32_t top_k) {
  (void)n_heads;
  (void)n_seq;
  if (nq <= 0 || l_max <= 0 || top_k <= 0 || n_screen_heads <= 0) return 0;
  return plan_cert(nq, head_dim, l_max, n_screen_heads, top_k).total;
}

int indexer_certified_topk(const void* q, const float* w, const void* k, int32_t dtype,
                           const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                           int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                           int32_t n_screen_heads, int32_t top_k, int32_t* out_idx,
                           float* out_score, int32_t* out_survivors, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  int st = check_common(q, w, k, dtype, q_pos, nq, n_heads, head_dim, n_seq, l_max, top_k, out_idx);
  if (st) return st;
  if (dtype != DSA_DTYPE_BF16) return fail(DSA_EUNSUPPORTED, "the certified call supports bf16 only");
  if (n_screen_heads < 1 || n_screen_heads > n_heads || n_screen_heads > dsa::kCertMaxHeads)
    return fail(DSA_EINVAL, "n_screen_heads must be in [1, min(n_heads, %d)] (got %d)",
                dsa::kCertMaxHeads, n_screen_heads);
  if (l_max > (int64_t)65535 * 4096)
    return fail(DSA_EUNSUPPORTED, "l_max above %lld is not supported by the certified call",
                (long long)65535 * 4096);
  if (out_survivors && !aligned(out_survivors, 4))
    return fail(DSA_EINVAL, "out_survivors must be 4-byte aligned");
  if (nq == 0) return DSA_OK;
  const CertPlan p = plan_cert(nq, head_dim, l_max, n_screen_heads, top_k);
  if ((st = check_ws(workspace, workspace_bytes, p.total))) return st;
  if ((st = run_prepare(workspace, p.zero_bytes, k, q_seq, q_pos, nq, n_seq, head_dim, 1, l_max,
                        nullptr, stream)))
    return st;
  dsa::CertArgs c{};
  c.q = reinterpret_cast<const uint16_t*>(q);
  c.w = w;
  c.q_seq = q_seq;
  c.q_pos = q_pos;
  c.nq = nq;
  c.n_heads = n_heads;
  c.head_dim = head_dim;
  c.n_seq = n_seq;
  c.h = n_screen_heads;
  c.top_k = top_k;
  c.l_max = l_max;
  c.heads = at<int32_t>(workspace, p.heads);
  c.cert = at<float>(workspace, p.cert);
  c.lb_idx = at<int32_t>(workspace, p.lb_idx);
  c.lb_score = at<float>(workspace, p.lb_score);
  c.ub = at<float>(workspace, p.ub);
  c.list = at<int32_t>(workspace, p.list);
  c.cnt = at<uint32_t>(workspace, p.cnt);
  if ((st = hip_status(timed(DSA_KERNEL_CERTIFY, stream,
                             [&] { return dsa::launch_certify_heads(c, stream); }),
                       "certify heads kernel", stream)))
    return st;
  // screening pass: the screened heads, ranked by lower bound, upper bounds stored
  dsa::SelArgs a = stage_args(p.s0, workspace);
  fill_common(a, q, w, k, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max);
  a.mode = dsa::MODE_RANGE;
  a.heads = c.heads;
  a.heads_stride = n_screen_heads;
  a.h_use = n_screen_heads;
  a.cert = c.cert;
  a.ub = at<float>(workspace, p.ub);
  a.ub_stride = l_max;
  a.top_k = top_k;
  a.out_idx = at<int32_t>(workspace, p.lb_idx);
  a.out_score = at<float>(workspace, p.lb_score);
  if ((st = hip_status(run_score_select(a, stream), "screening score/select kernel", stream)))
    return st;
  // survivors: upper bound at or above the k-th lower bound
  if ((st = hip_status(timed(DSA_KERNEL_CERTIFY, stream,
                             [&] { return dsa::launch_certify_compact(c, stream); }),
                       "certify compact kernel", stream)))
    return st;
  // every head over the survivors
  dsa::SelArgs b = stage_args(p.s1, workspace);
  fill_common(b, q, w, k, q_seq, q_pos, nq, n_heads, head_dim, n_seq, l_max);
  b.mode = dsa::MODE_LIST;
  b.list = c.list;
  b.list_len = (int)l_max;
  b.list_count = reinterpret_cast<const int32_t*>(c.cnt);
  b.top_k = top_k;
  b.out_idx = out_idx;
  b.out_score = out_score;
  if ((st = hip_status(run_score_select(b, stream), "rescore/select kernel", stream))) return st;
  if (!out_survivors) return DSA_OK;
  c.out_survivors = out_survivors;
  return hip_status(timed(DSA_KERNEL_CERTIFY, stream,
                          [&] { return dsa::launch_certify_counts(c, stream); }),
                    "certify counts kernel", stream);
}

}  // extern "C"

namespace {

// Sparse attention: each query's list in `splits` slices of whole 32-row
// steps, enough slices for about kTargetWorkgroups / 2 workgroups (one
// 8-wave workgroup fills a compute unit), at most kMlaMaxTiles steps each.
struct MlaPlan {
  int splits = 1, tiles_per_split = 1;
  size_t part_o = 0, part_ml = 0, total = 0;
};

MlaPlan plan_mla(int64_t nq, int n_heads, int top_k) {
  MlaPlan p;
  const int64_t tiles = cdiv(top_k, dsa::kMlaTile);
  // about one workgroup per compute unit: a workgroup takes one (query,
  // slice) and 64 heads (32 when 64 does not divide n_heads)
  const int64_t head_blocks = n_heads % 64 == 0 ? n_heads / 64 : n_heads / 32;
  int64_t splits = std::max<int64_t>(1, cdiv(kComputeUnits, nq * head_blocks));
  splits = std::min<int64_t>({splits, tiles, dsa::kMlaMaxSplits});
  splits = std::max<int64_t>(splits, cdiv(tiles, dsa::kMlaMaxTiles));
  p.tiles_per_split = (int)cdiv(tiles, splits);
  p.splits = (int)cdiv(tiles, p.tiles_per_split);
  if (p.splits > 1) {
    Arena A;
    p.part_o = A.take((size_t)nq * p.splits * n_heads * dsa::kMlaDv * 2);
    p.part_ml = A.take((size_t)nq * p.splits * n_heads * 8);
    p.total = A.off;
  }
  return p;
}

}  // namespace

extern "C" {

size_t sparse_mla_workspace_size(int32_t nq, int32_t n_heads, int32_t d_qk, int32_t d_v,
                                 int32_t top_k) {
  (void)d_qk;
  (void)d_v;
  if (nq <= 0 || n_heads <= 0 || top_k <= 0 || top_k > dsa::kMlaMaxTopK) return 0;
  return plan_mla(nq, n_heads, top_k).total;
}

int sparse_mla_attention(const void* q, const void* kv, int32_t dtype, const int32_t* q_seq,
                         const int32_t* q_pos, const int32_t* idx, int32_t nq, int32_t n_heads,
                         int32_t d_qk, int32_t d_v, int32_t n_seq, int64_t l_max, int32_t top_k,
                         float softmax_scale, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (dtype != DSA_DTYPE_BF16) return fail(DSA_EUNSUPPORTED, "sparse attention supports bf16 only");
  if (d_qk != dsa::kMlaDqk || d_v != dsa::kMlaDv)
    return fail(DSA_EUNSUPPORTED, "d_qk must be %d and d_v %d (got %d, %d)", dsa::kMlaDqk,
                dsa::kMlaDv, d_qk, d_v);
  if (n_heads < 32 || n_heads > 128 || n_heads % 32)
    return fail(DSA_EUNSUPPORTED, "n_heads must be 32, 64, 96 or 128 (got %d)", n_heads);
  if (top_k < 1 || top_k > dsa::kMlaMaxTopK)
    return fail(DSA_EUNSUPPORTED, "top_k must be in [1, %d] (got %d)", dsa::kMlaMaxTopK, top_k);
  if (nq < 0 || n_seq < 1 || l_max < 1) return fail(DSA_EINVAL, "bad nq / n_seq / l_max");
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f))
    return fail(DSA_EINVAL, "softmax_scale must be positive and finite");
  if (nq == 0) return DSA_OK;
  if (!q || !kv || !q_pos || !idx || !out)
    return fail(DSA_EINVAL, "q, kv, q_pos, idx and out must not be NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(DSA_EINVAL, "q, kv and out must be 16-byte aligned");
  if (!aligned(q_pos, 4) || !aligned(idx, 4) || (q_seq && !aligned(q_seq, 4)))
    return fail(DSA_EINVAL, "q_seq, q_pos and idx must be 4-byte aligned");
  const MlaPlan p = plan_mla(nq, n_heads, top_k);
  int st;
  if ((st = check_ws(workspace, workspace_bytes, p.total))) return st;
  dsa::MlaArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.kv = reinterpret_cast<const uint16_t*>(kv);
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.idx = idx;
  a.nq = nq;
  a.n_heads = n_heads;
  a.n_seq = n_seq;
  a.top_k = top_k;
  a.splits = p.splits;
  a.tiles_per_split = p.tiles_per_split;
  a.l_max = l_max;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = reinterpret_cast<uint16_t*>(out);
  a.part_o = p.splits > 1 ? at<uint16_t>(workspace, p.part_o) : nullptr;
  a.part_ml = p.splits > 1 ? at<float2>(workspace, p.part_ml) : nullptr;
  return hip_status(timed(DSA_KERNEL_MLA, stream, [&] { return dsa::launch_sparse_mla(a, stream); }),
                    "sparse attention kernel", stream);
}

int indexer_selection_iou(const int32_t* a, const int32_t* b, int32_t nq, int32_t k,
                          float* out_iou, hipStream_t stream) {
  if (nq < 0) return fail(DSA_EINVAL, "nq must be >= 0");
  if (k < 1 || k > 8192) return fail(DSA_EUNSUPPORTED, "k must be in [1, 8192] (got %d)", k);
  if (nq == 0) return DSA_OK;
  if (!a || !b || !out_iou) return fail(DSA_EINVAL, "a, b and out_iou must not be NULL");
  return hip_status(timed(DSA_KERNEL_IOU, stream,
                          [&] { return dsa::launch_iou(a, b, nq, k, out_iou, stream); }),
                    "IoU kernel", stream);
}

}  // extern "C"
