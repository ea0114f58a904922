// Score-and-select kernels for decode-shaped indexer work.
//
// k_score_emit: one workgroup = one query x one chunk of its items (prefix
// tokens, pooled blocks, or a gathered candidate list).  It streams the chunk's
// key rows straight from HBM into MFMA operands, computes the fused
// ReLU-weighted head reduction in registers and keeps the chunk's scores in LDS
// only; then it emits the chunk's candidates against a bound derived from the
// query's running score histogram (see dsa_select.h).
// k_merge: one workgroup per query merges the candidates into the exact top-k.
// No score vector is ever written to HBM and no workgroup waits on another.
//
// Method: the DSA indexer scores every causal prefix token with H_I heads and
// keeps the top-k (MISA summary, "problem" section); MISA's routed pass scores
// with h gathered heads ("method" step 2) and its dagger variant rescores a
// candidate list with all heads ("hierarchical variant"); HISA scores pooled
// block keys, then the tokens of the surviving blocks (HISA review, section 3).
#include "dsa_internal.h"
#include "dsa_scorers.h"
#include "dsa_select.h"

namespace dsa {

namespace {

constexpr int kNT = 256;                 // score-and-emit workgroup
constexpr int kNW = kNT / 64;
constexpr int kMT = 1024;                // merge workgroup

struct Row {
  int seq;
  int64_t pos;
  int64_t n_items;
};

template <int MODE>
DSA_DEVICE Row row_of(const SelArgs& a, int t) {
  Row r;
  r.seq = a.q_seq ? a.q_seq[t] : 0;
  r.pos = a.q_pos[t];
  r.n_items = 0;
  if (r.seq >= 0 && r.seq < a.n_seq && r.pos >= 0 && r.pos < a.l_max) {
    if (MODE == MODE_RANGE) r.n_items = r.pos + 1;
    else if (MODE == MODE_POOLED) r.n_items = (r.pos + a.block) / a.block;
    else if (MODE == MODE_LIST)
      r.n_items = a.list_count ? (a.list_count[t] < 0 ? 0
                                  : (a.list_count[t] < a.list_len ? a.list_count[t] : a.list_len))
                               : a.list_len;
    else r.n_items = (int64_t)a.list_len * a.block;
  }
  return r;
}

// id of an item and the address of its key row; returns false (and a safe row
// address) for items that are not valid keys of this query.
template <int MODE>
DSA_DEVICE bool item_of(const SelArgs& a, int t, const Row& r, int64_t item, int32_t& id,
                        const uint16_t*& row) {
  const size_t eb = a.f32 ? 4 : 2;
  const char* kb = reinterpret_cast<const char*>(a.keys);
  const size_t seq_base = (size_t)r.seq * (size_t)a.l_max;
  int64_t v;
  bool ok = true;
  if (MODE == MODE_RANGE) {
    v = item;
  } else if (MODE == MODE_POOLED) {
    id = (int32_t)item;
    if (a.partial && item == r.n_items - 1 && ((r.pos + 1) % a.block) != 0) {
      row = a.partial + (size_t)t * a.head_dim;
    } else {
      row = a.pooled + ((size_t)r.seq * (size_t)a.m_max + (size_t)item) * a.head_dim;
    }
    return true;
  } else if (MODE == MODE_LIST) {
    v = a.list[(size_t)t * a.list_len + item];
    ok = v >= 0 && v <= r.pos;
  } else {
    int64_t b = a.list[(size_t)t * a.list_len + item / a.block];
    v = b * a.block + item % a.block;
    ok = b >= 0 && v <= r.pos;
  }
  if (!ok) v = 0;
  id = ok ? (int32_t)v : -1;
  row = reinterpret_cast<const uint16_t*>(kb + (seq_base + (size_t)v) * a.head_dim * eb);
  return ok;
}

template <class SC, int MODE>
DSA_DEVICE void load_tile(const SelArgs& a, int t, const Row& r, int64_t i0, int n_c, int tile,
                          typename SC::Frag& f) {
  const uint16_t* rows[SC::kRows];
#pragma unroll
  for (int k = 0; k < SC::kRows; ++k) {
    int j = tile * 32 + SC::row_key(k);
    int32_t id;
    const uint16_t* p;
    if (j < n_c) {
      item_of<MODE>(a, t, r, i0 + j, id, p);
    } else {
      item_of<MODE>(a, t, r, i0, id, p);   // in-range stand-in; result is discarded
    }
    rows[k] = p;
  }
  SC::load(f, rows);
}

template <class SC, int MODE>
DSA_DEVICE void store_score(const SelArgs& a, int t, const Row& r, int64_t i0, int n_c, int tile,
                            float s, uint32_t* skey) {
  const int lane = lane_id();
  const int j = tile * 32 + lane;
  if (lane < 32 && j < n_c) {
    bool ok = true;
    if (MODE == MODE_LIST || MODE == MODE_BLOCKS) {
      int32_t id;
      const uint16_t* p;
      ok = item_of<MODE>(a, t, r, i0 + j, id, p);
    }
    skey[j] = ok ? score_to_key(s) : 0u;
  }
}

// Certified screening pass: the screened score s of the item this lane holds
// and its key's norm |k| give the bounds of the full score,
//   LB = s + |k| N- - e,  UB = s + |k| N+ + e,  e = kCertRel (|s| + |k| M)
// (every head j left out adds w_j max(0, q_j . k) with 0 <= max(0, q_j . k)
// <= |q_j| |k|, Cauchy-Schwarz); the item is ranked by LB and UB is stored.
// A NaN bound ranks lowest (key 1), so it can only lower the threshold.
DSA_DEVICE void cert_store(const SelArgs& a, int t, int64_t i0, int n_c, int tile, float s,
                           float n2, const float (&cb)[3], uint32_t* skey) {
  const int lane = lane_id();
  const int j = tile * 32 + lane;
  if (lane < 32 && j < n_c) {
    const float nk = sqrtf(n2);
    const float e = kCertRel * (fabsf(s) + nk * cb[2]);
    const float lb = s + nk * cb[1] - e;
    skey[j] = lb == lb ? score_to_key(lb) : 1u;
    a.ub[(size_t)t * a.ub_stride + i0 + j] = s + nk * cb[0] + e;
  }
}

// MISA head routing, finished by every workgroup of the routed pass: adds the
// router's per-slice head sums in slice order, I_j = |w_j| * sum, and ranks the
// heads by (I desc, j asc).  The order is fixed, so every workgroup of a query
// obtains the same head set; the chunk-0 workgroup reports it.
DSA_DEVICE void route_heads(const SelArgs& a, int t, int32_t* s_heads, float* s_I, bool report) {
  const int H = a.n_heads;
  for (int j = threadIdx.x; j < H; j += blockDim.x) {
    float tot = 0.f;
    for (int sp = 0; sp < a.route_splits; ++sp)
      tot += a.route_part[((size_t)t * a.route_splits + sp) * H + j];
    const float I = fabsf(a.w[(size_t)t * H + j]) * tot;
    s_I[j] = I;
    if (report && a.out_importance) a.out_importance[(size_t)t * H + j] = I;
  }
  __syncthreads();
  // ranked on the order-preserving keys of I: a total order even for NaN,
  // so the ranks are a permutation and every routed slot gets a head
  for (int j = threadIdx.x; j < H; j += blockDim.x) {
    const uint32_t Ij = score_to_key(s_I[j]);
    int rank = 0;
    for (int i = 0; i < H; ++i) {
      const uint32_t Ii = score_to_key(s_I[i]);
      rank += (Ii > Ij) || (Ii == Ij && i < j);
    }
    if (rank < a.h_use) {
      s_heads[rank] = j;
      if (report && a.out_heads) a.out_heads[(size_t)t * a.h_use + rank] = j;
    }
  }
  __syncthreads();
}

// Kernel 1 of a selection pass: score one chunk of one query, emit candidates.
// CERT: the certified screening pass (ranked by lower bounds, see cert_store).
template <class SC, int MODE, bool CERT>
__global__ __launch_bounds__(kNT) void k_score_emit(SelArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* skey = smem;
  uint32_t* hist = smem + a.chunk;
  uint32_t* scratch = hist + kBins;
  float* sc_lds = reinterpret_cast<float*>(scratch + 64);

  __shared__ int32_t s_heads[64];
  __shared__ float s_I[64];
  const int t = blockIdx.x, c = blockIdx.y;
  const Row r = row_of<MODE>(a, t);
  if (r.n_items == 0) {                             // the merge pads the row
    if (a.route_part && c == 0) {
      for (int j = threadIdx.x; j < a.h_use; j += kNT)
        if (a.out_heads) a.out_heads[(size_t)t * a.h_use + j] = -1;
      for (int j = threadIdx.x; j < a.n_heads; j += kNT)
        if (a.out_importance) a.out_importance[(size_t)t * a.n_heads + j] = 0.f;
    }
    return;
  }
  const int n_chunks_t = (int)((r.n_items + a.chunk - 1) / a.chunk);
  if (c >= n_chunks_t) return;

  // ---- scores of this chunk into LDS
  const size_t eb = a.f32 ? 4 : 2;
  const uint16_t* q_t = reinterpret_cast<const uint16_t*>(
      reinterpret_cast<const char*>(a.q) + (size_t)t * a.n_heads * a.head_dim * eb);
  const float* w_t = a.w + (size_t)t * a.n_heads;
  const int32_t* heads_t = a.heads ? a.heads + (size_t)t * a.heads_stride : nullptr;
  if (a.route_part) {
    route_heads(a, t, s_heads, s_I, c == 0);
    heads_t = s_heads;
  }
  SC sc;
  sc.init(q_t, w_t, heads_t, a.h_use, sc_lds);
  const int64_t i0 = (int64_t)c * a.chunk;
  const int n_c = (int)((r.n_items - i0) < a.chunk ? (r.n_items - i0) : a.chunk);
  const int n_tiles = (n_c + 31) / 32;
  const int wv = wave_id();
  float cb[3] = {0.f, 0.f, 0.f};
  if constexpr (CERT) {
#pragma unroll
    for (int i = 0; i < 3; ++i) cb[i] = a.cert[(size_t)t * 4 + i];
  }
  auto put = [&](int tl, const typename SC::Frag& f) {
    if constexpr (CERT) cert_store(a, t, i0, n_c, tl, sc.score(f), SC::norm2(f), cb, skey);
    else store_score<SC, MODE>(a, t, r, i0, n_c, tl, sc.score(f), skey);
  };
  {
    // three tile fragments in rotation: while one tile is scored, the wave's
    // next two tiles are in flight.  The first two are requested before the
    // histogram clear and the barrier (they read no LDS), so their latency
    // overlaps the query loads'.
    typename SC::Frag fa, fb, fc;
    int tile = wv;
    if (tile < n_tiles) load_tile<SC, MODE>(a, t, r, i0, n_c, tile, fa);
    if (tile + kNW < n_tiles) load_tile<SC, MODE>(a, t, r, i0, n_c, tile + kNW, fb);
    for (int i = threadIdx.x; i < kBins; i += kNT) hist[i] = 0;   // counted after the loop
    __syncthreads();
    for (; tile < n_tiles; tile += 3 * kNW) {
      const int t1 = tile + kNW, t2 = tile + 2 * kNW, t3 = tile + 3 * kNW, t4 = tile + 4 * kNW;
      if (t2 < n_tiles) load_tile<SC, MODE>(a, t, r, i0, n_c, t2, fc);
      put(tile, fa);
      if (t1 >= n_tiles) break;
      if (t3 < n_tiles) load_tile<SC, MODE>(a, t, r, i0, n_c, t3, fa);
      put(t1, fb);
      if (t2 >= n_tiles) break;
      if (t4 < n_tiles) load_tile<SC, MODE>(a, t, r, i0, n_c, t4, fb);
      put(t2, fc);
    }
  }
  __syncthreads();

  // ---- this chunk's candidates
  uint2* seg = a.cand + ((size_t)t * a.n_chunks + c) * (size_t)a.chunk;
  auto id_of = [&](int i) -> int32_t {
    int32_t id;
    const uint16_t* p;
    item_of<MODE>(a, t, r, i0 + i, id, p);
    return id;
  };
  if (a.store_all) {           // short pass: every item, key 0 = not a valid key
    for (int i = threadIdx.x; i < n_c; i += kNT) {
      const uint32_t k = skey[i];
      seg[i] = make_uint2(k, k ? (uint32_t)id_of(i) : 0u);
    }
    return;
  }
  chunk_emit<kNT>(skey, n_c, a.top_k, id_of, seg, a.cand_cnt + (size_t)t * a.n_chunks + c,
                  a.ghist + (size_t)t * kBins, hist, scratch);
}

// Kernel 2 of a selection pass: exact merge of one query's candidates.
template <int MODE>
__global__ __launch_bounds__(kMT) void k_merge(SelArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;                              // [kBins]
  uint32_t* scratch = hist + kBins;                   // [64]
  uint32_t* off = scratch + 64;                       // [kMaxChunks + 1]
  uint2* list = reinterpret_cast<uint2*>(off + kMaxChunks + 1 + 1);   // 8-byte aligned
  const int t = blockIdx.x;
  const Row r = row_of<MODE>(a, t);
  const int n_chunks_t = (int)((r.n_items + a.chunk - 1) / a.chunk);
  merge_query<kMT>(a.cand + (size_t)t * a.n_chunks * a.chunk, a.cand_cnt + (size_t)t * a.n_chunks,
                   n_chunks_t, a.chunk, a.ghist + (size_t)t * kBins, a.top_k,
                   a.out_idx + (size_t)t * a.top_k,
                   a.out_score ? a.out_score + (size_t)t * a.top_k : nullptr, list, kMergeListCap,
                   off, hist, scratch);
}

constexpr size_t kMergeLds = (kBins + 64 + kMaxChunks + 2) * 4 + (size_t)kMergeListCap * 8;

// Short-pass selection: one workgroup per query selects from all its (key, id)
// pairs (key 0 = not a valid item), which the scoring kernel stored
// contiguously per query.  The pairs stay in registers (kShortPer per
// thread); one 12-bit histogram in LDS gives the bin b* of the k-th entry;
// one wave-aggregated pass emits every entry above b* and collects b*, which
// finish_bin resolves (or, when b* overflows its LDS list, the radix finish
// over the query's pairs in memory).
constexpr int kST = 1024;
constexpr int kShortPer = kShortItems / kST;
constexpr uint32_t kShortListCap = 4096;
constexpr size_t kShortLds = (kBins + 64) * 4 + ((size_t)kShortListCap + 64) * 8;

template <int MODE>
__global__ __launch_bounds__(kST) void k_select_short(SelArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;                                    // [kBins]
  uint32_t* scratch = hist + kBins;                         // [64]
  uint2* list = reinterpret_cast<uint2*>(scratch + 64);     // [kShortListCap]
  uint2* tie = list + kShortListCap;                        // [64]
  __shared__ uint32_t s_out, s_ln;
  const int t = blockIdx.x, tid = (int)threadIdx.x;
  const Row r = row_of<MODE>(a, t);
  const int n = (int)(r.n_items < kShortItems ? r.n_items : kShortItems);
  int32_t* out_i = a.out_idx + (size_t)t * a.top_k;
  float* out_s = a.out_score ? a.out_score + (size_t)t * a.top_k : nullptr;
  const uint2* row = a.cand + (size_t)t * a.n_chunks * a.chunk;
  uint2 e[kShortPer];
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {
    const int i = tid + j * kST;
    e[j] = i < n ? row[i] : make_uint2(0u, 0u);
  }
  for (int i = tid; i < kBins; i += kST) hist[i] = 0;
  if (tid == 0) { s_out = 0; s_ln = 0; }
  __syncthreads();
  uint32_t nv = 0;
#pragma unroll
  for (int j = 0; j < kShortPer; ++j)
    if (e[j].x) {
      atomicAdd(&hist[e[j].x >> kBinShift], 1u);
      ++nv;
    }
  uint32_t n_valid;
  (void)block_exclusive_sum<kST>(nv, scratch, &n_valid);
  const uint32_t Kt = n_valid < (uint32_t)a.top_k ? n_valid : (uint32_t)a.top_k;
  for (int i = (int)Kt + tid; i < a.top_k; i += kST) {
    out_i[i] = -1;
    if (out_s) out_s[i] = -__builtin_inff();
  }
  if (Kt == 0) return;
  uint32_t above;
  const int bstar = block_find_threshold<kST>(hist, kBins, Kt, scratch, &above);
  const uint32_t nb = hist[bstar];
  const uint32_t need = Kt - above;
  const Emitter em{out_i, out_s, &s_out, Kt};
  const bool fits = nb <= kShortListCap;
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {
    const bool valid = e[j].x != 0u;
    const int b = (int)(e[j].x >> kBinShift);
    em.put_wave(valid && b > bstar, e[j].x, (int32_t)e[j].y);
    if (fits) list_put_wave(valid && b == bstar, e[j], list, &s_ln, kShortListCap);
  }
  __syncthreads();
  if (fits) {
    const uint32_t nl = s_ln < nb ? s_ln : nb;
    finish_bin<kST>(list, nl, need, bstar, em, hist, scratch, tie);
  } else {
    const uint64_t prefix = (uint64_t)bstar << (64 - kBinBits);
    const uint64_t mask = (uint64_t)(kBins - 1) << (64 - kBinBits);
    PairSource src{row, (uint32_t)n};
    radix_finish<kST>(src, prefix, mask, 64 - kBinBits, need, nb, em, hist, scratch);
  }
}

template <int MODE>
hipError_t launch_select_short_t(const SelArgs& a, hipStream_t stream) {
  auto k = k_select_short<MODE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kShortLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.nq), dim3(kST), kShortLds, stream, a);
  return hipGetLastError();
}

template <class SC, int MODE, bool CERT = false>
hipError_t launch_t(const SelArgs& a, hipStream_t stream) {
  if (a.n_chunks > kMaxChunks) return hipErrorInvalidValue;
  const size_t lds = score_select_lds_bytes(a.chunk, a.f32, a.head_dim);
  auto k1 = k_score_emit<SC, MODE, CERT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k1, dim3(a.nq, a.n_chunks), dim3(kNT), lds, stream, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_merge_t(const SelArgs& a, hipStream_t stream) {
  if (a.n_chunks > kMaxChunks) return hipErrorInvalidValue;
  auto k2 = k_merge<MODE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k2),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMergeLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k2, dim3(a.nq), dim3(kMT), kMergeLds, stream, a);
  return hipGetLastError();
}

template <class SC>
hipError_t launch_mode(const SelArgs& a, hipStream_t stream) {
  switch (a.mode) {
    case MODE_RANGE: return launch_t<SC, MODE_RANGE>(a, stream);
    case MODE_POOLED: return launch_t<SC, MODE_POOLED>(a, stream);
    case MODE_LIST: return launch_t<SC, MODE_LIST>(a, stream);
    case MODE_BLOCKS: return launch_t<SC, MODE_BLOCKS>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t score_select_lds_bytes(int chunk, int f32, int head_dim) {
  size_t b = (size_t)chunk * 4 + kBins * 4 + 64 * 4;
  if (f32) b += (size_t)(64 * head_dim + 64) * 4;
  return b;
}

hipError_t launch_select_short(const SelArgs& a, hipStream_t stream) {
  if ((int64_t)a.n_chunks * a.chunk < 1) return hipErrorInvalidValue;
  switch (a.mode) {
    case MODE_RANGE: return launch_select_short_t<MODE_RANGE>(a, stream);
    case MODE_POOLED: return launch_select_short_t<MODE_POOLED>(a, stream);
    case MODE_LIST: return launch_select_short_t<MODE_LIST>(a, stream);
    case MODE_BLOCKS: return launch_select_short_t<MODE_BLOCKS>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const SelArgs& a, hipStream_t stream) {
  switch (a.mode) {
    case MODE_RANGE: return launch_merge_t<MODE_RANGE>(a, stream);
    case MODE_POOLED: return launch_merge_t<MODE_POOLED>(a, stream);
    case MODE_LIST: return launch_merge_t<MODE_LIST>(a, stream);
    case MODE_BLOCKS: return launch_merge_t<MODE_BLOCKS>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score_emit(const SelArgs& a, hipStream_t stream) {
  if (a.cert) {                 // certified screening pass: bf16, prefix tokens, <= 16 heads
    if (a.f32 || a.mode != MODE_RANGE || a.h_use < 1 || a.h_use > kCertMaxHeads || !a.ub ||
        a.ub_stride < a.l_max)
      return hipErrorInvalidValue;
    if (a.head_dim == 128) return launch_t<ScorerMfma16<128>, MODE_RANGE, true>(a, stream);
    if (a.head_dim == 64) return launch_t<ScorerMfma16<64>, MODE_RANGE, true>(a, stream);
    return hipErrorInvalidValue;
  }
  if (a.f32) {
    if (a.mode != MODE_RANGE) return hipErrorInvalidValue;
    if (a.head_dim == 64) return launch_t<ScorerF32<64>, MODE_RANGE>(a, stream);
    if (a.head_dim == 128) return launch_t<ScorerF32<128>, MODE_RANGE>(a, stream);
    return hipErrorInvalidValue;
  }
  if (a.head_dim == 128) {
    if (a.h_use <= 16) return launch_mode<ScorerMfma16<128>>(a, stream);
    if (a.h_use <= 32) return launch_mode<ScorerMfma32<1, 128>>(a, stream);
    return launch_mode<ScorerMfma32<2, 128>>(a, stream);
  }
  if (a.head_dim == 64) {
    if (a.h_use <= 16) return launch_mode<ScorerMfma16<64>>(a, stream);
    if (a.h_use <= 32) return launch_mode<ScorerMfma32<1, 64>>(a, stream);
    return launch_mode<ScorerMfma32<2, 64>>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
