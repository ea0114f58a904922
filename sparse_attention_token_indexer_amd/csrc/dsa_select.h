// Exact top-k selection machinery shared by the scoring kernels.
//
// Selection order is the composite (score key desc, id asc), see dsa_common.h.
// A query's candidates live in per-chunk segments of (key, id) pairs in the
// workspace; a first-level histogram over the top 12 key bits (ghist) has been
// accumulated for exactly those candidates.  The merge finds the 12-bit bin
// that holds the K-th entry, emits everything above it, and resolves the bin
// itself by further radix digits over the composite key: in LDS when the bin
// fits, otherwise by re-reading the segments from global memory.
#pragma once
#include "dsa_common.h"

namespace dsa {

struct Emitter {
  int32_t* out_idx;    // row base
  float* out_score;    // row base or null
  uint32_t* counter;   // LDS slot counter
  uint32_t cap;        // slots available in the row
  DSA_DEVICE void put(uint32_t key, int32_t id) const {
    uint32_t o = atomicAdd(counter, 1u);
    if (o >= cap) return;
    out_idx[o] = id;
    if (out_score) out_score[o] = key_to_score(key);
  }
};

// Entries held in LDS.
struct LdsSource {
  const uint2* e;
  uint32_t n;
  template <int NT, class F>
  DSA_DEVICE void for_each(F&& f) const {
    for (uint32_t i = threadIdx.x; i < n; i += NT) f(e[i]);
  }
};

// Entries held in global per-chunk segments.
struct SegSource {
  const uint2* cand;        // query base: [n_chunks][chunk]
  const uint32_t* cnt;      // query base: [n_chunks]
  int n_chunks;
  int chunk;
  template <int NT, class F>
  DSA_DEVICE void for_each(F&& f) const {
    for (int c = 0; c < n_chunks; ++c) {
      uint32_t n = cnt[c];
      const uint2* s = cand + (size_t)c * chunk;
      for (uint32_t i = threadIdx.x; i < n; i += NT) f(s[i]);
    }
  }
};

// Resolve the selection among the active entries (those whose composite key
// matches `prefix` on the bits of `mask`): emit exactly `need` of them, the
// best by composite order.  `n_active` is their count; bits below `next_shift`
// are still undecided.  hist must hold >= 256 entries of LDS.
template <int NT, class Src>
DSA_DEVICE void radix_finish(const Src& src, uint64_t prefix, uint64_t mask, int next_shift,
                             uint32_t need, uint32_t n_active, const Emitter& em,
                             uint32_t* hist, uint32_t* scratch) {
  while (true) {
    if (need == 0) return;
    if (need >= n_active) {
      src.template for_each<NT>([&](uint2 e) {
        uint64_t c = composite(e.x, (int32_t)e.y);
        if ((c & mask) == prefix) em.put(e.x, (int32_t)e.y);
      });
      __syncthreads();
      return;
    }
    const int nbits = next_shift >= 8 ? 8 : next_shift;
    const int shift = next_shift - nbits;
    const uint32_t dmask = (1u << nbits) - 1u;
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    src.template for_each<NT>([&](uint2 e) {
      uint64_t c = composite(e.x, (int32_t)e.y);
      if ((c & mask) == prefix) atomicAdd(&hist[(uint32_t)(c >> shift) & dmask], 1u);
    });
    __syncthreads();
    uint32_t above;
    int d = block_find_threshold<NT>(hist, 1 << nbits, need, scratch, &above);
    uint32_t nd = hist[d];
    __syncthreads();
    if (above) {
      src.template for_each<NT>([&](uint2 e) {
        uint64_t c = composite(e.x, (int32_t)e.y);
        if ((c & mask) == prefix && ((uint32_t)(c >> shift) & dmask) > (uint32_t)d)
          em.put(e.x, (int32_t)e.y);
      });
      __syncthreads();
    }
    need -= above;
    n_active = nd;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)dmask << shift;
    next_shift = shift;
    if (next_shift == 0) {  // fully decided: the remaining entries are unique
      if (need) {
        src.template for_each<NT>([&](uint2 e) {
          uint64_t c = composite(e.x, (int32_t)e.y);
          if ((c & mask) == prefix) em.put(e.x, (int32_t)e.y);
        });
        __syncthreads();
      }
      return;
    }
  }
}

// Final merge of one query (run by the last workgroup of that query).
// Writes Kt = min(top_k, n_valid) entries (any order) and pads to top_k with
// (-1, -inf).  lds_list has room for lcap (key, id) pairs; hist for kBins.
template <int NT>
DSA_DEVICE void merge_query(const uint2* cand, const uint32_t* cnt, int n_chunks, int chunk,
                            const uint32_t* ghist_g, uint32_t n_valid, int top_k,
                            int32_t* out_idx, float* out_score, uint2* lds_list, uint32_t lcap,
                            uint32_t* hist, uint32_t* scratch) {
  __shared__ uint32_t s_out, s_ln;
  const uint32_t Kt = n_valid < (uint32_t)top_k ? n_valid : (uint32_t)top_k;
  for (int i = Kt + threadIdx.x; i < top_k; i += NT) {
    out_idx[i] = -1;
    if (out_score) out_score[i] = -__builtin_inff();
  }
  if (Kt == 0) return;
  for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = __hip_atomic_load(
      ghist_g + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0) { s_out = 0; s_ln = 0; }
  __syncthreads();
  uint32_t above;
  const int bstar = block_find_threshold<NT>(hist, kBins, Kt, scratch, &above);
  const uint32_t nb = hist[bstar];
  const uint32_t need = Kt - above;
  __syncthreads();
  Emitter em{out_idx, out_score, &s_out, Kt};
  SegSource seg{cand, cnt, n_chunks, chunk};
  const bool fits = nb <= lcap;
  seg.for_each<NT>([&](uint2 e) {
    int b = (int)(e.x >> kBinShift);
    if (b > bstar) {
      em.put(e.x, (int32_t)e.y);
    } else if (b == bstar && fits) {
      uint32_t l = atomicAdd(&s_ln, 1u);
      if (l < lcap) lds_list[l] = e;
    }
  });
  __syncthreads();
  const uint64_t prefix = (uint64_t)bstar << (64 - kBinBits);
  const uint64_t mask = (uint64_t)(kBins - 1) << (64 - kBinBits);
  if (fits) {
    LdsSource src{lds_list, nb};
    radix_finish<NT>(src, prefix, mask, 64 - kBinBits, need, nb, em, hist, scratch);
  } else {
    radix_finish<NT>(seg, prefix, mask, 64 - kBinBits, need, nb, em, hist, scratch);
  }
}

// Chunk-local candidate emission.  skey[0..n) holds the chunk's score keys
// (0 = invalid item).  Every entry whose 12-bit bin is >= the bin of the
// chunk's k-th best is appended to seg (so the chunk's top-k is always
// included); their bin counts are added to the query's global histogram.
// Returns the number of valid items (all threads).
template <int NT, class IdOf>
DSA_DEVICE uint32_t chunk_emit(const uint32_t* skey, int n, int top_k, IdOf id_of,
                               uint2* seg, uint32_t* seg_cnt, uint32_t* ghist_g,
                               uint32_t* hist, uint32_t* scratch) {
  __shared__ uint32_t s_cnt;
  for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0;
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  uint32_t nv = 0;
  for (int i = threadIdx.x; i < n; i += NT) {
    uint32_t k = skey[i];
    if (k) { atomicAdd(&hist[k >> kBinShift], 1u); ++nv; }
  }
  uint32_t total;
  (void)block_exclusive_sum<NT>(nv, scratch, &total);
  __syncthreads();
  if (total == 0) {
    if (threadIdx.x == 0) *seg_cnt = 0;
    return 0;
  }
  const uint32_t kc = total < (uint32_t)top_k ? total : (uint32_t)top_k;
  uint32_t above;
  const int bc = block_find_threshold<NT>(hist, kBins, kc, scratch, &above);
  const int lane = lane_id();
  for (int base = 0; base < n; base += NT) {
    int i = base + (int)threadIdx.x;
    uint32_t k = i < n ? skey[i] : 0u;
    bool take = k != 0u && (int)(k >> kBinShift) >= bc;
    uint64_t m = __ballot(take);
    uint32_t wbase = 0;
    if (lane == 0 && m) wbase = atomicAdd(&s_cnt, (uint32_t)__popcll(m));
    wbase = __shfl(wbase, 0, 64);
    if (take) {
      uint32_t off = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      seg[wbase + off] = make_uint2(k, (uint32_t)id_of(i));
    }
  }
  for (int b = bc + (int)threadIdx.x; b < kBins; b += NT) {
    uint32_t h = hist[b];
    if (h) atomicAdd(ghist_g + b, h);
  }
  __syncthreads();
  if (threadIdx.x == 0) *seg_cnt = s_cnt;
  return total;
}

}  // namespace dsa
