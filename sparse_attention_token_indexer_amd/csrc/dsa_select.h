// Exact top-k selection machinery shared by the scoring kernels.
//
// Selection order is the composite (score key desc, id asc), see dsa_common.h.
//
// Two kernels per selection pass, with no ordering between workgroups of one
// kernel:
//  * score-and-emit: every chunk of a query adds the 12-bit histogram of ALL its
//    scores to the query's global histogram, reads back the running histogram
//    and appends to its workspace segment every entry whose bin is at or above
//    the highest bin b with (running count of bins >= b) >= top_k.  The running
//    counts only ever under-count entries that exist, so that bin never exceeds
//    the bin of the query's k-th best entry: the segments always hold the exact
//    top-k, whatever the other chunks have published so far.
//  * merge: after the kernel boundary the histogram is complete; one workgroup
//    per query finds the bin b* of the k-th entry, emits every candidate above
//    it and resolves b* itself by further radix digits over the composite key,
//    in LDS when the bin fits, else by re-reading the segments.
#pragma once
#include "dsa_common.h"

namespace dsa {

struct Emitter {
  int32_t* out_idx;    // row base
  float* out_score;    // row base or null
  uint32_t* counter;   // LDS slot counter
  uint32_t cap;        // slots available in the row
  DSA_DEVICE void write(uint32_t o, uint32_t key, int32_t id) const {
    if (o >= cap) return;
    out_idx[o] = id;
    if (out_score) out_score[o] = key_to_score(key);
  }
  DSA_DEVICE void put(uint32_t key, int32_t id) const { write(atomicAdd(counter, 1u), key, id); }
  // Wave-collective: every lane of the wave calls it; lanes with take set
  // append their entry (one LDS atomic per wave).
  DSA_DEVICE void put_wave(bool take, uint32_t key, int32_t id) const {
    const uint64_t m = __ballot(take);
    if (!m) return;
    const int lane = lane_id();
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = __shfl(base, 0, 64);
    if (take) write(base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull)), key, id);
  }
};

// Wave-collective append of (key, id) to an LDS list of capacity cap.
DSA_DEVICE void list_put_wave(bool take, uint2 e, uint2* list, uint32_t* count, uint32_t cap) {
  const uint64_t m = __ballot(take);
  if (!m) return;
  const int lane = lane_id();
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(count, (uint32_t)__popcll(m));
  base = __shfl(base, 0, 64);
  const uint32_t o = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
  if (take && o < cap) list[o] = e;
}

// (key, id) pairs at a plain pointer (LDS or device memory).
struct PairSource {
  const uint2* e;
  uint32_t n;
  template <int NT, class F>
  DSA_DEVICE void for_each(F&& f) const {
    for (uint32_t i = threadIdx.x; i < n; i += NT) f(e[i]);
  }
};

// Entries held in global per-chunk segments, walked as one flat index space
// (off[c] = first flat index of chunk c, off[n_chunks] = total) so that every
// thread keeps several independent loads in flight.
struct FlatSegSource {
  const uint2* cand;        // query base: [n_chunks][chunk]
  const uint32_t* off;      // LDS, n_chunks + 1 prefix offsets
  int n_chunks;
  int chunk;
  DSA_DEVICE uint2 at(uint32_t f) const {
    int lo = 0, hi = n_chunks;              // last c with off[c] <= f
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (off[mid] <= f) lo = mid; else hi = mid;
    }
    return cand[(size_t)lo * chunk + (f - off[lo])];
  }
  template <int NT, class F>
  DSA_DEVICE void for_each(F&& f) const {
    constexpr int U = 8;
    const uint32_t total = off[n_chunks];
    for (uint32_t base = 0; base < total; base += NT * U) {
      uint2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t fi = base + threadIdx.x + u * NT;
        if (fi < total) v[u] = at(fi);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t fi = base + threadIdx.x + u * NT;
        if (fi < total) f(v[u]);
      }
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

// Exact finish of a tied first-level bin held in LDS (list[0..nl), all entries
// share the top FB bits of their key): emit the `need` best by composite order.
// One 10-bit digit histogram narrows the tie to a sub-bin; if that holds at
// most 64 entries they are ranked by brute force inside one wave, otherwise the
// general radix finish takes over.  hist needs 1024 words, tie 64 pairs of LDS.
template <int NT, int FB = kBinBits>
DSA_DEVICE void finish_bin(const uint2* list, uint32_t nl, uint32_t need, int bstar,
                           const Emitter& em, uint32_t* hist, uint32_t* scratch, uint2* tie) {
  __shared__ uint32_t s_tn;
  if (need == 0) return;
  if (need >= nl) {
    for (uint32_t i = threadIdx.x; i < nl; i += NT) em.put(list[i].x, (int32_t)list[i].y);
    __syncthreads();
    return;
  }
  constexpr int D2 = 10;
  constexpr int SH2 = 32 - FB - D2;                // the 10 key bits below the first level
  for (int i = threadIdx.x; i < (1 << D2); i += NT) hist[i] = 0;
  if (threadIdx.x == 0) s_tn = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nl; i += NT)
    atomicAdd(&hist[(list[i].x >> SH2) & ((1u << D2) - 1u)], 1u);
  __syncthreads();
  uint32_t above2;
  const int d2 = block_find_threshold<NT>(hist, 1 << D2, need, scratch, &above2);
  const uint32_t nd2 = hist[d2];
  const uint32_t need2 = need - above2;
  __syncthreads();
  for (uint32_t base = 0; base < nl; base += NT) {
    const uint32_t i = base + threadIdx.x;
    const uint2 e = i < nl ? list[i] : make_uint2(0u, 0u);
    const int dg = i < nl ? (int)((e.x >> SH2) & ((1u << D2) - 1u)) : -1;
    em.put_wave(dg > d2, e.x, (int32_t)e.y);
    if (nd2 <= 64) list_put_wave(dg == d2, e, tie, &s_tn, 64u);
  }
  __syncthreads();
  if (need2 == 0) return;
  if (nd2 <= 64) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const uint32_t nt = s_tn < nd2 ? s_tn : nd2;
      const bool have = (uint32_t)lane < nt;
      const uint2 me = have ? tie[lane] : make_uint2(0u, 0u);
      const uint64_t cm = composite(me.x, (int32_t)me.y);
      uint32_t rank = 0;
      for (uint32_t j = 0; j < nt; ++j) {
        const uint2 o = tie[j];
        rank += composite(o.x, (int32_t)o.y) > cm;
      }
      em.put_wave(have && rank < need2, me.x, (int32_t)me.y);
    }
    __syncthreads();
    return;
  }
  PairSource src{list, nl};
  const uint64_t prefix = ((uint64_t)bstar << (64 - FB)) | ((uint64_t)d2 << (32 + SH2));
  const uint64_t mask = ((uint64_t)((1u << (FB + D2)) - 1u)) << (32 + SH2);
  radix_finish<NT>(src, prefix, mask, 32 + SH2, need2, nd2, em, hist, scratch);
}

// Chunk-side half of a selection pass (run by every chunk workgroup).
// skey[0..n) holds the chunk's score keys (0 = invalid item); hist is LDS of
// kBins words, already zeroed (the caller has synchronised the workgroup).
// Appends the chunk's candidates (key, id) to seg and writes their count to
// *seg_cnt.
template <int NT, class IdOf>
DSA_DEVICE void chunk_emit(const uint32_t* skey, int n, int top_k, IdOf id_of, uint2* seg,
                           uint32_t* seg_cnt, uint32_t* ghist_g, uint32_t* hist,
                           uint32_t* scratch) {
  static_assert(kBins % NT == 0, "whole bin runs per thread");
  constexpr int PER = kBins / NT;
  constexpr int U = 8;
  __shared__ uint32_t s_cnt;
  __shared__ int s_bc;
  // the chunk's 12-bit histogram (keys read U at a time so that the reads
  // are in flight together)
  for (int base = 0; base < n; base += NT * U) {
    uint32_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + (int)threadIdx.x + u * NT;
      k[u] = i < n ? skey[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k[u]) atomicAdd(&hist[k[u] >> kBinShift], 1u);
  }
  __syncthreads();
  // Publish this chunk's histogram and read back the query's running counts
  // (bin b = threadIdx.x + j * NT: every instruction covers consecutive
  // words), never taking less than this chunk's own count (its own
  // publication may not be visible yet; other chunks' counts only ever
  // under-count).
  {
    uint32_t own[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) own[j] = hist[threadIdx.x + j * NT];
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (own[j]) atomicAdd(ghist_g + threadIdx.x + j * NT, own[j]);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t g = __hip_atomic_load(ghist_g + threadIdx.x + j * NT, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      hist[threadIdx.x + j * NT] = g > own[j] ? g : own[j];
    }
  }
  if (threadIdx.x == 0) { s_cnt = 0; s_bc = 0; }
  __syncthreads();
  // the bound: the highest bin b with (running count of bins >= b) >= top_k,
  // bin 0 (every entry) when the running counts hold fewer than top_k.
  // Thread t scans the run of PER bins just below the runs of threads < t.
  const int top = kBins - 1 - (int)threadIdx.x * PER;
  uint32_t cnt[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    cnt[i] = hist[top - i];
    mine += cnt[i];
  }
  uint32_t total;
  const uint32_t before = block_exclusive_sum<NT>(mine, scratch, &total);   // higher bins
  if (total >= (uint32_t)top_k && before < (uint32_t)top_k && before + mine >= (uint32_t)top_k) {
    uint32_t acc = before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      acc += cnt[i];
      if (acc >= (uint32_t)top_k) { s_bc = top - i; break; }
    }
  }
  __syncthreads();
  const int bc = s_bc;
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
  __syncthreads();
  if (threadIdx.x == 0) *seg_cnt = s_cnt;
}

// Brute-force finish of nl <= 64 entries held in LDS (distinct composites),
// by the first wave alone: entry i is emitted iff fewer than `need` entries
// beat it.
DSA_DEVICE void rank_finish64(const uint2* list, uint32_t nl, uint32_t need, const Emitter& em) {
  if (threadIdx.x < 64) {
    const uint32_t i = threadIdx.x;
    const bool have = i < nl;
    const uint2 me = have ? list[i] : make_uint2(0u, 0u);
    const uint64_t cm = composite(me.x, (int32_t)me.y);
    uint32_t rank = 0;
    for (uint32_t j = 0; j < nl; ++j) {         // every lane reads the same entry
      const uint2 o = list[j];
      rank += composite(o.x, (int32_t)o.y) > cm ? 1u : 0u;
    }
    em.put_wave(have && rank < need, me.x, (int32_t)me.y);
  }
  __syncthreads();
}

// Block-wide exclusive prefix of v (returned) and totals of v and u, with one
// pair of barriers.  scratch: 2 * NT / 64 words.
template <int NT>
DSA_DEVICE uint32_t block_exclusive_sum2(uint32_t v, uint32_t u, uint32_t* scratch,
                                         uint32_t* tot_v, uint32_t* tot_u) {
  constexpr int NW = NT / 64;
  const int lane = lane_id(), wv = wave_id();
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  uint32_t su = u;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) su += __shfl_xor(su, o, 64);
  if (lane == 63) scratch[wv] = x;
  if (lane == 0) scratch[NW + wv] = su;
  __syncthreads();
  uint32_t base = 0, tv = 0, tu = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t sv = scratch[i];
    if (i < wv) base += sv;
    tv += sv;
    tu += scratch[NW + i];
  }
  __syncthreads();
  *tot_v = tv;
  *tot_u = tu;
  return base + x - v;
}

// LDS histograms read by NT threads in runs of P = kBins / NT consecutive bins
// are padded with one word after every P bins, so the runs start on distinct
// banks.
template <int NT>
struct Hist {
  static constexpr int P = kBins / NT;
  static constexpr int kWords = kBins + kBins / P;
  DSA_DEVICE static int at(int b) { return b + b / P; }
};

// Shared scalars of one selection.
struct SelVars {
  uint32_t out, ln, above, nb;
  int b;
};

// Exact top-k of entries held in registers: thread tid holds entries tid + u *
// NT (u < U) as (k[u], id[u]), key 0 = empty.  Kt = min(top_k, valid entries)
// ids and scores go to out_idx / out_score (LDS or device memory), slots
// [Kt, top_k) are padded with (-1, -inf).
//  * First-level bins are linear in the score over the valid entries' own
//    range, bin = min(4095, (s - smin) * 4096 / (smax - smin)) (every step is
//    monotone, so the bins are ordered like the keys), which spreads one
//    query's scores evenly where bins of the key's top bits would put most of
//    them into the few bins of their shared exponents.  When the range is not
//    finite (infinite or NaN scores) the bins are the key's offset from the
//    smallest key, shifted to 12 bits.
//  * Entries above the k-th entry's bin b* take consecutive slots (a wave scan
//    of the per-thread counts, one LDS atomic per wave), through the LDS
//    `stage` (stage_cap pairs) when given, then in one coalesced copy.
//  * Entries in b* go to the LDS list (LCAP pairs), or, when they overflow
//    it, to `spill` (>= NT * U pairs of LDS that are free here), and are
//    resolved there by brute force (up to 64) or by the radix finish over
//    their whole (key, id) composites.
// hist must be zero on entry when `hist_clear` is set; scratch >= 64 words.
template <int NT, int U, uint32_t LCAP>
DSA_DEVICE void select_regs(const uint32_t (&k)[U], const int32_t (&id)[U], int top_k,
                            int32_t* out_idx, float* out_score, uint2* stage, uint32_t stage_cap,
                            uint32_t* hist, uint32_t* scratch, uint2* list, uint2* tie,
                            uint2* spill, SelVars& sv, bool hist_clear) {
  typedef Hist<NT> H;
  constexpr int PB = H::P;
  constexpr int NW = NT / 64;
  static_assert(3 * NW <= 64, "range reduction fits the scratch words");
  const int tid = (int)threadIdx.x, lane = lane_id(), wv = tid >> 6;
  // the valid entries' count and key range
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, nv = 0u;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (k[u]) {
      mn = k[u] < mn ? k[u] : mn;
      mx = k[u] > mx ? k[u] : mx;
      ++nv;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t a = (uint32_t)__shfl_xor((int)mn, o, 64);
    const uint32_t b = (uint32_t)__shfl_xor((int)mx, o, 64);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
    nv += (uint32_t)__shfl_xor((int)nv, o, 64);
  }
  if (lane == 0) {
    scratch[wv] = mn;
    scratch[NW + wv] = mx;
    scratch[2 * NW + wv] = nv;
  }
  if (!hist_clear)
    for (int i = tid; i < H::kWords; i += NT) hist[i] = 0;
  if (tid == 0) {
    sv.out = 0;
    sv.ln = 0;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
  nv = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t a = scratch[w], b = scratch[NW + w];
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
    nv += scratch[2 * NW + w];
  }
  const uint32_t Kt = nv < (uint32_t)top_k ? nv : (uint32_t)top_k;
  for (int i = (int)Kt + tid; i < top_k; i += NT) {
    out_idx[i] = -1;
    if (out_score) out_score[i] = -__builtin_inff();
  }
  if (Kt == 0) {                               // (every path ends at a barrier)
    __syncthreads();
    return;
  }
  const Emitter em{out_idx, out_score, &sv.out, Kt};
  if (nv <= (uint32_t)top_k) {                 // every valid entry
#pragma unroll
    for (int u = 0; u < U; ++u) em.put_wave(k[u] != 0u, k[u], id[u]);
    __syncthreads();
    return;
  }
  // first-level bins (see above)
  const float smin = key_to_score(mn), span = key_to_score(mx) - smin;
  const float scale = (float)kBins / span;
  const bool lin = span > 0.f && span <= 3.402823466e38f && scale <= 3.402823466e38f;
  const uint32_t range = mx - mn;
  const int len = range ? 32 - __clz((int)range) : 0;          // bits of the key range
  const int shift = len > kBinBits ? len - kBinBits : 0;
  auto bin_of = [&](uint32_t x) -> int {
    if (!lin) return (int)((x - mn) >> shift);
    const int b = (int)((key_to_score(x) - smin) * scale);
    return b < kBins - 1 ? b : kBins - 1;
  };
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (k[u]) atomicAdd(&hist[H::at(bin_of(k[u]))], 1u);
  __syncthreads();
  const int b0 = kBins - PB * (tid + 1);                   // this thread's bins, from the top
  uint32_t h[PB], mine = 0;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    h[j] = hist[H::at(b0) + j];
    mine += h[j];
  }
  uint32_t tot;
  const uint32_t before = block_exclusive_sum<NT>(mine, scratch, &tot);
  if (before < Kt && before + mine >= Kt) {
    uint32_t acc = before;
#pragma unroll
    for (int j = PB - 1; j >= 0; --j) {
      if (acc + h[j] >= Kt) {
        sv.b = b0 + j;
        sv.above = acc;
        sv.nb = h[j];
        break;
      }
      acc += h[j];
    }
  }
  __syncthreads();
  const int bstar = sv.b;
  const uint32_t above = sv.above, nb = sv.nb;
  const bool fits = nb <= LCAP;
  uint32_t na = 0, nt = 0;
  int bu[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    bu[u] = k[u] ? bin_of(k[u]) : -1;
    na += bu[u] > bstar ? 1u : 0u;
    nt += (fits && bu[u] == bstar) ? 1u : 0u;
  }
  const uint32_t cnt = na | (nt << 16);
  const uint32_t inc = wave_incl_scan(cnt);
  uint32_t base = 0;
  if (lane == 63) {
    if (inc & 0xffffu) base = atomicAdd(&sv.out, inc & 0xffffu);
    if (inc >> 16) base |= atomicAdd(&sv.ln, inc >> 16) << 16;
  }
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, 63);
  const uint32_t ex = inc - cnt;
  uint32_t oa = (base & 0xffffu) + (ex & 0xffffu), ot = (base >> 16) + (ex >> 16);
  const bool staged = stage != nullptr && above <= stage_cap;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (bu[u] > bstar) {
      if (oa < above) {
        if (staged) {
          stage[oa] = make_uint2(k[u], (uint32_t)id[u]);
        } else {
          out_idx[oa] = id[u];
          if (out_score) out_score[oa] = key_to_score(k[u]);
        }
      }
      ++oa;
    } else if (fits && bu[u] == bstar) {
      if (ot < LCAP) list[ot] = make_uint2(k[u], (uint32_t)id[u]);
      ++ot;
    }
  }
  __syncthreads();
  if (staged) {
    for (uint32_t base2 = 0; base2 < above; base2 += 8 * NT) {
      uint2 ev[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = base2 + tid + u * NT;
        ev[u] = i < above ? stage[i] : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = base2 + tid + u * NT;
        if (i < above) {
          out_idx[i] = (int32_t)ev[u].y;
          if (out_score) out_score[i] = key_to_score(ev[u].x);
        }
      }
    }
  }
  const uint32_t need = Kt - above;                        // sv.out == above here
  const uint2* ties = list;
  uint32_t nl = sv.ln < nb ? sv.ln : nb;
  if (!fits) {
    // the tied bin's entries into spill (sv.ln is still 0: nothing was listed)
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) c += bu[u] == bstar ? 1u : 0u;
    const uint32_t ci = wave_incl_scan(c);
    uint32_t sb = 0;
    if (lane == 63) sb = atomicAdd(&sv.ln, ci);
    sb = (uint32_t)__builtin_amdgcn_readlane((int)sb, 63) + (ci - c);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (bu[u] == bstar) spill[sb++] = make_uint2(k[u], (uint32_t)id[u]);
    __syncthreads();
    ties = spill;
    nl = nb;
  }
  if (need < nl && nl <= 64) rank_finish64(ties, nl, need, em);
  else radix_finish<NT>(PairSource{ties, nl}, 0ull, 0ull, 64, need, nl, em, hist, scratch);
}

// Merge of one query's candidates (merge kernel, one workgroup per query).
// ghist_g is the complete histogram of all the query's valid items; off_lds
// must hold n_chunks + 1 words; lds_list room for lcap pairs; hist kBins words;
// scratch 64 words.  Writes Kt = min(top_k, valid items) entries (any order),
// then (-1, -inf).
template <int NT>
DSA_DEVICE void merge_query(const uint2* cand, const uint32_t* cnt, int n_chunks, int chunk,
                            const uint32_t* ghist_g, int top_k, int32_t* out_idx,
                            float* out_score, uint2* lds_list, uint32_t lcap, uint32_t* off_lds,
                            uint32_t* hist, uint32_t* scratch) {
  static_assert(kBins % NT == 0 && 2 * NT / 64 <= 64, "merge block shape");
  constexpr int PER = kBins / NT;
  __shared__ uint32_t s_out, s_ln;
  const int tid = (int)threadIdx.x;
  // the histogram and the first NT segment counts are loaded together
  uint32_t h[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) h[j] = ghist_g[tid + j * NT];
  uint32_t v0 = 0;
  if (tid < n_chunks) {
    v0 = cnt[tid];
    if (v0 > (uint32_t)chunk) v0 = (uint32_t)chunk;   // clamp to the segment capacity
  }
  uint32_t nv = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    hist[tid + j * NT] = h[j];
    nv += h[j];
  }
  uint32_t run, n_valid;
  const uint32_t ex0 = block_exclusive_sum2<NT>(v0, nv, scratch, &run, &n_valid);
  if (tid < n_chunks) off_lds[tid] = ex0;
  for (int base = NT; base < n_chunks; base += NT) {     // more than NT chunks
    const int c = base + tid;
    uint32_t v = 0;
    if (c < n_chunks) {
      v = cnt[c];
      if (v > (uint32_t)chunk) v = (uint32_t)chunk;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_sum<NT>(v, scratch, &tot);
    if (c < n_chunks) off_lds[c] = run + ex;
    run += tot;
  }
  if (tid == 0) {
    off_lds[n_chunks] = run;
    s_out = 0;
    s_ln = 0;
  }
  const uint32_t Kt = n_valid < (uint32_t)top_k ? n_valid : (uint32_t)top_k;
  for (int i = Kt + tid; i < top_k; i += NT) {
    out_idx[i] = -1;
    if (out_score) out_score[i] = -__builtin_inff();
  }
  __syncthreads();
  if (Kt == 0) return;
  uint32_t above;
  const int bstar = block_find_threshold<NT>(hist, kBins, Kt, scratch, &above);
  const uint32_t nb = hist[bstar];
  const uint32_t need = Kt - above;
  __syncthreads();
  const Emitter em{out_idx, out_score, &s_out, Kt};
  const FlatSegSource seg{cand, off_lds, n_chunks, chunk};
  const bool fits = nb <= lcap;
  // one wave-uniform pass over the candidates: emit everything above the
  // k-th entry's bin, collect that bin
  {
    constexpr int U = 4;
    const uint32_t total = off_lds[n_chunks];
    for (uint32_t base = 0; base < total; base += NT * U) {
      uint2 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t f = base + tid + u * NT;
        e[u] = f < total ? seg.at(f) : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool valid = base + tid + u * NT < total;
        const int b = (int)(e[u].x >> kBinShift);
        em.put_wave(valid && b > bstar, e[u].x, (int32_t)e[u].y);
        if (fits) list_put_wave(valid && b == bstar, e[u], lds_list, &s_ln, lcap);
      }
    }
  }
  __syncthreads();
  const uint64_t prefix = (uint64_t)bstar << (64 - kBinBits);
  const uint64_t mask = (uint64_t)(kBins - 1) << (64 - kBinBits);
  if (fits) {
    const uint32_t nl = s_ln < nb ? s_ln : nb;   // the list holds s_ln <= lcap entries
    if (need < nl && nl <= 64) {
      rank_finish64(lds_list, nl, need, em);
    } else {
      PairSource src{lds_list, nl};
      radix_finish<NT>(src, prefix, mask, 64 - kBinBits, need, nl, em, hist, scratch);
    }
  } else {
    radix_finish<NT>(seg, prefix, mask, 64 - kBinBits, need, nb, em, hist, scratch);
  }
}

}  // namespace dsa
