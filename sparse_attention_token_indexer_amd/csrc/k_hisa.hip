// HISA for decode-shaped calls (HISA review, section 3: block scores of the
// query against mean-pooled block keys, the top-m blocks, then the tokens of
// the surviving blocks scored with the full indexer and the exact top-k among
// them) in two kernels.
//
// k_hisa: per query, block-pass and token-pass workgroups share its work.
// When the grid fits the chip at once it is (G, nq) and every workgroup takes
// part in both passes; otherwise (many queries) it is 1-D, every query's
// block-pass items first and the token-pass items after, so that no
// workgroup waits for a selection on a slot that block-pass work still needs.
//  1. block pass: workgroup g scores pooled blocks [g*ch1, (g+1)*ch1) into LDS
//     and writes those whose 12-bit bin is at or above its local top-m bin (a
//     superset of its part of the query's top-m).  The last of the query's
//     block-pass workgroups to arrive selects the exact top-m from these
//     candidates and publishes each kept block as id + 1 in a cleared array.
//  2. token pass: workgroup g waits for the entries of that array its items
//     need, scores token items [g*ch2, (g+1)*ch2) of the block list (item i =
//     token list[i / block] * block + i % block) and stores their keys.
// k_hisa_topk, one workgroup per query: the exact top-k of the token keys.
// (The final selection is a kernel of its own: inside k_hisa its scalar
// register needs pushed the whole kernel into heavy spilling.)
//
// Data that one workgroup of k_hisa writes and another reads (candidates,
// counts, the block list) is stored and loaded with device-scope accesses,
// which bypass the per-die L2 copies; a workgroup drains its stores (vmcnt 0)
// before it bumps the arrival counter, so the workgroup that sees the final
// count sees the data.  (A device-scope fence would instead write back and
// invalidate the whole L2 at every step, which costs far more than the work.)
// Only the token pass waits, and only for its query's block selection, which
// block-pass work that never waits produces: in the (G, nq) grid a query's
// workgroups are consecutive in dispatch order (blockIdx.x runs fastest), so
// the query groups dispatched first can always finish and free room for the
// rest; in the 1-D grid every block-pass item precedes every token-pass
// item.  The waits are also bounded in time (HisaArgs::spin_ticks): a
// workgroup whose wait times out marks its query in the query's sync words and
// stops; k_hisa_topk then writes an all-padding row for that query and reports
// it in out_status, so an incomplete query never returns a partial selection.
#include "dsa_hisa.h"
#include "dsa_internal.h"
#include "dsa_scorers.h"
#include "dsa_select.h"

namespace dsa {

static_assert(kBins == kHisaBins, "histogram size shared with the host plan");
static_assert(kHisaMaxBlocks <= 1024, "k_hisa_topk reads one kept block per thread");

namespace {

constexpr int kHT = 256;                        // threads per workgroup
constexpr int kHW = kHT / 64;
constexpr int kPB = kBins / kHT;                // histogram bins per thread
constexpr int kTT = 1024;                       // threads of the selection kernel
constexpr int kHistWords = Hist<kHT>::kWords;
DSA_DEVICE int hpad(int b) { return Hist<kHT>::at(b); }
constexpr int kSU = 8;                          // entries per thread per pass step
static_assert(kSU * kTT >= kHisaRegKeys, "k_hisa_topk loads every token key in one batch");
constexpr int kHisaSegRead = 128;               // candidate slots read per segment up front

enum SyncWord {
  S_ARRIVE1 = 0,                  // block-pass workgroups done
  S_TIMEOUT = kHisaSyncTimeout,   // a wait of this query timed out
};

// Device-scope stores and loads of data shared between workgroups.
DSA_DEVICE void st_dev(uint2* p, uint2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), ((uint64_t)v.y << 32) | v.x,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEVICE void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEVICE void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEVICE uint2 ld_dev(const uint2* p) {
  const uint64_t x = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<uint2*>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)x, (uint32_t)(x >> 32));
}
DSA_DEVICE uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEVICE int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every memory operation this wave issued has completed (the
// device-scope stores are then visible to every workgroup).
DSA_DEVICE void drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// (key, id) pairs in per-workgroup segments of device memory, walked as one
// flat index space (off[c] = first flat index of segment c, in LDS).
struct DevSegSource {
  const uint2* cand;
  const uint32_t* off;
  int n_seg;
  int seg_len;
  DSA_DEVICE uint2 at(uint32_t f) const {
    int lo = 0, hi = n_seg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= f) lo = mid; else hi = mid;
    }
    return ld_dev(cand + (size_t)lo * seg_len + (f - off[lo]));
  }
  template <int NT, class F>
  DSA_DEVICE void for_each(F&& f) const {
    constexpr int U = 8;
    const uint32_t total = off[n_seg];
    for (uint32_t base = 0; base < total; base += NT * U) {
      uint2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t fi = base + threadIdx.x + u * NT;
        if (fi < total) v[u] = at(fi);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t fi = base + threadIdx.x + u * NT;
        if (fi < total) f(v[u]);
      }
    }
  }
};

// Thread-level wait until *p != 0; returns *p, or 0 (and the query marked)
// when `ticks` of the wall clock pass first.
DSA_DEVICE int32_t wait_nonzero(int32_t* p, uint32_t* timeout_word, uint64_t ticks) {
  int32_t v = ld_dev(p);
  if (v != 0) return v;
  const uint64_t t0 = wall_clock64();
  while ((v = ld_dev(p)) == 0) {
    __builtin_amdgcn_s_sleep(1);
    if (wall_clock64() - t0 > ticks) {
      __hip_atomic_store(timeout_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return 0;
    }
  }
  return v;
}

// Scores items [0, n) of this workgroup into skey (key 0 = not a valid item)
// and, with COUNT, counts every valid key in the LDS histogram.  row(j, id)
// gives item j's key row and id (id < 0: not a valid item, the row is a safe
// stand-in).  Each wave keeps its next NF tiles of 32 items in flight.
template <class SC, int NF, bool COUNT, class RowF>
DSA_DEVICE void score_items(const SC& sc, int n, RowF&& row, uint32_t* skey, uint32_t* hist) {
  const int lane = lane_id(), wv = wave_id();
  const int n_tiles = (n + 31) / 32;
  typename SC::Frag f[NF];
  auto load = [&](int tile, typename SC::Frag& fr) {
    const uint16_t* rows[SC::kRows];
#pragma unroll
    for (int k = 0; k < SC::kRows; ++k) {
      const int j = tile * 32 + SC::row_key(k);
      int32_t id;
      rows[k] = row(j < n ? j : 0, id);
    }
    SC::load(fr, rows);
  };
  static_for<NF>([&](auto i) {
    const int tile = wv + (int)i * kHW;
    if (tile < n_tiles) load(tile, f[i]);
  });
  for (int base = wv; base < n_tiles; base += NF * kHW) {
    static_for<NF>([&](auto i) {
      const int tile = base + (int)i * kHW;
      if (tile < n_tiles) {
        const float s = sc.score(f[i]);
        const int nx = tile + NF * kHW;
        if (nx < n_tiles) load(nx, f[i]);
        const int j = tile * 32 + lane;
        if (lane < 32 && j < n) {
          int32_t id;
          (void)row(j, id);
          const uint32_t k = id >= 0 ? score_to_key(s) : 0u;
          skey[j] = k;
          if (COUNT && k) atomicAdd(&hist[hpad((int)(k >> kBinShift))], 1u);
        }
      }
    });
  }
}

// Highest bin b with (count of bins >= b) >= need, or 0 when the histogram
// holds fewer than need entries.  Collective; hist is a padded LDS histogram.
DSA_DEVICE int local_bin(const uint32_t* hist, uint32_t need, uint32_t* scratch, int* s_b) {
  const int b0 = kBins - kPB * ((int)threadIdx.x + 1);
  uint32_t h[kPB], mine = 0;
#pragma unroll
  for (int j = 0; j < kPB; ++j) {
    h[j] = hist[hpad(b0) + j];
    mine += h[j];
  }
  if (threadIdx.x == 0) *s_b = 0;
  uint32_t total;
  const uint32_t before = block_exclusive_sum<kHT>(mine, scratch, &total);
  if (total >= need && before < need && before + mine >= need) {
    uint32_t acc = before;
#pragma unroll
    for (int j = kPB - 1; j >= 0; --j) {
      acc += h[j];
      if (acc >= need) {
        *s_b = b0 + j;
        break;
      }
    }
  }
  __syncthreads();
  return *s_b;
}

// Exact top-k of the entries of src (key 0 entries are skipped): Kt =
// min(top_k, valid entries) are emitted, slots [Kt, top_k) of em's row are
// padded with (-1, -inf).  12-bit histogram, everything above the k-th
// entry's bin, then that bin resolved in LDS (or by the radix finish over src
// when it overflows the list).  em's counter must hold 0.
template <class Src>
DSA_DEVICE void select_exact(const Src& src, uint32_t top_k, const Emitter& em, uint32_t* hist,
                             uint32_t* scratch, uint2* list, uint32_t lcap, uint2* tie,
                             uint32_t* s_ln) {
  for (int i = threadIdx.x; i < kBins; i += kHT) hist[i] = 0;
  if (threadIdx.x == 0) *s_ln = 0;
  __syncthreads();
  src.template for_each<kHT>([&](uint2 e) {
    if (e.x) atomicAdd(&hist[e.x >> kBinShift], 1u);
  });
  __syncthreads();
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kPB; ++j) mine += hist[threadIdx.x * kPB + j];
  uint32_t n_valid;
  (void)block_exclusive_sum<kHT>(mine, scratch, &n_valid);
  const uint32_t Kt = n_valid < top_k ? n_valid : top_k;
  for (uint32_t i = Kt + threadIdx.x; i < top_k; i += kHT) {
    em.out_idx[i] = -1;
    if (em.out_score) em.out_score[i] = -__builtin_inff();
  }
  if (Kt == 0) return;
  uint32_t above;
  const int bstar = block_find_threshold<kHT>(hist, kBins, Kt, scratch, &above);
  const uint32_t nb = hist[bstar];
  const uint32_t need = Kt - above;
  const bool fits = nb <= lcap;
  src.template for_each<kHT>([&](uint2 e) {
    if (!e.x) return;
    const int b = (int)(e.x >> kBinShift);
    if (b > bstar) {
      em.put(e.x, (int32_t)e.y);
    } else if (fits && b == bstar) {
      const uint32_t o = atomicAdd(s_ln, 1u);
      if (o < lcap) list[o] = e;
    }
  });
  __syncthreads();
  if (fits) {
    const uint32_t nl = *s_ln < nb ? *s_ln : nb;
    if (need < nl && nl <= 64) rank_finish64(list, nl, need, em);
    else finish_bin<kHT>(list, nl, need, bstar, em, hist, scratch, tie);
  } else {
    const uint64_t prefix = (uint64_t)bstar << (64 - kBinBits);
    const uint64_t mask = (uint64_t)(kBins - 1) << (64 - kBinBits);
    radix_finish<kHT>(src, prefix, mask, 64 - kBinBits, need, nb, em, hist, scratch);
  }
}

// MISA head routing finished inside a workgroup: the router's per-slice sums
// added in slice order, I_j = |w_j| * sum, the h_use heads of largest I (ties
// to the lower index) into s_heads.  The arithmetic and order are fixed, so
// every workgroup of a query keeps the same heads.  The query's sums are
// contiguous ([slice][head]): they come into buf (buf_words words, free until
// the block pass) with one coalesced load per round, thread j then adds head
// j's slices.
static_assert(kHT >= 64, "one thread per head in the routing step");
DSA_DEVICE void hisa_route_heads(const HisaArgs& a, int t, float* buf, int buf_words,
                                 int32_t* s_heads, float* s_I, bool report) {
  const int H = a.n_heads, tid = (int)threadIdx.x;
  const int per = buf_words / H;                               // slices per round
  const float* part = a.route_part + (size_t)t * a.route_splits * H;
  float tot = 0.f;
  for (int s0 = 0; s0 < a.route_splits; s0 += per) {
    const int ns = a.route_splits - s0 < per ? a.route_splits - s0 : per;
    for (int i = tid; i < ns * H; i += (int)blockDim.x) buf[i] = part[(size_t)s0 * H + i];
    __syncthreads();
    if (tid < H)
      for (int sp = 0; sp < ns; ++sp) tot += buf[sp * H + tid];
    __syncthreads();
  }
  if (tid < H) {
    const float I = fabsf(a.w[(size_t)t * H + tid]) * tot;
    s_I[tid] = I;
    if (report && a.out_importance) a.out_importance[(size_t)t * H + tid] = I;
  }
  __syncthreads();
  if (tid < H) {
    // (order-preserving keys of I: a total order even for NaN, so the ranks
    // are a permutation and every routed slot gets a head)
    const uint32_t Ij = score_to_key(s_I[tid]);
    int rank = 0;
    for (int i = 0; i < H; ++i) {
      const uint32_t Ii = score_to_key(s_I[i]);
      rank += (Ii > Ij) || (Ii == Ij && i < tid);
    }
    if (rank < a.h_use) {
      s_heads[rank] = tid;
      if (report && a.out_heads) a.out_heads[(size_t)t * a.h_use + rank] = tid;
    }
  }
  __syncthreads();
}

template <class SC, int NF, int D>
__global__ __launch_bounds__(kHT) __attribute__((amdgpu_waves_per_eu(2))) void k_hisa(HisaArgs a) {
  extern __shared__ uint32_t smem[];
  const int chmax = a.ch1 > a.ch2 ? a.ch1 : a.ch2;
  uint32_t* skey = smem;                                        // [chmax]
  uint32_t* hist = skey + chmax;                                // [kHistWords]
  uint32_t* scratch = hist + kHistWords;                        // [64]
  const int g1 = a.split ? a.groups1 : a.groups, g2 = a.split ? a.groups2 : a.groups;
  uint32_t* off = scratch + 64;                                 // [g1 + 2]
  uint32_t* scnt = off + g1 + 2;                                // [g1]
  int32_t* sblk = reinterpret_cast<int32_t*>(scnt + g1);        // [sblk_n]
  int32_t* sbid = sblk + a.sblk_n;                              // [m_blocks] kept blocks
  float* sbsc = reinterpret_cast<float*>(sbid + a.m_blocks);    // [m_blocks] their scores
  uint2* list = reinterpret_cast<uint2*>(smem + hisa_list_offset_words(a));   // [kHisaListCap]
  uint2* tie = list + kHisaListCap;                             // [64]
  uint2* cl = tie + 64;                                         // [kHisaCandCap] block candidates
  __shared__ uint32_t s_cnt, s_ln, s_out, s_sel, s_go;
  __shared__ int s_b;
  __shared__ SelVars sv;
  __shared__ int32_t s_heads[64];
  __shared__ float s_I[64];

  // grid: (groups, nq), each workgroup taking part in both passes; or, with
  // split, a 1-D grid of the block-pass items of every query followed by the
  // token-pass items (each query's items consecutive)
  int t, g;
  bool pass1, pass2;
  if (a.split) {
    const int nb1 = a.nq * g1;
    pass1 = (int)blockIdx.x < nb1;
    pass2 = !pass1;
    const int bid = pass1 ? (int)blockIdx.x : (int)blockIdx.x - nb1;
    const int gq = pass1 ? g1 : g2;
    t = bid / gq;
    g = bid - t * gq;
  } else {
    g = blockIdx.x;
    t = blockIdx.y;
    pass1 = pass2 = true;
  }
  const int tid = (int)threadIdx.x, lane = lane_id();
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  int32_t* blocks = a.blocks + (size_t)t * a.m_blocks;
  float* bscore = a.out_block_score ? a.out_block_score + (size_t)t * a.m_blocks : nullptr;
  if (!(seq >= 0 && seq < a.n_seq && pos >= 0 && pos < a.l_max)) {   // no keys: padding only
    if (pass1 && g == 0) {                       // (k_hisa_topk pads the top-k row)
      for (int i = tid; i < a.m_blocks; i += kHT) {
        blocks[i] = -1;
        if (bscore) bscore[i] = -__builtin_inff();
      }
      if (a.route_part) {
        for (int j = tid; j < a.h_use; j += kHT)
          if (a.out_heads) a.out_heads[(size_t)t * a.h_use + j] = -1;
        for (int j = tid; j < a.n_heads; j += kHT)
          if (a.out_importance) a.out_importance[(size_t)t * a.n_heads + j] = 0.f;
      }
    }
    return;
  }
  const int M = (int)((pos + a.block) / a.block);               // pooled blocks of the prefix
  const int m1 = a.m_blocks < M ? a.m_blocks : M;               // blocks kept
  const int n1 = (M + a.ch1 - 1) / a.ch1;                       // block-pass workgroups
  const int items2 = m1 * a.block;                              // token items (list slots)
  const int n2 = (items2 + a.ch2 - 1) / a.ch2;                  // token-pass workgroups
  pass1 = pass1 && g < n1;
  pass2 = pass2 && g < n2;
  if (!pass1 && !pass2) return;
  uint32_t* sy = a.sync + (size_t)t * kHisaSyncWords;
  int32_t* bflag = a.bflag + (size_t)t * a.m_blocks;            // kept block + 1 (0: not yet)

  const int32_t* heads_t = a.heads ? a.heads + (size_t)t * a.heads_stride : nullptr;
  if (a.route_part) {
    hisa_route_heads(a, t, reinterpret_cast<float*>(hist), kHistWords, s_heads, s_I,
                     pass1 && g == 0);
    heads_t = s_heads;
  }
  SC sc;
  sc.init(a.q + (size_t)t * a.n_heads * D, a.w + (size_t)t * a.n_heads, heads_t, a.h_use,
          nullptr);
  // ---- 1. block pass
  if (pass1) {
    for (int i = tid; i < kHistWords; i += kHT) hist[i] = 0;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    const int i0 = g * a.ch1;
    const int nc = (M - i0) < a.ch1 ? (M - i0) : a.ch1;
    const bool part = ((pos + 1) % a.block) != 0;
    const uint16_t* pool_s = a.pooled + (size_t)seq * (size_t)a.m_max * D;
    const uint16_t* part_t = a.partial + (size_t)t * D;
    auto row1 = [&](int j, int32_t& id) -> const uint16_t* {
      const int b = i0 + j;
      id = b;
      return (part && b == M - 1) ? part_t : pool_s + (size_t)b * D;
    };
    score_items<SC, NF, true>(sc, nc, row1, skey, hist);
    __syncthreads();
    const int bl = local_bin(hist, (uint32_t)m1, scratch, &s_b);
    // candidates: every block of a bin >= bl, at consecutive slots (per wave
    // one LDS atomic, then ballots: each store instruction writes consecutive
    // slots)
    uint2* seg = a.cand1 + ((size_t)t * g1 + g) * a.ch1;
    const int rounds = (nc + kHT - 1) / kHT;
    uint32_t cw = 0;
    for (int r = 0; r < rounds; ++r) {
      const int j = tid + r * kHT;
      const uint32_t k = j < nc ? skey[j] : 0u;
      cw += (uint32_t)__popcll(__ballot(k && (int)(k >> kBinShift) >= bl));
    }
    uint32_t wb = 0;
    if (lane == 0 && cw) wb = atomicAdd(&s_cnt, cw);
    wb = (uint32_t)__builtin_amdgcn_readlane((int)wb, 0);
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int r = 0; r < rounds; ++r) {
      const int j = tid + r * kHT;
      const uint32_t k = j < nc ? skey[j] : 0u;
      const bool take = k && (int)(k >> kBinShift) >= bl;
      const uint64_t m = __ballot(take);
      if (take) st_dev(seg + wb + (uint32_t)__popcll(m & lt), make_uint2(k, (uint32_t)(i0 + j)));
      wb += (uint32_t)__popcll(m);
    }
    __syncthreads();
    if (tid == 0) st_dev(&a.cnt1[(size_t)t * g1 + g], s_cnt);
    drain();
    __syncthreads();
    if (tid == 0) s_sel = atomicAdd(&sy[S_ARRIVE1], 1u) == (uint32_t)(n1 - 1) ? 1u : 0u;
    __syncthreads();
    if (s_sel) {
      // The exact top-m1 of all candidates.  The segment counts and the first
      // S entries of every segment are loaded in one round (entries past a
      // segment's count are dropped); longer segments are completed after.
      const uint2* cbase = a.cand1 + (size_t)t * g1 * a.ch1;
      int S = (int)kHisaCandCap / n1 < a.ch1 ? (int)kHisaCandCap / n1 : a.ch1;
      if (S > kHisaSegRead) S = kHisaSegRead;         // a segment holds about m1
      constexpr int U = kHisaCandCap / kHT;
      uint32_t c = 0;
      if (tid < n1) c = ld_dev(&a.cnt1[(size_t)t * g1 + tid]);
      uint2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = tid + u * kHT, sg = f / S;
        if (sg < n1) v[u] = ld_dev(cbase + (size_t)sg * a.ch1 + (f - sg * S));
      }
      // (the selection's histogram is cleared while the loads are in flight;
      // the barrier of the scan below orders it before the first count)
      for (int i = tid; i < kHistWords; i += kHT) hist[i] = 0;
      if (c > (uint32_t)a.ch1) c = (uint32_t)a.ch1;
      if (tid < n1) scnt[tid] = c;
      uint32_t tot;
      const uint32_t ex = block_exclusive_sum<kHT>(c, scratch, &tot);
      if (tid < n1) off[tid] = ex;
      if (tid == 0) {
        off[n1] = tot;
        s_out = 0;
      }
      __syncthreads();
      if (tot <= kHisaCandCap) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int f = tid + u * kHT, sg = f / S, i = f - sg * S;
          if (sg < n1 && i < (int)scnt[sg]) cl[off[sg] + i] = v[u];
        }
        for (int sg = 0; sg < n1; ++sg)
          for (int i = S + tid; i < (int)scnt[sg]; i += kHT)
            cl[off[sg] + i] = ld_dev(cbase + (size_t)sg * a.ch1 + i);
        __syncthreads();
        uint32_t kk[kSU];
        int32_t ii[kSU];
#pragma unroll
        for (int u = 0; u < kSU; ++u) {
          const int i = tid + u * kHT;
          const uint2 e = i < (int)tot ? cl[i] : make_uint2(0u, 0u);
          kk[u] = e.x;
          ii[u] = (int32_t)e.y;
        }
        select_regs<kHT, kSU, kHisaListCap>(kk, ii, m1, sbid, sbsc, nullptr, 0u, hist, scratch,
                                            list, tie, cl, sv, true);
      } else {
        const Emitter em{sbid, sbsc, &s_out, (uint32_t)m1};     // into LDS, then out
        const DevSegSource src{cbase, off, n1, a.ch1};
        select_exact(src, (uint32_t)m1, em, hist, scratch, list, kHisaListCap, tie, &s_ln);
      }
      // the kept blocks: to the waiting token-pass workgroups (as id + 1) and out
      for (int i = tid; i < a.m_blocks; i += kHT) {
        if (i < m1) st_dev(&bflag[i], sbid[i] + 1);
        blocks[i] = i < m1 ? sbid[i] : -1;
        if (bscore) bscore[i] = i < m1 ? sbsc[i] : -__builtin_inff();
      }
    }
  }
  if (!pass2) return;

  // ---- 2. token pass: wait for this workgroup's block ids, score, store keys
  const int j0 = g * a.ch2;
  const int nc2 = (items2 - j0) < a.ch2 ? (items2 - j0) : a.ch2;
  const int li0 = j0 / a.block, li1 = (j0 + nc2 - 1) / a.block;
  if (tid == 0) s_go = 1;
  __syncthreads();
  for (int i = tid; i <= li1 - li0; i += kHT) {
    const int32_t v = wait_nonzero(&bflag[li0 + i], &sy[S_TIMEOUT], a.spin_ticks);
    if (v == 0) s_go = 0;
    sblk[i] = v - 1;
  }
  __syncthreads();
  if (!s_go) return;
  const uint16_t* keys_s = a.keys + (size_t)seq * (size_t)a.l_max * D;
  auto row2 = [&](int j, int32_t& id) -> const uint16_t* {
    const int it = j0 + j;
    const int li = it / a.block;
    const int b = sblk[li - li0];
    const int64_t u = (int64_t)b * a.block + (it - li * a.block);
    const bool v = b >= 0 && u <= pos;
    id = v ? (int32_t)u : -1;
    return keys_s + (size_t)(v ? u : 0) * D;
  };
  score_items<SC, NF, false>(sc, nc2, row2, skey, hist);
  __syncthreads();
  // the keys go to the query's key array; the selection kernel that follows
  // in stream order reads them
  uint32_t* keys_t = a.keys2 + (size_t)t * g2 * a.ch2;
  for (int j = tid; j < nc2; j += kHT) keys_t[j0 + j] = skey[j];
}

// The token pass's exact top-k: one workgroup per query reads the query's
// kept blocks and its (at most kHisaRegKeys) token keys, written by k_hisa
// before it in stream order, and selects from LDS.
__global__ __launch_bounds__(kTT) void k_hisa_topk(HisaArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;                                        // [Hist<kTT>::kWords]
  uint32_t* scratch = hist + Hist<kTT>::kWords;                 // [64]
  int32_t* sbid = reinterpret_cast<int32_t*>(scratch + 64);     // [m_blocks]
  uint2* list = reinterpret_cast<uint2*>(smem + hisa_topk_list_offset_words(a));   // [kHisaListCap]
  uint2* tie = list + kHisaListCap;                             // [64]
  uint2* stage = tie + 64;                                      // [kHisaCandCap]
  uint2* ent = stage + kHisaCandCap;                            // [kHisaRegKeys] radix spill
  __shared__ SelVars sv;
  const int t = blockIdx.x, tid = (int)threadIdx.x;
  // Every load in one round: the token keys of up to m_blocks * block items
  // (k_hisa stored the query's items2 <= m_blocks * block of them; slots past
  // items2 lie inside the query's key array and are masked below), the kept
  // blocks (m_blocks <= kTT: one per thread), the query's row and its timeout
  // word.
  const uint32_t* keys_t = a.keys2 + (size_t)t * (a.split ? a.groups2 : a.groups) * a.ch2;
  const int32_t* blocks = a.blocks + (size_t)t * a.m_blocks;
  const int items_max = a.m_blocks * a.block;
  uint32_t k[kSU];
#pragma unroll
  for (int u = 0; u < kSU; ++u) {
    const int i = tid + u * kTT;
    k[u] = i < items_max ? keys_t[i] : 0u;
  }
  const int32_t my_block = tid < a.m_blocks ? blocks[tid] : 0;
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  const uint32_t to_word = ld_dev(a.sync + (size_t)t * kHisaSyncWords + S_TIMEOUT);
  int32_t* out_i = a.out_idx + (size_t)t * a.top_k;
  float* out_s = a.out_score ? a.out_score + (size_t)t * a.top_k : nullptr;
  const bool valid = seq >= 0 && seq < a.n_seq && pos >= 0 && pos < a.l_max;
  // a token-pass workgroup of this query gave up its wait (k_hisa ended before
  // this kernel started, so the mark is final): its keys were never stored
  const bool timed_out = valid && to_word != 0u;
  if (a.out_status && tid == 0) a.out_status[t] = timed_out ? 1 : 0;
  if (!valid || timed_out) {                   // no keys, or incomplete: padding only
    for (int i = tid; i < a.top_k; i += kTT) {
      out_i[i] = -1;
      if (out_s) out_s[i] = -__builtin_inff();
    }
    return;
  }
  const int M = (int)((pos + a.block) / a.block);
  const int m1 = a.m_blocks < M ? a.m_blocks : M;
  const int items2 = m1 * a.block;
  if (tid < m1) sbid[tid] = my_block;
  __syncthreads();
  // token id of every item: item i = tid + u * kTT is token list[i / block] *
  // block + i % block; list index and offset advance by kTT per step without a
  // division (kSU * kTT = kHisaRegKeys >= items2: one batch)
  const int blk = a.block, step = kTT / blk, rem = kTT % blk;
  int li = tid / blk, r = tid % blk;
  int32_t idv[kSU];
#pragma unroll
  for (int u = 0; u < kSU; ++u) {
    const int i = tid + u * kTT;
    if (i >= items2) k[u] = 0u;
    idv[u] = sbid[li < m1 ? li : m1 - 1] * blk + r;
    li += step;
    r += rem;
    if (r >= blk) {
      r -= blk;
      ++li;
    }
  }
  select_regs<kTT, kSU, kHisaListCap>(k, idv, a.top_k, out_i, out_s, stage, kHisaCandCap, hist,
                                      scratch, list, tie, ent, sv, false);
}

template <class SC, int NF, int D>
hipError_t launch_hisa_t(const HisaArgs& a, hipStream_t stream) {
  auto k = k_hisa<SC, NF, D>;
  const size_t lds = hisa_lds_bytes(a);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (a.split)
    hipLaunchKernelGGL(k, dim3(a.nq * (a.groups1 + a.groups2)), dim3(kHT), lds, stream, a);
  else
    hipLaunchKernelGGL(k, dim3(a.groups, a.nq), dim3(kHT), lds, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t lds2 = hisa_topk_lds_bytes(a);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_hisa_topk),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hisa_topk, dim3(a.nq), dim3(kTT), lds2, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hisa(const HisaArgs& a, hipStream_t stream) {
  const int gmax = a.split ? (a.groups1 > a.groups2 ? a.groups1 : a.groups2) : a.groups;
  const int gmin = a.split ? (a.groups1 < a.groups2 ? a.groups1 : a.groups2) : a.groups;
  if (gmin < 1 || gmax > kHisaMaxGroups || a.ch1 < 32 || a.ch2 < 32 ||
      (a.split && (int64_t)a.nq * (a.groups1 + a.groups2) > 0x7FFFFFFF) ||
      a.ch1 > kHisaMaxChunk || a.ch2 > kHisaMaxChunk || a.ch1 % 32 || a.ch2 % 32 ||
      a.sblk_n < a.ch2 / a.block + 2 || a.nq < 1 || a.nq > 65535 || a.m_blocks < 1 ||
      a.m_blocks > kHisaMaxBlocks || (int64_t)a.m_blocks * a.block > kHisaRegKeys)
    return hipErrorInvalidValue;
  if (a.h_use < 1 || a.h_use > a.n_heads || (a.heads && a.heads_stride < a.h_use))
    return hipErrorInvalidValue;
  if (a.route_part && (a.heads || a.route_splits < 1 || a.n_heads > 64))
    return hipErrorInvalidValue;
  if (a.head_dim == 128) {
    if (a.h_use <= 16) return launch_hisa_t<ScorerMfma16<128>, 4, 128>(a, stream);
    if (a.h_use <= 32) return launch_hisa_t<ScorerMfma32<1, 128>, 4, 128>(a, stream);
    return launch_hisa_t<ScorerMfma32<2, 128>, 3, 128>(a, stream);
  }
  if (a.head_dim == 64) {
    if (a.h_use <= 16) return launch_hisa_t<ScorerMfma16<64>, 4, 64>(a, stream);
    if (a.h_use <= 32) return launch_hisa_t<ScorerMfma32<1, 64>, 4, 64>(a, stream);
    return launch_hisa_t<ScorerMfma32<2, 64>, 4, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
