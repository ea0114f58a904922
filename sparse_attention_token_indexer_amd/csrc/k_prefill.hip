// Prefill-shaped dense indexer: every query row t of one sequence scores its
// causal prefix u = 0..pos_t (MISA summary, "problem": the H_I-head indexer
// scores every prefix token; its cost grows as O(L^2) over a prefill, HISA
// review section 2) and keeps the exact top-k.
//
// k_prefill_score: one workgroup = 8 consecutive query rows, one wave
// per row with its query block (heads x 128) resident in registers.  The rows
// share the key cache: 128-key stages are staged in LDS (double-buffered, rows
// padded so the MFMA operand reads are free of bank conflicts) and each wave runs
// v_mfma_f32_32x32x16_bf16 with heads as rows and keys as columns, then the
// fused ReLU-weighted head reduction in registers.  Two 32-key sub-tiles are
// finished together (one lane-half exchange gives 64 consecutive keys' scores
// across the wave).  Scores go to a workspace row and into a per-row
// histogram in LDS; at the end each wave finds the bin that holds its row's
// k-th score.  Workgroups run longest rows first.  The histogram has 12-bit
// bins with 16-bit counters while a row holds at most 65535 keys, and 11-bit
// bins with 32-bit counters beyond (the same 8 KB of LDS per row).
// When there are too few row groups to fill the chip (decode queries sharing
// one cache, a short chunk of a long prefill), the keys are split as well:
// workgroup (g, c) scores its rows over key chunk c only, keeps no histogram
// (two workgroups then share a compute unit), and the row select splits each
// stored row into parts of 8192 keys: k_rows_count (one workgroup per part:
// the part's 12-bit histogram), k_rows_threshold (one per row: the parts'
// sum and the k-th key's bin), k_rows_emit (one per part: keys above the bin
// to the output, keys in it to a tie buffer) and k_rows_finish (one per row:
// the tie bin resolved exactly).  Kernel boundaries order the four; an
// agent-scope fence inside a kernel would write back and invalidate the whole
// L2 once per workgroup on this chip.
// k_prefill_select: one workgroup per row emits every score above that bin and
// resolves the bin itself exactly (radix digits over (score, ~index)).
#include "dsa_internal.h"
#include "dsa_common.h"
#include "dsa_select.h"

namespace dsa {

namespace {

constexpr int kStageKeys = 128;          // keys per LDS stage (2 pairs of 32-key sub-tiles)
constexpr int kPBinBits = kBinBits;      // per-row histogram: top 12 bits of the score key
constexpr int kPBins = 1 << kPBinBits;
constexpr int kPBinShift = 32 - kPBinBits;
constexpr int kST = 256;                 // select workgroup
constexpr uint32_t kSelListCap = 2048;   // tie-bin entries kept in LDS (global fallback beyond)

// Query rows per scoring workgroup (one wave each).  With 64 heads the row's
// query block takes 64 VGPRs; 8 rows keep each wave within 256 registers (two
// waves per SIMD) and the stages plus 8 KB histograms per row within 160 KB.
constexpr int kRows = 8;

template <int D, int ROWS, bool SPLIT = false>
constexpr size_t prefill_lds_bytes() {
  return 2 * (size_t)kStageKeys * (D * 2 + 16) + (SPLIT ? 0 : (size_t)ROWS * (kPBins / 2) * 4);
}

template <int HT, int D, int ROWS, bool W32, bool SPLIT>
__global__ __launch_bounds__(64 * ROWS) void k_prefill_score(PrefillArgs a) {
  constexpr int kPT = 64 * ROWS;
  constexpr int S = D / 16;                    // k-steps
  constexpr int RB = D * 2;                    // bytes per key row in the cache
  constexpr int NC = RB / 16;                  // 16-byte pieces per key row
  constexpr int LB = RB + 16;                  // LDS row stride: one pad piece per key
  constexpr int STAGE = kStageKeys * LB;       // bytes per LDS stage
  constexpr int PIECES = kStageKeys * NC;
  constexpr int LOADS = (PIECES + kPT - 1) / kPT;   // 16-byte loads per thread per stage
  constexpr int PAIRS = kStageKeys / 64;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* ktile = smem;                                           // [2][STAGE]
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + 2 * STAGE);  // [rows][kPBins / 2]
  __shared__ int s_maxpos;

  const int wv = wave_id(), lane = lane_id();
  const int grp = (int)gridDim.x - 1 - (int)blockIdx.x;            // longest rows first
  const int t = grp * ROWS + wv;
  int pos = -1;
  if (t < a.nq) {
    const int seq = a.q_seq ? a.q_seq[t] : 0;
    const int p = a.q_pos[t];
    if (seq == 0 && p >= 0 && (int64_t)p < a.l_max) pos = p;
  }
  if constexpr (!SPLIT)
    for (int i = threadIdx.x; i < ROWS * (kPBins / 2); i += kPT) hist[i] = 0u;
  if (threadIdx.x == 0) s_maxpos = -1;
  __syncthreads();
  if (lane == 0) atomicMax(&s_maxpos, pos);
  __syncthreads();
  const int maxpos = s_maxpos;
  if (maxpos < 0) return;                      // the select kernel pads these rows
  // keys [kb, ke) of this workgroup: the whole prefix of its rows, or with
  // SPLIT one chunk of it (whole stages; key_chunk is a multiple of 128)
  const int kb = SPLIT ? (int)blockIdx.y * a.key_chunk : 0;
  if (kb > maxpos) return;
  const int ke_last = SPLIT ? min(kb + a.key_chunk - 1, maxpos) : maxpos;   // last key scored
  const int n_stages = (ke_last - kb) / kStageKeys + 1;

  // this wave's query row in registers (zeros for an invalid row).  Head
  // weights: accumulator register r of head tile ht holds head
  // ht*32 + 8*(r/4) + 4*(lane/32) + r%4, and W[ht] holds that head's weight
  // for r = lane%16 in every 16-lane row, ready for a row broadcast.
  const int m = lane & 31, h = lane >> 5;
  bf16x8 qa[HT][S];
  float W[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int r = lane & 15;
    const int head = ht * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    W[ht] = (pos >= 0 && head < a.n_heads) ? a.w[(size_t)t * a.n_heads + head] : 0.f;
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int row = ht * 32 + m;
    const bool ok = pos >= 0 && row < a.n_heads;
    const uint16_t* src = a.q + ((size_t)t * a.n_heads + (ok ? row : 0)) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < S; ++s) qa[ht][s] = ok ? load_bf16x8(src + 16 * s) : zero_bf16x8();
  }
  // The padded row stride keeps both LDS access patterns conflict-free: 16
  // lanes storing one key's pieces touch 256 contiguous bytes, and 16 lanes
  // reading piece 2s+h of 16 consecutive keys start 4 banks apart.  The lane's
  // read offset is one base plus compile-time offsets.
  const uint32_t boff = (uint32_t)(m * LB + h * 16);

  // stage loading: thread piece p is key p / NC, piece p % NC.  A stage is
  // loaded in four slots, LOADS / 4 pieces per thread each (see the pipeline
  // below); pre[j] carries piece j from its global load to its LDS store.
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.keys);
  constexpr int PER_SLOT = (LOADS + 3) / 4;
  u32x4 pre[LOADS];
  static_assert(PIECES % kPT == 0, "every thread stores whole pieces");
  // (no branches around these memory operations: the wait counts before the
  // stores then stay exact.  Keys past the last stage are clamped to the last
  // key and land in a buffer nobody reads.)
  auto fetch_piece = [&](int j, int st) {
    const int p = threadIdx.x + j * kPT;
    const int key = min(kb + st * kStageKeys + p / NC, ke_last);   // inside the cache
    pre[j] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * RB + (p % NC) * 16);
  };
  auto stash_piece = [&](int j, int buf) {
    const int p = threadIdx.x + j * kPT;
    const int key = p / NC, pc = p % NC;
    *reinterpret_cast<u32x4*>(ktile + buf * STAGE + key * LB + pc * 16) = pre[j];
  };
  // slot q of the round that publishes stage st: store its pieces of slot q
  // and fetch the same pieces of stage st + 1 (one round = one stage ahead)
  auto slot = [&](int q, int st) {
#pragma unroll
    for (int j = q * PER_SLOT; j < (q + 1) * PER_SLOT && j < LOADS; ++j) {
      stash_piece(j, st & 1);
      fetch_piece(j, st + 1);
    }
  };
  // Finish of a pair of 32-key sub-tiles (keys key0 .. key0+63): one lane-half
  // swap of the two sub-tiles' partials puts key key0 + l in lane l, and the
  // two lane halves' partials of a key meet in one add.  Branch-free: every
  // lane stores (score rows span whole stages; a row that is not scored writes
  // the spare row) and keys past the row's position add 0 to the histogram.
  // Histogram bin b counts in word b % 2048: low half for b < 2048 (negative
  // scores, key bit 31 clear), high half otherwise.
  const int pos_u = __builtin_amdgcn_readfirstlane(pos);
  uint8_t* srow = reinterpret_cast<uint8_t*>(
      pos_u >= 0 ? a.scores + (size_t)__builtin_amdgcn_readfirstlane(t) * (size_t)a.row_stride
                 : a.spare_row);
  uint32_t* hrow = hist + wv * (kPBins / 2);
  float fin_sc = 0.f;
  auto fin_store = [&](int key0, float pa, float pb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb),
                                                     false, false);
    fin_sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    *reinterpret_cast<float*>(srow + (uint32_t)(kb + key0 + lane) * 4u) = fin_sc;
  };
  auto fin_count = [&](int key0) {
    if constexpr (SPLIT) {                     // (the select kernel counts the row)
      (void)key0;
    } else if constexpr (W32) {                // 11-bit bin b in word b, 32-bit counts
      const uint32_t word = fast_key(fin_sc) >> (kPBinShift + 1);
      atomicAdd(hrow + word, key0 + lane <= pos_u ? 1u : 0u);
    } else {
      const uint32_t word = (fast_key(fin_sc) >> kPBinShift) & (kPBins / 2 - 1);
      const uint32_t inc =
          key0 + lane <= pos_u ? ((int32_t)__float_as_uint(fin_sc) < 0 ? 1u : 0x10000u) : 0u;
      atomicAdd(hrow + word, inc);
    }
  };

  // Software pipeline over 32-key sub-tiles c = 0..3 of each 128-key stage
  // (the same count for every wave; keys past a row's position are computed
  // and dropped).  The sub-tile's S k-steps are S fenced steps; step s issues
  // both head tiles' MFMAs for k-step s (B operands read one sub-tile
  // earlier), reads the next sub-tile's B operand for k-step s, and adds 32 / S
  // accumulator registers of the previous sub-tile to its partial pe[c - 1].
  // Pair (0,1) of a stage is finished in its sub-tile 3, pair (2,3) in the next
  // stage's sub-tile 1 (store in one step, count in the next).  One
  // stage-loading slot per sub-tile; the barrier that publishes stage st+1
  // closes sub-tile 2 of stage st, after every wave has read its last operands
  // of stage st (whose buffer stage st+2 reuses), so sub-tile 3 can already
  // read stage st+1.  Each slot stores its pieces a full stage after their
  // global loads.
#pragma unroll
  for (int j = 0; j < LOADS; ++j) fetch_piece(j, 0);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) stash_piece(j, 0);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) fetch_piece(j, 1);
  slot(0, 1);
  __syncthreads();
  bf16x8 bb[S];
  f32x16 acc[2][HT];
  float pe[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < S; ++s)
    bb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ktile + boff + s * 32));
  constexpr int EPR = 16 * HT / S;             // epilogue registers per step
  auto step = [&](auto C, auto SS, int st, bool live) {
    constexpr int c = decltype(C)::value, s = decltype(SS)::value;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      if constexpr (s == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c & 1][ht][r] = 0.f;
      }
      acc[c & 1][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][s], bb[s], acc[c & 1][ht], 0, 0, 0);
    }
    {
      const uint8_t* nt = ktile + ((c == 3 ? st + 1 : st) & 1) * STAGE;
      constexpr int nsub = (c + 1) & 3;
      bb[s] = __builtin_bit_cast(bf16x8,
                                 *reinterpret_cast<const u32x4*>(nt + boff + nsub * 32 * LB + s * 32));
    }
    if (c != 0 || live) {
      float& p = pe[(c + 3) & 3];
      if constexpr (s == 0) p = 0.f;
      static_for<EPR>([&](auto I) {
        constexpr int i = s * EPR + decltype(I)::value;
        p = fmac_rowbcast<i & 15>(p, W[i >> 4], relu(acc[(c + 1) & 1][i >> 4][i & 15]));
      });
    }
    constexpr int fs = 1, fc = S >= 8 ? 2 : 1;   // steps of the finish's store and count
    if constexpr (c == 3) {
      if constexpr (s == fs) fin_store(st * kStageKeys, pe[0], pe[1]);
      if constexpr (s == fc) fin_count(st * kStageKeys);
    }
    if constexpr (c == 1) {
      if (live) {
        if constexpr (s == fs) fin_store((st - 1) * kStageKeys + 64, pe[2], pe[3]);
        if constexpr (s == fc) fin_count((st - 1) * kStageKeys + 64);
      }
    }
    if constexpr (s == S - 2) slot((c + 1) & 3, c == 3 ? st + 2 : st + 1);
    if constexpr (c == 2 && s == S - 1) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int st = 0; st < n_stages; ++st) {
    const bool live = st > 0;
    static_for<S>([&](auto SS) { step(std::integral_constant<int, 0>{}, SS, st, live); });
    static_for<S>([&](auto SS) { step(std::integral_constant<int, 1>{}, SS, st, live); });
    static_for<S>([&](auto SS) { step(std::integral_constant<int, 2>{}, SS, st, live); });
    static_for<S>([&](auto SS) { step(std::integral_constant<int, 3>{}, SS, st, live); });
  }
  // drain: the last sub-tile's epilogue, then pair (2,3) of the last stage
  {
    pe[3] = weighted_relu_sum<HT>(acc[1], W, std::make_integer_sequence<int, 16>{});
    const int k_last = (n_stages - 1) * kStageKeys + 64;
    fin_store(k_last, pe[2], pe[3]);
    fin_count(k_last);
  }

  // this row's threshold: the bin (12-bit, or 11-bit with W32) holding its
  // k-th score
  if (SPLIT || pos < 0) return;
  int32_t* meta = a.rowmeta + (size_t)t * 4;
  if (pos + 1 <= a.top_k) {                    // short row: every key is selected
    if (lane == 0) { meta[0] = -1; meta[1] = 0; meta[2] = 0; }
    return;
  }
  // lane l owns bins [NB - PER (l + 1), NB - PER l), counted from the top
  constexpr int NB = W32 ? kPBins / 2 : kPBins;
  constexpr int PER = NB / 64;
  const int b_hi = NB - PER * lane;             // exclusive
  const int sh = W32 ? 0 : 16 * ((b_hi - 1) / (kPBins / 2));   // all in one half of the words
  const uint32_t cmask = W32 ? 0xFFFFFFFFu : 0xFFFFu;
  const int w0 = (b_hi - PER) & (kPBins / 2 - 1);
  uint32_t mine = 0;
  for (int i = 0; i < PER; ++i) mine += (hrow[w0 + i] >> sh) & cmask;
  uint32_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const uint32_t before = incl - mine, need = (uint32_t)a.top_k;
  if (before < need && incl >= need) {
    uint32_t accum = before;
    for (int b = b_hi - 1; b >= b_hi - PER; --b) {
      const uint32_t c = (hrow[b & (kPBins / 2 - 1)] >> sh) & cmask;
      if (accum + c >= need) {
        meta[0] = b;
        meta[1] = (int32_t)accum;
        meta[2] = (int32_t)c;
        break;
      }
      accum += c;
    }
  }
}

// (score key, index) pairs of one row, generated from the stored scores.
struct RowSource {
  const float* sc;
  uint32_t n;
  template <int NT, class F>
  DSA_DEVICE void for_each(F&& f) const {
    for (uint32_t u = threadIdx.x; u < n; u += NT) f(make_uint2(score_to_key(sc[u]), u));
  }
};

// FB: first-level bins of the rows' histograms (rowmeta).
template <int FB, int NT>
__global__ __launch_bounds__(NT) void k_prefill_select(PrefillArgs a) {
  constexpr int kFBShift = 32 - FB;
  extern __shared__ __align__(16) uint8_t smem[];
  uint2* list = reinterpret_cast<uint2*>(smem);                          // [kSelListCap]
  uint2* tie = list + kSelListCap;                                        // [64]
  uint32_t* hist = reinterpret_cast<uint32_t*>(tie + 64);                 // [1024]
  uint32_t* scratch = hist + 1024;                                        // [64]
  __shared__ uint32_t s_out, s_ln;
  const int t = (int)gridDim.x - 1 - (int)blockIdx.x;          // longest rows first
  int pos = -1;
  {
    const int seq = a.q_seq ? a.q_seq[t] : 0;
    const int p = a.q_pos[t];
    if (seq == 0 && p >= 0 && (int64_t)p < a.l_max) pos = p;
  }
  int32_t* out_i = a.out_idx + (size_t)t * a.top_k;
  float* out_s = a.out_score ? a.out_score + (size_t)t * a.top_k : nullptr;
  const uint32_t n = (uint32_t)(pos + 1);
  const uint32_t Kt = pos < 0 ? 0u : (n < (uint32_t)a.top_k ? n : (uint32_t)a.top_k);
  for (int i = Kt + threadIdx.x; i < a.top_k; i += NT) {
    out_i[i] = -1;
    if (out_s) out_s[i] = -__builtin_inff();
  }
  if (Kt == 0) return;
  const float* sc = a.scores + (size_t)t * (size_t)a.row_stride;
  if (n <= (uint32_t)a.top_k) {                // every key of a short row
    for (uint32_t u = threadIdx.x; u < n; u += NT) {
      out_i[u] = (int32_t)u;
      if (out_s) out_s[u] = key_to_score(score_to_key(sc[u]));
    }
    return;
  }
  constexpr int U = 4;
  const uint32_t n4 = (n + 3) / 4;
  auto load_iter = [&](uint32_t base, auto& v) {
    constexpr int UU = sizeof(v) / sizeof(v[0]);
#pragma unroll
    for (int j = 0; j < UU; ++j) {
      const uint32_t i4 = base + threadIdx.x + j * NT;
      v[j] = *reinterpret_cast<const f32x4*>(sc + 4 * (size_t)(i4 < n4 ? i4 : n4 - 1));
    }
    __builtin_amdgcn_sched_barrier(0);             // issue every load first
  };
  int bstar;
  uint32_t above, nb;
  {
    const int32_t* meta = a.rowmeta + (size_t)t * 4;
    bstar = meta[0];
    above = (uint32_t)meta[1];
    nb = (uint32_t)meta[2];
  }
  const bool fits = nb <= kSelListCap;
  if (threadIdx.x == 0) { s_out = 0; s_ln = 0; }
  if (!fits)                                    // second-digit histogram of the bin
    for (int i = threadIdx.x; i < 1024; i += NT) hist[i] = 0;
  __syncthreads();
  const Emitter em{out_i, out_s, &s_out, Kt};
  constexpr int kSub = kFBShift - 10;          // the 10 key bits below the first level
  const int lane = lane_id();
  // Passes over the row (16-byte loads, U per thread in flight): the loads are
  // unconditional (clamped to the row's last piece, masked afterwards) so that
  // all of them are in flight together.  Keys are formed as in the scoring
  // kernel's histogram (the stored scores are never -0.0).  Each thread flags
  // its 4U scores of an iteration in two masks (emitted now / kept in the LDS
  // list); one wave scan of the packed counts and one LDS atomic per wave
  // reserve consecutive slots, and each lane writes its flagged scores there.
  auto append = [&](uint32_t base, const f32x4 (&v)[U], uint32_t take_m, uint32_t keep_m,
                    uint32_t kcap) {
    const uint32_t packed = (uint32_t)__builtin_popcount(take_m) |
                            ((uint32_t)__builtin_popcount(keep_m) << 16);
    const uint32_t incl = wave_incl_scan(packed);
    const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
    if (tot == 0) return;                          // wave-uniform
    uint32_t bt = 0, bk = 0;
    if (lane == 63) {
      if (tot & 0xFFFFu) bt = atomicAdd(&s_out, tot & 0xFFFFu);
      if (tot >> 16) bk = atomicAdd(&s_ln, tot >> 16);
    }
    const uint32_t excl = incl - packed;
    uint32_t o = __builtin_amdgcn_readlane(bt, 63) + (excl & 0xFFFFu);
    uint32_t l = __builtin_amdgcn_readlane(bk, 63) + (excl >> 16);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t u0 = 4 * (base + threadIdx.x + j * NT);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bit = 4 * j + e;
        if ((take_m >> bit) & 1u) {
          if (o < Kt) {
            out_i[o] = (int32_t)(u0 + e);
            if (out_s) out_s[o] = v[j][e];
          }
          ++o;
        }
        if ((keep_m >> bit) & 1u) {
          if (l < kcap) list[l] = make_uint2(fast_key(v[j][e]), u0 + e);
          ++l;
        }
      }
    }
  };
  // first pass: emit every score above the bin, collect the bin (or, when it
  // overflows the list, count its next 10-bit digit).  Iterations wholly
  // inside the row skip the end-of-row masks; the path is fixed per row.
  const uint32_t n_whole = n / (4 * NT * U) * (NT * U);   // in 16-byte pieces
  auto pass1_iter = [&](uint32_t base, auto MASKED, auto FITS) {
    constexpr bool kMasked = decltype(MASKED)::value, kFits = decltype(FITS)::value;
    f32x4 v[U];
    load_iter(base, v);
    uint32_t take_m = 0, keep_m = 0;
#pragma unroll
    for (int j = 0; j < U; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = 4 * (base + threadIdx.x + j * NT) + e;
        const bool ok = !kMasked || u < n;
        const uint32_t key = fast_key(v[j][e]);
        const int b = (int)(key >> kFBShift);
        take_m |= (uint32_t)(ok && b > bstar) << (4 * j + e);
        if constexpr (kFits) keep_m |= (uint32_t)(ok && b == bstar) << (4 * j + e);
        else if (ok && b == bstar) atomicAdd(&hist[(key >> kSub) & 1023u], 1u);
      }
    }
    append(base, v, take_m, keep_m, kSelListCap);
  };
  auto pass1 = [&](auto FITS) {
    uint32_t base = 0;
    for (; base < n_whole; base += NT * U) pass1_iter(base, std::false_type{}, FITS);
    for (; base < n4; base += NT * U) pass1_iter(base, std::true_type{}, FITS);
  };
  if (fits) pass1(std::true_type{});
  else pass1(std::false_type{});
  __syncthreads();
  const uint32_t need = Kt - above;
  if (fits) {
    const uint32_t nl = s_ln < nb ? s_ln : nb;
    finish_bin<NT, FB>(list, nl, need, bstar, em, hist, scratch, tie);
    return;
  }
  // The bin overflowed the list: its second-digit histogram (counted in the
  // first pass) gives the sub-bin d2 of the k-th entry; one more pass over the
  // row emits the bin's entries above d2 and collects d2 itself.
  uint32_t above2;
  const int d2 = block_find_threshold<NT>(hist, 1024, need, scratch, &above2);
  const uint32_t nd2 = hist[d2];
  const uint32_t need2 = need - above2;
  if (threadIdx.x == 0) s_ln = 0;
  __syncthreads();
  const bool fits2 = nd2 <= kSelListCap;
  for (uint32_t base = 0; base < n4; base += NT * U) {
    f32x4 v[U];
    load_iter(base, v);
    uint32_t take_m = 0, keep_m = 0;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t i4 = base + threadIdx.x + j * NT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = 4 * i4 + e;
        const bool ok = i4 < n4 && u < n;
        const uint32_t key = ok ? fast_key(v[j][e]) : 0u;
        const bool in_bin = ok && (int)(key >> kFBShift) == bstar;
        const int sub = (int)((key >> kSub) & 1023u);
        take_m |= (uint32_t)(in_bin && sub > d2) << (4 * j + e);
        if (fits2) keep_m |= (uint32_t)(in_bin && sub == d2) << (4 * j + e);
      }
    }
    append(base, v, take_m, keep_m, kSelListCap);
  }
  __syncthreads();
  const uint64_t prefix = ((uint64_t)bstar << (64 - FB)) | ((uint64_t)d2 << (64 - FB - 10));
  const uint64_t mask = (uint64_t)((1u << (FB + 10)) - 1u) << (64 - FB - 10);
  if (fits2) {
    const uint32_t nl = s_ln < nd2 ? s_ln : nd2;
    PairSource src{list, nl};
    radix_finish<NT>(src, prefix, mask, 64 - FB - 10, need2, nl, em, hist, scratch);
  } else {
    RowSource src{sc, n};
    radix_finish<NT>(src, prefix, mask, 64 - FB - 10, need2, nd2, em, hist, scratch);
  }
}

// ---- select of key-split rows: every row in parts of kRowPartKeys scores,
// one 256-thread workgroup per (part, row).
constexpr int kRT = 256;

DSA_DEVICE int row_pos(const PrefillArgs& a, int t) {   // the row's last key, or -1
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int p = a.q_pos[t];
  return (seq == 0 && p >= 0 && (int64_t)p < a.l_max) ? p : -1;
}

// A part's scores (16-byte loads, all issued first; the part starts on a
// multiple of 4 and the row stride covers the last piece).
template <int U>
DSA_DEVICE void load_part(const float* sc, uint32_t u0, uint32_t u1, f32x4 (&v)[U]) {
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const uint32_t i4 = (u0 >> 2) + threadIdx.x + j * kRT;
    v[j] = 4 * i4 < u1 ? *reinterpret_cast<const f32x4*>(sc + 4 * (size_t)i4) : f32x4{0, 0, 0, 0};
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Count: each part of a row longer than top_k stores its 12-bit histogram
// (16-bit counts, plain stores: the next kernel reads them).
__global__ __launch_bounds__(kRT) void k_rows_count(PrefillArgs a) {
  __shared__ uint32_t hist[kBins];
  const int t = (int)blockIdx.y, p = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int pos = row_pos(a, t);
  const uint32_t n = (uint32_t)pos + 1u;
  if (pos < 0 || n <= (uint32_t)a.top_k) return;
  const uint32_t parts = (n + kRowPartKeys - 1) / kRowPartKeys;
  if ((uint32_t)p >= parts) return;
  for (int i = tid; i < kBins; i += kRT) hist[i] = 0u;
  __syncthreads();
  const float* sc = a.scores + (size_t)t * (size_t)a.row_stride;
  const uint32_t u0 = (uint32_t)p * kRowPartKeys, u1 = min(n, u0 + kRowPartKeys);
  constexpr int U = kRowPartKeys / 4 / kRT;
  f32x4 v[U];
  load_part<U>(sc, u0, u1, v);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const uint32_t i4 = (u0 >> 2) + tid + j * kRT;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * i4 + e < u1) atomicAdd(&hist[fast_key(v[j][e]) >> kBinShift], 1u);
  }
  __syncthreads();
  // thread i: bins 16 i .. 16 i + 15, as 8 words of two 16-bit counts
  static_assert(kBins == 16 * kRT && kRowPartKeys < 65536, "16 bins per thread, 16-bit counts");
  uint32_t* ph = a.parthist + ((size_t)t * a.row_parts + p) * (kBins / 2) + 8 * tid;
  u32x4 w0, w1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0[i] = hist[16 * tid + 2 * i] | (hist[16 * tid + 2 * i + 1] << 16);
    w1[i] = hist[16 * tid + 8 + 2 * i] | (hist[16 * tid + 8 + 2 * i + 1] << 16);
  }
  *reinterpret_cast<u32x4*>(ph) = w0;
  *reinterpret_cast<u32x4*>(ph + 4) = w1;
}

// Threshold: one workgroup per row adds its parts' histograms (every load of
// up to 16 parts in flight at once) and finds the bin of the row's k-th best
// key and the count above it; it also clears the emission's counters.  Rows
// of at most top_k keys keep every key.
constexpr int kRowT = 1024;                     // threads of the per-row kernels
__global__ __launch_bounds__(kRowT) void k_rows_threshold(PrefillArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scratch[64];
  const int t = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int pos = row_pos(a, t);
  if (pos < 0) return;                          // (the finish pads the row)
  const uint32_t n = (uint32_t)pos + 1u;
  uint32_t* rc = a.rowctl + (size_t)t * kRowCtlWords;
  if (n <= (uint32_t)a.top_k) {
    if (tid == 0) {
      rc[RH_EMIT] = 0u;
      rc[RH_TIES] = 0u;
      rc[RH_BSTAR] = 0xFFFFFFFFu;               // every bin is above
      rc[RH_ABOVE] = n;
      rc[RH_NB] = 0u;
    }
    return;
  }
  const uint32_t parts = (n + kRowPartKeys - 1) / kRowPartKeys;
  // thread i: bins 4 i .. 4 i + 3, one word pair of 16-bit counts per part
  static_assert(kBins == 4 * kRowT, "4 bins per thread");
  const uint2* ph0 = reinterpret_cast<const uint2*>(a.parthist + (size_t)t * a.row_parts * (kBins / 2)) + tid;
  uint32_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
  for (uint32_t q0 = 0; q0 < parts; q0 += 16) {
    uint2 x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
      x[q] = q0 + q < parts ? ph0[(size_t)(q0 + q) * (kBins / 4)] : make_uint2(0u, 0u);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      s0 += x[q].x & 0xFFFFu;
      s1 += x[q].x >> 16;
      s2 += x[q].y & 0xFFFFu;
      s3 += x[q].y >> 16;
    }
  }
  hist[4 * tid] = s0;
  hist[4 * tid + 1] = s1;
  hist[4 * tid + 2] = s2;
  hist[4 * tid + 3] = s3;
  __syncthreads();
  uint32_t above;
  const int bstar = block_find_threshold<kRowT>(hist, kBins, (uint32_t)a.top_k, scratch, &above);
  if (tid == 0) {
    rc[RH_EMIT] = 0u;
    rc[RH_TIES] = 0u;
    rc[RH_BSTAR] = (uint32_t)bstar;
    rc[RH_ABOVE] = above;
    rc[RH_NB] = hist[bstar];
  }
}

// Emission: every part writes its keys above the threshold bin to the output
// and those in the bin to the row's tie buffer (up to its capacity), at slots
// reserved with one atomic per wave.
__global__ __launch_bounds__(kRT) void k_rows_emit(PrefillArgs a) {
  const int t = (int)blockIdx.y, p = (int)blockIdx.x, tid = (int)threadIdx.x, lane = lane_id();
  const int pos = row_pos(a, t);
  if (pos < 0) return;
  const uint32_t n = (uint32_t)pos + 1u;
  const uint32_t parts = (n + kRowPartKeys - 1) / kRowPartKeys;
  if ((uint32_t)p >= parts) return;
  const uint32_t Kt = n < (uint32_t)a.top_k ? n : (uint32_t)a.top_k;
  uint32_t* rc = a.rowctl + (size_t)t * kRowCtlWords;
  const int bstar = (int)rc[RH_BSTAR];          // -1: every key is selected
  int32_t* out_i = a.out_idx + (size_t)t * a.top_k;
  float* out_s = a.out_score ? a.out_score + (size_t)t * a.top_k : nullptr;
  const float* sc = a.scores + (size_t)t * (size_t)a.row_stride;
  uint2* ties = a.ties + (size_t)t * kRowTieCap;
  const uint32_t u0 = (uint32_t)p * kRowPartKeys, u1 = min(n, u0 + kRowPartKeys);
  constexpr int U = kRowPartKeys / 4 / kRT;
  f32x4 v[U];
  load_part<U>(sc, u0, u1, v);
  uint32_t take_m = 0, tie_m = 0;               // bit 4 j + e: key taken / in the bin
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const uint32_t i4 = (u0 >> 2) + tid + j * kRT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = 4 * i4 + e < u1;
      const int b = (int)(fast_key(v[j][e]) >> kBinShift);
      take_m |= (uint32_t)(ok && b > bstar) << (4 * j + e);
      tie_m |= (uint32_t)(ok && b == bstar) << (4 * j + e);
    }
  }
  const uint32_t packed = (uint32_t)__builtin_popcount(take_m) |
                          ((uint32_t)__builtin_popcount(tie_m) << 16);
  const uint32_t incl = wave_incl_scan(packed);
  const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
  if (tot == 0) return;                         // wave-uniform
  uint32_t bt = 0, bk = 0;
  if (lane == 63) {
    if (tot & 0xFFFFu) bt = atomicAdd(&rc[RH_EMIT], tot & 0xFFFFu);
    if (tot >> 16) bk = atomicAdd(&rc[RH_TIES], tot >> 16);
  }
  const uint32_t excl = incl - packed;
  uint32_t o = __builtin_amdgcn_readlane(bt, 63) + (excl & 0xFFFFu);
  uint32_t l = __builtin_amdgcn_readlane(bk, 63) + (excl >> 16);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const uint32_t u = 4 * ((u0 >> 2) + tid + j * kRT);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bit = 4 * j + e;
      if ((take_m >> bit) & 1u) {
        if (o < Kt) {
          out_i[o] = (int32_t)(u + e);
          if (out_s) out_s[o] = v[j][e];
        }
        ++o;
      }
      if ((tie_m >> bit) & 1u) {
        if (l < (uint32_t)kRowTieCap) ties[l] = make_uint2(fast_key(v[j][e]), u + e);
        ++l;
      }
    }
  }
}

// Finish: one workgroup per row pads the row past its key count and takes the
// best entries of the threshold bin: from the tie buffer when the bin fit in
// it, else with a radix select over the row's stored scores.
__global__ __launch_bounds__(kRowT) void k_rows_finish(PrefillArgs a) {
  __shared__ uint2 list[kRowTieCap];
  __shared__ uint2 tie[64];
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t scratch[64];
  __shared__ uint32_t s_out;
  const int t = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int pos = row_pos(a, t);
  int32_t* out_i = a.out_idx + (size_t)t * a.top_k;
  float* out_s = a.out_score ? a.out_score + (size_t)t * a.top_k : nullptr;
  const uint32_t n = (uint32_t)pos + 1u;
  const uint32_t Kt = pos < 0 ? 0u : (n < (uint32_t)a.top_k ? n : (uint32_t)a.top_k);
  for (uint32_t i = Kt + tid; i < (uint32_t)a.top_k; i += kRowT) {
    out_i[i] = -1;
    if (out_s) out_s[i] = -__builtin_inff();
  }
  if (Kt == 0) return;
  const uint32_t* rc = a.rowctl + (size_t)t * kRowCtlWords;
  const int bstar = (int)rc[RH_BSTAR];
  const uint32_t above = rc[RH_ABOVE], nb = rc[RH_NB];
  const uint32_t need = Kt - above;             // entries of the threshold bin to take
  if (need == 0) return;
  if (tid == 0) s_out = above;
  __syncthreads();
  const Emitter em{out_i, out_s, &s_out, Kt};
  if (nb <= (uint32_t)kRowTieCap) {
    const uint2* ties = a.ties + (size_t)t * kRowTieCap;
    for (uint32_t i = tid; i < nb; i += kRowT) list[i] = ties[i];
    __syncthreads();
    finish_bin<kRowT, kBinBits>(list, nb, need, bstar, em, hist, scratch, tie);
  } else {
    const float* sc = a.scores + (size_t)t * (size_t)a.row_stride;
    const uint64_t prefix = (uint64_t)bstar << (64 - kBinBits);
    const uint64_t mask = (uint64_t)(kBins - 1) << (64 - kBinBits);
    radix_finish<kRowT>(RowSource{sc, n}, prefix, mask, 64 - kBinBits, need, nb, em, hist, scratch);
  }
}

template <int HT, int D, bool W32, bool SPLIT>
hipError_t launch_score_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr int ROWS = kRows;
  const size_t lds = prefill_lds_bytes<D, ROWS, SPLIT>();
  static_assert(prefill_lds_bytes<D, ROWS>() <= 160 * 1024, "LDS");
  auto k = k_prefill_score<HT, D, ROWS, W32, SPLIT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = (a.nq + ROWS - 1) / ROWS;
  const int chunks = SPLIT ? (int)((a.l_max + a.key_chunk - 1) / a.key_chunk) : 1;
  hipLaunchKernelGGL(k, dim3(groups, chunks), dim3(64 * ROWS), lds, stream, a);
  return hipGetLastError();
}

template <int HT, int D>
hipError_t launch_score_hd(const PrefillArgs& a, hipStream_t stream) {
  if (a.key_chunk > 0) return launch_score_t<HT, D, false, true>(a, stream);
  if (a.bin_bits == 11) return launch_score_t<HT, D, true, false>(a, stream);
  return launch_score_t<HT, D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_prefill_score(const PrefillArgs& a, hipStream_t stream) {
  if (a.nq <= 0) return hipSuccess;
  // every key of a row's last stage is stored: rows span whole stages
  if (a.row_stride % kStageKeys != 0 || a.row_stride < a.l_max || !a.spare_row) return hipErrorInvalidValue;
  // 16-bit counters hold rows of up to 65535 keys; 32-bit counters (11-bit
  // bins) any row; the row offsets are 32-bit byte offsets; split key chunks
  // are whole stages (and are counted by the select kernel in 12-bit bins)
  if (a.l_max >= (int64_t)1 << 30 || (a.bin_bits == 12 && a.l_max > 65535 && a.key_chunk == 0) ||
      (a.bin_bits != 12 && a.bin_bits != 11) || a.key_chunk < 0 || a.key_chunk % kStageKeys ||
      (a.key_chunk > 0 && a.bin_bits != 12))
    return hipErrorInvalidValue;
  if (a.head_dim == 128)
    return a.n_heads <= 32 ? launch_score_hd<1, 128>(a, stream) : launch_score_hd<2, 128>(a, stream);
  if (a.head_dim == 64)
    return a.n_heads <= 32 ? launch_score_hd<1, 64>(a, stream) : launch_score_hd<2, 64>(a, stream);
  return hipErrorInvalidValue;
}

template <int FB>
hipError_t launch_select_t(const PrefillArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)kSelListCap * 8 + 64 * 8 + (1024 + 64) * 4;
  constexpr int NT = kST;
  auto k = k_prefill_select<FB, NT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.nq), dim3(NT), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t stream) {
  if (a.nq <= 0) return hipSuccess;
  if (a.key_chunk > 0) {
    // (parts along x, rows along y: at most 65535 rows)
    const int64_t parts = (a.l_max + kRowPartKeys - 1) / kRowPartKeys;
    if (a.bin_bits != 12 || !a.rowctl || !a.parthist || !a.ties || a.row_parts < parts ||
        a.nq > 65535 || parts > 65535)
      return hipErrorInvalidValue;
    const dim3 grid((unsigned)parts, (unsigned)a.nq);
    hipLaunchKernelGGL(k_rows_count, grid, dim3(kRT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rows_threshold, dim3(a.nq), dim3(kRowT), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_rows_emit, grid, dim3(kRT), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_rows_finish, dim3(a.nq), dim3(kRowT), 0, stream, a);
    return hipGetLastError();
  }
  if (a.bin_bits == 12) return launch_select_t<12>(a, stream);
  if (a.bin_bits == 11) return launch_select_t<11>(a, stream);
  if (a.bin_bits == 10) return launch_select_t<10>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
