// MISA's routed token pass on the prefill shape: many query rows of one
// sequence, each scored with only its h <= 8 routed heads (MISA summary,
// "method" step 2: the token pass runs with the routed head subset), then the
// exact per-row top-k by the prefill select kernel.
//
// The rows share the key cache, so a wave packs four rows x eight head slots
// into the 32 rows of one v_mfma_f32_32x32x16_bf16 tile (A operand); 32 rows
// per workgroup share each 128-key LDS stage.  With the head count cut from 64
// to 8 per row, the MFMA work and the fused ReLU-weighted epilogue per (row,
// key) shrink eightfold against the dense prefill kernel.  The accumulator
// register r of a lane holds MFMA row 8*(r/4) + 4*(lane/32) + r%4, i.e. row
// slot r/4 of the wave, so registers 4g .. 4g+3 sum into row g's partial, and
// one lane-half swap of two sub-tiles' partials gives row g's scores of 64
// consecutive keys in one register.
// Per-row histograms are 10-bit with 16-bit counters, two per word (bin b in
// word b % 512), 2 KiB per row, so that 32 rows' fit in LDS beside the two
// stages.  With SPLIT (too few row groups to fill the chip) the keys are split
// into chunks as well, one workgroup per (row group, chunk), with no
// histograms: the select kernel counts the stored rows itself.
#include "dsa_internal.h"
#include "dsa_common.h"

namespace dsa {

namespace {

constexpr int kStageKeys = 128;
constexpr int kWaves = 8;
constexpr int kPer = 4;                       // query rows per wave
constexpr int kRowsWg = kWaves * kPer;        // 32 rows per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRBinBits = 10;
constexpr int kRBins = 1 << kRBinBits;
constexpr int kRBinShift = 32 - kRBinBits;

template <int D, bool SPLIT = false>
constexpr size_t routed_lds_bytes() {
  return 2 * (size_t)kStageKeys * (D * 2 + 16) + (SPLIT ? 0 : (size_t)kRowsWg * (kRBins / 2) * 4);
}

// per-row partial sums of one sub-tile: p[g] = sum over registers 4g..4g+3 of
// w * max(0, acc) (weights by row broadcast, see fmac_rowbcast); registers R0 ..
// R0+N-1 at a time, so that the epilogue can be spread over MFMA steps
template <int R>
DSA_DEVICE void row_term(f32x4& p, float W, float x) {
  if constexpr ((R & 3) == 0) p[R >> 2] = fmul_rowbcast<R>(W, x);   // first term of row R/4
  else p[R >> 2] = fmac_rowbcast<R>(p[R >> 2], W, x);
}

template <int R0, int... R>
DSA_DEVICE void epi_seq(f32x4& p, const f32x16& acc, float W, std::integer_sequence<int, R...>) {
  (row_term<R0 + R>(p, W, relu(acc[R0 + R])), ...);
}

template <int R0, int N>
DSA_DEVICE void epi_regs(f32x4& p, const f32x16& acc, float W) {
  epi_seq<R0>(p, acc, W, std::make_integer_sequence<int, N>{});
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void k_prefill_routed_score(PrefillArgs a) {
  constexpr int S = D / 16;
  constexpr int RB = D * 2;
  constexpr int NC = RB / 16;
  constexpr int LB = RB + 16;
  constexpr int STAGE = kStageKeys * LB;
  constexpr int PIECES = kStageKeys * NC;
  constexpr int LOADS = PIECES / kThreads;
  static_assert(PIECES % kThreads == 0, "every thread stores whole pieces");
  constexpr int PER_SLOT = (LOADS + 3) / 4;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* ktile = smem;                                           // [2][STAGE]
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + 2 * STAGE);  // [32 rows][kRBins / 2]
  __shared__ int s_maxpos;

  const int wv = wave_id(), lane = lane_id();
  const int grp = (int)gridDim.x - 1 - (int)blockIdx.x;            // longest rows first
  const int t0 = grp * kRowsWg + wv * kPer;                         // this wave's first row
  int pos[kPer];
  int wave_max = -1;
#pragma unroll
  for (int g = 0; g < kPer; ++g) {
    pos[g] = -1;
    const int t = t0 + g;
    if (t < a.nq) {
      const int seq = a.q_seq ? a.q_seq[t] : 0;
      const int p = a.q_pos[t];
      if (seq == 0 && p >= 0 && (int64_t)p < a.l_max) pos[g] = p;
    }
    wave_max = pos[g] > wave_max ? pos[g] : wave_max;
  }
  if constexpr (!SPLIT)
    for (int i = threadIdx.x; i < kRowsWg * (kRBins / 2); i += kThreads) hist[i] = 0u;
  if (threadIdx.x == 0) s_maxpos = -1;
  __syncthreads();
  if (lane == 0) atomicMax(&s_maxpos, wave_max);
  __syncthreads();
  const int maxpos = __builtin_amdgcn_readfirstlane(s_maxpos);
  if (maxpos < 0) return;
  // keys [kb, ke_last] of this workgroup (SPLIT: one chunk of whole stages)
  const int kb = SPLIT ? (int)blockIdx.y * a.key_chunk : 0;
  if (kb > maxpos) return;
  const int ke_last = SPLIT ? min(kb + a.key_chunk - 1, maxpos) : maxpos;
  const int n_stages = (ke_last - kb) / kStageKeys + 1;
  auto pos_of = [&](int g) {                 // pos[g] for a per-lane g
    int p = pos[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) p = g == i ? pos[i] : p;
    return p;
  };

  // A operand: MFMA row m = lane % 32 is head slot j = m % 8 of row g = m / 8
  const int m = lane & 31, h = lane >> 5;
  bf16x8 qa[S];
  {
    const int g = m >> 3, j = m & 7, t = t0 + g;
    const bool ok = pos_of(g) >= 0 && j < a.h_use;
    const int head = ok ? a.heads[(size_t)t * a.heads_stride + j] : 0;
    const uint16_t* src = a.q + ((size_t)(ok ? t : 0) * a.n_heads + head) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < S; ++s) qa[s] = ok ? load_bf16x8(src + 16 * s) : zero_bf16x8();
  }
  // weights: lane 16*q + r holds the weight of MFMA row 8*(r/4) + 4*(q/2) + r%4
  // (row r/4, head slot 4*(q/2) + r%4), ready for the row broadcast
  float W;
  {
    const int r = lane & 15, q4 = lane >> 4;
    const int g = r >> 2, j = 4 * (q4 >> 1) + (r & 3), t = t0 + g;
    const bool ok = pos_of(g) >= 0 && j < a.h_use;
    W = ok ? a.w[(size_t)t * a.n_heads + a.heads[(size_t)t * a.heads_stride + j]] : 0.f;
  }
  const uint32_t boff = (uint32_t)(m * LB + h * 16);

  // stage loading (as in the dense prefill kernel): four slots per stage
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.keys);
  u32x4 pre[LOADS];
  // (a wave-uniform stage base plus a 32-bit lane offset; keys clamp to maxpos)
  auto fetch_piece = [&](int j, int st) {
    const int p = threadIdx.x + j * kThreads;
    const int sk = min(kb + st * kStageKeys, ke_last);
    const int key = min(p / NC, ke_last - sk);
    const uint8_t* sbase = kbase + (size_t)sk * RB;
    pre[j] = *reinterpret_cast<const u32x4*>(sbase + (uint32_t)(key * RB + (p % NC) * 16));
  };
  auto stash_piece = [&](int j, int buf) {
    const int p = threadIdx.x + j * kThreads;
    const int key = p / NC, pc = p % NC;
    *reinterpret_cast<u32x4*>(ktile + buf * STAGE + key * LB + pc * 16) = pre[j];
  };
  auto slot = [&](int q, int st) {
#pragma unroll
    for (int j = q * PER_SLOT; j < (q + 1) * PER_SLOT && j < LOADS; ++j) {
      stash_piece(j, st & 1);
      fetch_piece(j, st + 1);
    }
  };
  auto load_b = [&](bf16x8 (&b)[S], const uint8_t* tile, int sub) {
#pragma unroll
    for (int s = 0; s < S; ++s)
      b[s] = __builtin_bit_cast(bf16x8,
                                *reinterpret_cast<const u32x4*>(tile + boff + sub * 32 * LB + s * 32));
  };

  // Finish of a pair of sub-tiles (keys key0 .. key0+63): for row g of the
  // wave, one lane-half swap of the two sub-tiles' partials puts key key0 + l
  // in lane l, so one register holds row g's 64 scores.  Branch-free: every
  // lane stores (score rows are padded to whole stages, rows that are not
  // scored write a spare row) and keys past the row's position add 0 to the
  // histogram.  The +0.0 turns a -0.0 sum (all terms -0.0) into +0.0, so that
  // score keys need no -0.0 fold.
  const size_t rs = (size_t)a.row_stride;
  const int t0u = __builtin_amdgcn_readfirstlane(t0);
  uint8_t* srow[kPer];
#pragma unroll
  for (int g = 0; g < kPer; ++g) {
    pos[g] = __builtin_amdgcn_readfirstlane(pos[g]);
    srow[g] = reinterpret_cast<uint8_t*>(pos[g] >= 0 ? a.scores + (size_t)(t0u + g) * rs : a.spare_row);
  }
  uint32_t* hwave = hist + wv * kPer * (kRBins / 2);
  float fin_sc[2];
  auto fin_store = [&](int i, int g, int key0, const f32x4& pa, const f32x4& pb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa[g]), __float_as_uint(pb[g]),
                                                     false, false);
    fin_sc[i] = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) + 0.0f;
    *reinterpret_cast<float*>(srow[g] + (uint32_t)(kb + key0 + lane) * 4u) = fin_sc[i];
  };
  // bin b counts in word b % 512: low half for b < 512 (negative scores, key
  // bit 31 clear), high half otherwise
  auto fin_count = [&](int i, int g, int key0) {
    if constexpr (SPLIT) return;                // (the select kernel counts the rows)
    const float sc = fin_sc[i];
    const uint32_t word = (fast_key(sc) >> kRBinShift) & (kRBins / 2 - 1);
    const uint32_t inc = key0 + lane <= pos[g] ? ((int32_t)__float_as_uint(sc) < 0 ? 1u : 0x10000u) : 0u;
    atomicAdd(hwave + g * (kRBins / 2) + word, inc);
  };

  // Software pipeline over 32-key sub-tiles c = 0..3 of each 128-key stage.
  // The section of sub-tile c issues its S MFMAs (B operands read one section
  // earlier), one step each, and, spread over the steps: the B reads of the
  // next sub-tile, the ReLU-weighted epilogue of the previous sub-tile into
  // P[c-1], two rows' finish of an earlier pair and one stage-loading slot.
  // Pair (0,1) of a stage is finished in its section 3 (rows 0, 1) and the
  // next stage's section 0 (rows 2, 3); pair (2,3) in the next stage's
  // sections 1 and 2.  The stage barrier closes section 2.  Steps are fenced
  // so that the interleave is kept as written.
#pragma unroll
  for (int j = 0; j < LOADS; ++j) fetch_piece(j, 0);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) stash_piece(j, 0);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) fetch_piece(j, 1);
  slot(0, 1);
  __syncthreads();
  bf16x8 bb[2][S];
  f32x16 acc[2];
  f32x4 P[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) P[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  load_b(bb[0], ktile, 0);
  constexpr int EPR = 16 / S;                 // epilogue registers per step
  // step s of section c in stage st (c, s compile-time; st runtime)
  auto step = [&](auto C, auto SS, int st, bool live) {
    constexpr int c = decltype(C)::value, s = decltype(SS)::value;
    const uint8_t* tile = ktile + (st & 1) * STAGE;
    f32x16& ac = acc[c & 1];
    if constexpr (s == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) ac[r] = 0.f;
    }
    ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], bb[c & 1][s], ac, 0, 0, 0);
    // B of the next sub-tile
    {
      const uint8_t* nt = c == 3 ? ktile + ((st + 1) & 1) * STAGE : tile;
      constexpr int nsub = (c + 1) & 3;
      bb[(c + 1) & 1][s] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(nt + boff + nsub * 32 * LB + s * 32));
    }
    // epilogue of the previous sub-tile (c - 1, or sub-tile 3 of the previous stage)
    if (c != 0 || live) {
      const f32x16& ap = acc[(c + 1) & 1];
      f32x4& pp = P[(c + 3) & 3];
      epi_regs<s * EPR, EPR>(pp, ap, W);
    }
    // finish: two rows of a pair
    // (store and count of a row one step apart when there are 8 steps)
    constexpr int fa = 1, fb = S >= 8 ? 4 : 2, lag = S >= 8 ? 1 : 0;
    constexpr bool prev_pair = c != 3;                          // pair of the previous stage
    const int pk0 = c == 0 ? (st - 1) * kStageKeys : c == 3 ? st * kStageKeys : (st - 1) * kStageKeys + 64;
    constexpr int pi = (c == 0 || c == 3) ? 0 : 2;              // first sub-tile of the pair
    constexpr int g0 = (c == 0 || c == 2) ? 2 : 0;              // first row
    if (!prev_pair || live) {
      if constexpr (s == fa) fin_store(0, g0, pk0, P[pi], P[pi + 1]);
      if constexpr (s == fa + lag) fin_count(0, g0, pk0);
      if constexpr (s == fb) fin_store(1, g0 + 1, pk0, P[pi], P[pi + 1]);
      if constexpr (s == fb + lag) fin_count(1, g0 + 1, pk0);
    }
    if constexpr (s == S - 2) slot((c + 1) & 3, c == 3 ? st + 2 : st + 1);
    if constexpr (c == 2 && s == S - 1) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto section = [&](auto C, int st, bool live) {
    static_for<S>([&](auto SS) { step(C, SS, st, live); });
  };
  for (int st = 0; st < n_stages; ++st) {
    const bool live = st > 0;
    section(std::integral_constant<int, 0>{}, st, live);
    section(std::integral_constant<int, 1>{}, st, live);
    section(std::integral_constant<int, 2>{}, st, live);
    section(std::integral_constant<int, 3>{}, st, live);
  }
  // drain: epilogue of the last sub-tile, rows 2, 3 of pair (0,1), pair (2,3)
  {
    const int k0 = (n_stages - 1) * kStageKeys;
    epi_regs<0, 16>(P[3], acc[1], W);
    fin_store(0, 2, k0, P[0], P[1]); fin_count(0, 2, k0);
    fin_store(1, 3, k0, P[0], P[1]); fin_count(1, 3, k0);
#pragma unroll
    for (int g = 0; g < kPer; ++g) { fin_store(0, g, k0 + 64, P[2], P[3]); fin_count(0, g, k0 + 64); }
  }
  __syncthreads();

  // each row's threshold: the 10-bit bin holding its k-th score
  if constexpr (SPLIT) return;
  constexpr int PERB = kRBins / 64;          // bins per lane
#pragma unroll
  for (int g = 0; g < kPer; ++g) {
    const int p = pos[g];
    if (p < 0) continue;
    int32_t* meta = a.rowmeta + (size_t)(t0 + g) * 4;
    if (p + 1 <= a.top_k) {
      if (lane == 0) { meta[0] = -1; meta[1] = 0; meta[2] = 0; }
      continue;
    }
    const uint32_t* hrow = hist + (wv * kPer + g) * (kRBins / 2);
    const int b_hi = kRBins - PERB * lane;   // lane owns bins [b_hi - PERB, b_hi)
    const int sh = 16 * ((b_hi - 1) / (kRBins / 2));   // all in one half of the words
    const int w0 = (b_hi - PERB) & (kRBins / 2 - 1);
    uint32_t mine = 0;
    for (int i = 0; i < PERB; ++i) mine += (hrow[w0 + i] >> sh) & 0xFFFFu;
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const uint32_t before = incl - mine, need = (uint32_t)a.top_k;
    if (before < need && incl >= need) {
      uint32_t accum = before;
      for (int b = b_hi - 1; b >= b_hi - PERB; --b) {
        const uint32_t c = (hrow[b & (kRBins / 2 - 1)] >> sh) & 0xFFFFu;
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
}

template <int D, bool SPLIT>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr size_t lds = routed_lds_bytes<D, SPLIT>();
  static_assert(routed_lds_bytes<D>() <= 160 * 1024, "LDS");
  auto k = k_prefill_routed_score<D, SPLIT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = (a.nq + kRowsWg - 1) / kRowsWg;
  const int chunks = SPLIT ? (int)((a.l_max + a.key_chunk - 1) / a.key_chunk) : 1;
  hipLaunchKernelGGL(k, dim3(groups, chunks), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_routed_score(const PrefillArgs& a, hipStream_t stream) {
  if (a.nq <= 0) return hipSuccess;
  // (16-bit row histograms without a key split; with one the select counts
  // the rows in 12-bit bins)
  const bool split = a.key_chunk > 0;
  if (a.h_use < 1 || a.h_use > kRoutedMaxHeads || a.key_chunk < 0 || a.key_chunk % kStageKeys ||
      a.bin_bits != (split ? 12 : kRBinBits) || (!split && a.l_max > 65535) ||
      a.l_max >= (int64_t)1 << 30)
    return hipErrorInvalidValue;
  // every key of a row's last stage is stored: rows span whole stages
  if (a.row_stride % kStageKeys != 0 || a.row_stride < a.l_max || !a.spare_row) return hipErrorInvalidValue;
  if (a.head_dim == 128) return split ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
  if (a.head_dim == 64) return split ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
