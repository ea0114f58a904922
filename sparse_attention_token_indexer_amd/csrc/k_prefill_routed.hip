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
// Per-row histograms are 10-bit (u16 pairs, 2 KiB per row) so that 32 rows'
// fit in LDS beside the two stages.
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

template <int D>
constexpr size_t routed_lds_bytes() {
  return 2 * (size_t)kStageKeys * (D * 2 + 16) + (size_t)kRowsWg * (kRBins / 2) * 4;
}

// per-row partial sums of one sub-tile: p[g] = sum over registers 4g..4g+3 of
// w * max(0, acc) (weights by row broadcast, see weighted_relu_sum)
template <int R>
DSA_DEVICE void row_term(f32x4& p, float W, float x) {
  if constexpr ((R & 3) == 0) p[R >> 2] = fmul_rowbcast<R>(W, x);   // first term of row R/4
  else p[R >> 2] = fmac_rowbcast<R>(p[R >> 2], W, x);
}

template <int... R>
DSA_DEVICE f32x4 row_partials(const f32x16& acc, float W, std::integer_sequence<int, R...>) {
  f32x4 p;
  (row_term<R>(p, W, relu(acc[R])), ...);
  return p;
}

template <int D>
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
  for (int i = threadIdx.x; i < kRowsWg * (kRBins / 2); i += kThreads) hist[i] = 0u;
  if (threadIdx.x == 0) s_maxpos = -1;
  __syncthreads();
  if (lane == 0) atomicMax(&s_maxpos, wave_max);
  __syncthreads();
  const int maxpos = s_maxpos;
  if (maxpos < 0) return;
  const int n_stages = maxpos / kStageKeys + 1;
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
  auto fetch_piece = [&](int j, int st) {
    const int p = threadIdx.x + j * kThreads;
    const int key = min(st * kStageKeys + p / NC, maxpos);   // inside the cache
    pre[j] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * RB + (p % NC) * 16);
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
  auto mfma = [&](f32x16& acc, const bf16x8 (&b)[S]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], b[s], acc, 0, 0, 0);
  };

  // finish of two sub-tiles A (keys key0..key0+31) and B (key0+32..key0+63):
  // for each row g of the wave, one lane-half swap of its partials puts A's
  // key l in lane l and B's key l-32 in lane l (l >= 32), so one register
  // holds row g's scores of 64 consecutive keys and its score row and
  // histogram are addressed from a wave-uniform base
  const size_t rs = (size_t)a.row_stride;
  auto finish_pair = [&](int key0, const f32x4& pa, const f32x4& pb) {
    const int u = key0 + lane;
#pragma unroll
    for (int g = 0; g < kPer; ++g) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa[g]), __float_as_uint(pb[g]),
                                                       false, false);
      const float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int p = pos[g];                     // wave-uniform
      if (key0 > p) continue;
      float* srow = a.scores + (size_t)(t0 + g) * rs;
      uint32_t* hrow = hist + (wv * kPer + g) * (kRBins / 2);
      if (key0 + 63 <= p || u <= p) {
        srow[u] = sc;
        const uint32_t bin = fast_key(sc) >> kRBinShift;
        atomicAdd(hrow + (bin >> 1), 1u << ((bin & 1u) << 4));
      }
    }
  };
  auto epi = [&](const f32x16& acc) {
    return row_partials(acc, W, std::make_integer_sequence<int, 16>{});
  };

  // software pipeline over 32-key sub-tiles, stage barrier in sub-tile 2 (see
  // the dense prefill kernel); sub-tiles are finished in pairs
#pragma unroll
  for (int j = 0; j < LOADS; ++j) fetch_piece(j, 0);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) stash_piece(j, 0);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) fetch_piece(j, 1);
  slot(0, 1);
  __syncthreads();
  bf16x8 b0[S], b1[S];
  f32x16 accx, accy;
  f32x4 pe = {0.f, 0.f, 0.f, 0.f};
  load_b(b0, ktile, 0);
  for (int st = 0; st < n_stages; ++st) {
    const uint8_t* tile = ktile + (st & 1) * STAGE;
    const int k0 = st * kStageKeys;
    load_b(b1, tile, 1);
    mfma(accx, b0);
    if (st > 0) finish_pair(k0 - 64, pe, epi(accy));
    slot(1, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(b0, tile, 2);
    mfma(accy, b1);
    pe = epi(accx);
    slot(2, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(b1, tile, 3);
    mfma(accx, b0);
    slot(3, st + 1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    finish_pair(k0, pe, epi(accy));
    load_b(b0, ktile + ((st + 1) & 1) * STAGE, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma(accy, b1);
    pe = epi(accx);
    slot(0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  finish_pair(n_stages * kStageKeys - 64, pe, epi(accy));
  __syncthreads();

  // each row's threshold: the 10-bit bin holding its k-th score
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
    uint32_t mine = 0;
    for (int wd = (b_hi - PERB) / 2; wd < b_hi / 2; ++wd) {
      const uint32_t v = hrow[wd];
      mine += (v & 0xFFFFu) + (v >> 16);
    }
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
        const uint32_t c = (hrow[b >> 1] >> ((b & 1) * 16)) & 0xFFFFu;
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

template <int D>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr size_t lds = routed_lds_bytes<D>();
  static_assert(lds <= 160 * 1024, "LDS");
  auto k = k_prefill_routed_score<D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = (a.nq + kRowsWg - 1) / kRowsWg;
  hipLaunchKernelGGL(k, dim3(groups), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_routed_score(const PrefillArgs& a, hipStream_t stream) {
  if (a.nq <= 0) return hipSuccess;
  if (a.h_use < 1 || a.h_use > kRoutedMaxHeads || a.bin_bits != kRBinBits) return hipErrorInvalidValue;
  if (a.head_dim == 128) return launch_t<128>(a, stream);
  if (a.head_dim == 64) return launch_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
