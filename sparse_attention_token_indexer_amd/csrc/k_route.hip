// MISA router: per-head importance from the mean-pooled block keys and the
// top-h head set of each query.
//
// MISA summary, "method" step 1: the router computes per-head affinities
// against pooled block-level keys instead of individual tokens, aggregates them
// into an importance per head for the current query and keeps the top-h heads;
// it touches only M = ceil(L/B) pooled keys, so its cost is O(H_I M).
// Reading taken where the page gives no formula: affinity = max(0, q_j . kbar_b),
// importance I_j = |w_j| * sum_b affinity, ties to the lower head index.
//
// One workgroup = one query x one slice of its blocks; bf16 MFMA with heads as
// rows and pooled blocks as columns, the ReLU'd affinities summed per head in
// registers, then across lanes and waves in a fixed order, and written per
// slice.  The routed scoring pass adds the slices in slice order, weights by |w|
// and ranks the heads (route_heads in k_score_select.hip), so no workgroup waits on another.
#include "dsa_internal.h"
#include "dsa_common.h"

namespace dsa {

namespace {

constexpr int kRT = 256;

template <int HT, int D>
__global__ __launch_bounds__(kRT) void k_route(RouteArgs a) {
  constexpr int S = D / 16;
  __shared__ float s_part[kRT / 64][64];
  const int t = blockIdx.y, sp = blockIdx.x;
  const int lane = lane_id(), wv = wave_id(), h = lane >> 5, n = lane & 31;
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  const bool ok = seq >= 0 && seq < a.n_seq && pos >= 0 && pos < a.l_max;
  const int64_t M = ok ? (pos + a.block) / a.block : 0;
  const int64_t b0 = (int64_t)sp * a.blocks_per_split;
  const int64_t b1 = (b0 + a.blocks_per_split) < M ? (b0 + a.blocks_per_split) : M;
  const bool partial_last = a.partial && ok && ((pos + 1) % a.block) != 0;

  float hsum[HT][16];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) hsum[ht][r] = 0.f;

  if (b0 < b1) {
    bf16x8 qa[HT][S];
    const uint16_t* q_t = a.q + (size_t)t * a.n_heads * D;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int row = ht * 32 + n;
#pragma unroll
      for (int s = 0; s < S; ++s)
        qa[ht][s] = row < a.n_heads ? load_bf16x8(q_t + (size_t)row * D + 8 * h + 16 * s)
                                    : zero_bf16x8();
    }
    const int n_tiles = (int)((b1 - b0 + 31) / 32);
    // each wave walks every (kRT / 64)-th tile, the next one's pooled rows
    // loaded while the current one is multiplied
    auto load = [&](bf16x8 (&kb)[S], int tile) {
      const int64_t b = b0 + (int64_t)tile * 32 + n;
      const int64_t bb = b < b1 ? b : b0;
      const uint16_t* rowp = (partial_last && bb == M - 1)
                                 ? a.partial + (size_t)t * D
                                 : a.pooled + ((size_t)seq * (size_t)a.m_max + (size_t)bb) * D;
#pragma unroll
      for (int s = 0; s < S; ++s) kb[s] = load_bf16x8(rowp + 8 * h + 16 * s);
    };
    bf16x8 ka[S], kn[S];
    if (wv < n_tiles) load(ka, wv);
    for (int tile = wv; tile < n_tiles; tile += kRT / 64) {
      if (tile + kRT / 64 < n_tiles) load(kn, tile + kRT / 64);
      const bool valid = b0 + (int64_t)tile * 32 + n < b1;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][s], ka[s], acc, 0, 0, 0);
        if (valid) {
#pragma unroll
          for (int r = 0; r < 16; ++r) hsum[ht][r] += relu(acc[r]);
        }
      }
#pragma unroll
      for (int s = 0; s < S; ++s) ka[s] = kn[s];
    }
  }
  // sum over the 32 block columns held by lanes with the same half h
#pragma unroll
  for (int m = 1; m < 32; m <<= 1)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r) hsum[ht][r] += shfl_xor_f(hsum[ht][r], m);
  if (n == 0) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_part[wv][ht * 32 + 8 * (r >> 2) + 4 * h + (r & 3)] = hsum[ht][r];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < a.n_heads; j += kRT) {
    float p = 0.f;
    for (int w = 0; w < kRT / 64; ++w) p += s_part[w][j];
    a.part[((size_t)t * a.splits + sp) * a.n_heads + j] = p;
  }
}

// Router for many queries with one slice each (prefill shape): one wave per
// query over all of its blocks, the next tile's pooled rows loaded while the
// current one is multiplied; the per-head sums over the 32 block columns are
// reduced through LDS (rows padded to 33 words: conflict-free both ways).
// The partial last block's pooled key comes from a.partial by position
// (prefix means of every position, a.partial_by_pos) or by query.
template <int HT, int D>
__global__ __launch_bounds__(256) void k_route_rows(RouteArgs a) {
  constexpr int S = D / 16;
  __shared__ float s_red[4][64 * 33];
  const int wv = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
  const int t = (int)blockIdx.x * 4 + wv;
  if (t >= a.nq) return;
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  const bool ok = seq >= 0 && seq < a.n_seq && pos >= 0 && pos < a.l_max;
  const int64_t M = ok ? (pos + a.block) / a.block : 0;
  const bool partial_last = a.partial && ok && ((pos + 1) % a.block) != 0;
  const uint16_t* partial_row =
      partial_last ? a.partial + (size_t)(a.partial_by_pos ? pos : t) * D : nullptr;

  float hsum[HT][16];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) hsum[ht][r] = 0.f;
  const int n_tiles = (int)((M + 31) / 32);
  if (n_tiles > 0) {
    bf16x8 qa[HT][S];
    const uint16_t* q_t = a.q + (size_t)t * a.n_heads * D;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int row = ht * 32 + n;
#pragma unroll
      for (int s = 0; s < S; ++s)
        qa[ht][s] = row < a.n_heads ? load_bf16x8(q_t + (size_t)row * D + 8 * h + 16 * s)
                                    : zero_bf16x8();
    }
    auto load = [&](bf16x8 (&kb)[S], int tile) {
      const int64_t b = (int64_t)tile * 32 + n;
      const int64_t bb = b < M ? b : 0;
      const uint16_t* rowp = (partial_last && bb == M - 1)
                                 ? partial_row
                                 : a.pooled + ((size_t)seq * (size_t)a.m_max + (size_t)bb) * D;
#pragma unroll
      for (int s = 0; s < S; ++s) kb[s] = load_bf16x8(rowp + 8 * h + 16 * s);
    };
    bf16x8 ka[S], kn[S];
    load(ka, 0);
    for (int tile = 0; tile < n_tiles; ++tile) {
      if (tile + 1 < n_tiles) load(kn, tile + 1);
      const bool valid = (int64_t)tile * 32 + n < M;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][s], ka[s], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) hsum[ht][r] += valid ? relu(acc[r]) : 0.f;
      }
#pragma unroll
      for (int s = 0; s < S; ++s) ka[s] = kn[s];
    }
  }
  // per head: the sum over the 32 block columns (lane n holds column n)
  float* red = s_red[wv];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(ht * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * 33 + n] = hsum[ht][r];
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  if (lane < a.n_heads) {
    float p = 0.f;
    for (int c = 0; c < 32; ++c) p += red[lane * 33 + c];
    a.part[(size_t)t * a.n_heads + lane] = p;
  }
}

// Router for many queries on ONE sequence (prefill shape): the rows share the
// pooled keys, so 4 rows per workgroup (one wave each, heads x 32 blocks per
// MFMA) read 64-block stages from LDS (double-buffered, rows padded to
// 2*D + 16 bytes, as in the prefill scorers).  Each row sums max(0, q_j . kbar_b)
// over its full blocks b < (pos + 1) / B; the partial last block (prefix mean
// of the row's position, from a.partial by position) is one extra tile with a
// single valid column.  Per-head sums over the 32 block columns go through a
// padded LDS transpose in the stage buffers; one slice per query (part[t][j]).
// The router streams every row's q (all heads) from HBM once: small
// workgroups (35 KB of LDS at D = 128) let two share a CU, so one's q loads
// overlap the other's MFMAs.
constexpr int kPRStage = 64;
constexpr int kPRRows = 4;

// the two stages, or the column transpose that reuses them if larger
template <int D>
constexpr size_t prefill_route_lds() {
  constexpr size_t stages = 2 * (size_t)kPRStage * (2 * D + 16);
  constexpr size_t red = (size_t)kPRRows * 64 * 33 * 4;
  return stages > red ? stages : red;
}

template <int HT, int D>
// (two workgroups per CU: at most 256 registers per lane)
__global__ __launch_bounds__(64 * kPRRows) __attribute__((amdgpu_waves_per_eu(2)))
void k_route_prefill(RouteArgs a) {
  constexpr int kT = 64 * kPRRows;
  constexpr int S = D / 16, RB = 2 * D, NC = RB / 16, LB = RB + 16;
  constexpr int STAGE = kPRStage * LB, PIECES = kPRStage * NC;
  constexpr int LOADS = PIECES / kT;
  static_assert(PIECES % kT == 0, "every thread stores whole pieces");
  constexpr int NSUB = kPRStage / 32;                    // sub-tiles per stage
  constexpr int PER_SLOT = (LOADS + NSUB - 1) / NSUB;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* ktile = smem;                                        // [2][STAGE]
  __shared__ int s_maxfull;
  const int wv = wave_id(), lane = lane_id(), h = lane >> 5, m = lane & 31;
  const int t = ((int)gridDim.x - 1 - (int)blockIdx.x) * kPRRows + wv;   // longest rows first
  int64_t pos = -1;
  if (t < a.nq) {
    const int seq = a.q_seq ? a.q_seq[t] : 0;
    const int64_t p = a.q_pos[t];
    if (seq == 0 && p >= 0 && p < a.l_max) pos = p;
  }
  const int nfull = pos >= 0 ? (int)((pos + 1) / a.block) : 0;   // full blocks of the row
  if (threadIdx.x == 0) s_maxfull = 0;
  __syncthreads();
  if (lane == 0) atomicMax(&s_maxfull, nfull);
  __syncthreads();
  const int maxfull = __builtin_amdgcn_readfirstlane(s_maxfull);

  bf16x8 qa[HT][S];
  {
    const uint16_t* q_t = a.q + (size_t)(pos >= 0 ? t : 0) * a.n_heads * D;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int row = ht * 32 + m;
      const bool ok = pos >= 0 && row < a.n_heads;
#pragma unroll
      for (int s = 0; s < S; ++s)
        qa[ht][s] = ok ? load_bf16x8(q_t + (size_t)(ok ? row : 0) * D + 8 * h + 16 * s) : zero_bf16x8();
    }
  }
  // hsum[ht][r] += max(0, x) for block columns the row counts: med3(x, 0, cap)
  // with cap = +inf for a counted column and 0 otherwise
  float hsum[HT][16];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) hsum[ht][r] = 0.f;
  auto cap_of = [&](int b0) { return b0 + m < nfull ? __builtin_inff() : 0.f; };

  const int n_stages = (maxfull + kPRStage - 1) / kPRStage;
  if (n_stages > 0) {
    const uint8_t* pbase = reinterpret_cast<const uint8_t*>(a.pooled);
    const uint32_t boff = (uint32_t)(m * LB + h * 16);
    const int last = maxfull - 1;
    u32x4 pre[LOADS];
    auto fetch_piece = [&](int j, int st) {
      const int p = threadIdx.x + j * kT;
      const int row = min(st * kPRStage + p / NC, last);     // inside the pooled keys
      pre[j] = *reinterpret_cast<const u32x4*>(pbase + (size_t)row * RB + (p % NC) * 16);
    };
    auto stash_piece = [&](int j, int buf) {
      const int p = threadIdx.x + j * kT;
      *reinterpret_cast<u32x4*>(ktile + buf * STAGE + (p / NC) * LB + (p % NC) * 16) = pre[j];
    };
    auto slot = [&](int q, int st) {
#pragma unroll
      for (int j = q * PER_SLOT; j < (q + 1) * PER_SLOT && j < LOADS; ++j) {
        stash_piece(j, st & 1);
        fetch_piece(j, st + 1);
      }
    };
    // Software pipeline over units (sub-tile c of a stage, head tile u), as in
    // the routed prefill scorer: step s of a unit issues its MFMA for k-step s
    // and adds 16 / S accumulator
    // registers of the previous unit into hsum; the last head tile of a
    // sub-tile also reads the next sub-tile's B operand for k-step s.  Units
    // alternate between two accumulators.  One stage-loading slot per
    // sub-tile; the stage barrier closes the second-to-last sub-tile.
#pragma unroll
    for (int j = 0; j < LOADS; ++j) fetch_piece(j, 0);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) stash_piece(j, 0);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) fetch_piece(j, 1);
    slot(0, 1);
    __syncthreads();
    bf16x8 bb[S];
    f32x16 acc[2];
    // (zero accumulators and cap 0 make the first unit's epilogue add +0)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][r] = acc[1][r] = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s)
      bb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ktile + boff + s * 32));
    constexpr int EPR = 16 / S;
    float cap_prev = 0.f;
    auto step = [&](auto C, auto U, auto SS, int st, float cap_p) {
      constexpr int c = decltype(C)::value, u = decltype(U)::value, s = decltype(SS)::value;
      constexpr int par = (c * HT + u) & 1, pu = u == 0 ? HT - 1 : u - 1;
      if constexpr (s == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[par][r] = 0.f;
      }
      acc[par] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[u][s], bb[s], acc[par], 0, 0, 0);
      if constexpr (u == HT - 1) {
        const uint8_t* nt = ktile + ((c == NSUB - 1 ? st + 1 : st) & 1) * STAGE;
        constexpr int nsub = (c + 1) % NSUB;
        bb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(nt + boff + nsub * 32 * LB + s * 32));
      }
#pragma unroll
      for (int r = s * EPR; r < (s + 1) * EPR; ++r)
        hsum[pu][r] += __builtin_amdgcn_fmed3f(acc[par ^ 1][r], 0.f, cap_p);
      if constexpr (u == HT - 1 && s == S - 2) slot((c + 1) % NSUB, c == NSUB - 1 ? st + 2 : st + 1);
      if constexpr (c == NSUB - 2 && u == HT - 1 && s == S - 1) __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto unit = [&](auto C, auto U, int st, float cap_p) {
      static_for<S>([&](auto SS) { step(C, U, SS, st, cap_p); });
    };
    // all units of sub-tile C; cap_in is the cap of the unit before them
    auto subtile = [&](auto C, int st, float cap_in, float cap_c) {
      unit(C, std::integral_constant<int, 0>{}, st, cap_in);
      if constexpr (HT > 1) unit(C, std::integral_constant<int, 1>{}, st, cap_c);
    };
    static_assert(NSUB == 2, "two sub-tiles per stage");
    for (int st = 0; st < n_stages; ++st) {
      const int k0 = st * kPRStage;
      const float c0 = cap_of(k0), c1 = cap_of(k0 + 32);
      subtile(std::integral_constant<int, 0>{}, st, cap_prev, c0);
      subtile(std::integral_constant<int, 1>{}, st, c0, c1);
      cap_prev = c1;
    }
    // the last unit (sub-tile NSUB - 1, head tile HT - 1)
    constexpr int last_par = ((NSUB - 1) * HT + HT - 1) & 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) hsum[HT - 1][r] += __builtin_amdgcn_fmed3f(acc[last_par][r], 0.f, cap_prev);
  }
  // the partial last block: one tile whose column 0 is the prefix mean of pos
  if (pos >= 0 && ((pos + 1) % a.block) != 0) {
    bf16x8 b[S];
    const uint16_t* rowp = a.partial + (size_t)pos * D;
#pragma unroll
    for (int s = 0; s < S; ++s) b[s] = m == 0 ? load_bf16x8(rowp + 8 * h + 16 * s) : zero_bf16x8();
    const float cap = m == 0 ? __builtin_inff() : 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < S; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][s], b[s], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) hsum[ht][r] += __builtin_amdgcn_fmed3f(acc[r], 0.f, cap);
    }
  }
  // per head: the sum over the 32 block columns (lane m holds column m), in
  // the stage buffers once every wave is done with them
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + wv * (64 * 33);
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(ht * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * 33 + m] = hsum[ht][r];
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  if (t < a.nq && lane < a.n_heads) {
    float p = 0.f;
    for (int c = 0; c < 32; ++c) p += red[lane * 33 + c];
    a.part[(size_t)t * a.n_heads + lane] = p;
  }
}

}  // namespace

template <int HT, int D>
hipError_t launch_route_prefill_t(const RouteArgs& a, hipStream_t stream) {
  constexpr size_t lds = prefill_route_lds<D>();
  static_assert(lds <= 160 * 1024, "LDS");
  auto k = k_route_prefill<HT, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((a.nq + kPRRows - 1) / kPRRows), dim3(64 * kPRRows), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.splits == 1 && a.n_seq == 1 && a.partial_by_pos) {   // rows of one sequence
    if (a.head_dim == 128) return a.n_heads <= 32 ? launch_route_prefill_t<1, 128>(a, stream)
                                                  : launch_route_prefill_t<2, 128>(a, stream);
    if (a.head_dim == 64) return a.n_heads <= 32 ? launch_route_prefill_t<1, 64>(a, stream)
                                                 : launch_route_prefill_t<2, 64>(a, stream);
    return hipErrorInvalidValue;
  }
  if (a.splits == 1) {                        // one wave per query
    const dim3 g((a.nq + 3) / 4);
    if (a.head_dim == 128) {
      if (a.n_heads <= 32) hipLaunchKernelGGL((k_route_rows<1, 128>), g, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((k_route_rows<2, 128>), g, dim3(256), 0, stream, a);
    } else if (a.head_dim == 64) {
      if (a.n_heads <= 32) hipLaunchKernelGGL((k_route_rows<1, 64>), g, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((k_route_rows<2, 64>), g, dim3(256), 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid(a.splits, a.nq);
  if (a.head_dim == 128) {
    if (a.n_heads <= 32) hipLaunchKernelGGL((k_route<1, 128>), grid, dim3(kRT), 0, stream, a);
    else hipLaunchKernelGGL((k_route<2, 128>), grid, dim3(kRT), 0, stream, a);
  } else if (a.head_dim == 64) {
    if (a.n_heads <= 32) hipLaunchKernelGGL((k_route<1, 64>), grid, dim3(kRT), 0, stream, a);
    else hipLaunchKernelGGL((k_route<2, 64>), grid, dim3(kRT), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Head selection from the router's per-slice sums, one wave per query (lane j
// = head j): I_j = |w_j| * (sum of the slices in slice order), top h by
// (I desc, j asc) -- the same order and arithmetic as the decode-shaped routed
// pass, which finishes the selection inside its scoring workgroups.
__global__ __launch_bounds__(256) void k_route_heads(RouteHeadsArgs a) {
  const int t = (int)blockIdx.x * 4 + wave_id();
  const int j = lane_id();
  if (t >= a.nq) return;
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  const bool row_ok = seq >= 0 && seq < a.n_seq && pos >= 0 && pos < a.l_max;
  const bool head_ok = j < a.n_heads;
  float I = 0.f;
  if (head_ok) {
    float tot = 0.f;
    for (int sp = 0; sp < a.splits; ++sp) tot += a.part[((size_t)t * a.splits + sp) * a.n_heads + j];
    I = fabsf(a.w[(size_t)t * a.n_heads + j]) * tot;
    if (a.out_importance) a.out_importance[(size_t)t * a.n_heads + j] = row_ok ? I : 0.f;
  }
  // ranked on the order-preserving keys of I: a total order even for NaN, so
  // the ranks are a permutation and every routed slot gets a head
  const uint32_t kI = score_to_key(I);
  int rank = 0;
  for (int i = 0; i < a.n_heads; ++i) {
    const uint32_t Ii = (uint32_t)__shfl((int)kI, i, 64);
    rank += (Ii > kI) || (Ii == kI && i < j);
  }
  if (head_ok && rank < a.h_use) {
    a.heads[(size_t)t * a.heads_stride + rank] = row_ok ? j : 0;
    if (a.out_heads) a.out_heads[(size_t)t * a.h_use + rank] = row_ok ? j : -1;
  }
}

hipError_t launch_route_heads(const RouteHeadsArgs& a, hipStream_t stream) {
  if (a.nq <= 0) return hipSuccess;
  if (a.n_heads > 64 || a.h_use > a.heads_stride) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_route_heads, dim3((a.nq + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
