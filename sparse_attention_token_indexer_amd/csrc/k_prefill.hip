// Prefill-shaped dense indexer: every query row t of one sequence scores its
// causal prefix u = 0..pos_t (MISA summary, "problem": the H_I-head indexer
// scores every prefix token; its cost grows as O(L^2) over a prefill, HISA
// review section 2) and keeps the exact top-k.
//
// k_prefill_score: one workgroup = 8 consecutive query rows, one wave per row
// with its 64x128 query block resident in registers.  The rows share the key
// cache: 64-key stages are staged in LDS (double-buffered, XOR-swizzled so the
// MFMA operand reads are free of bank conflicts) and each wave runs
// v_mfma_f32_32x32x16_bf16 with heads as rows and keys as columns, then the
// fused ReLU-weighted head reduction in registers.  Scores go to a workspace row
// and into a per-row 12-bit histogram in LDS; at the end each wave finds the
// bin that holds its row's k-th score.  Workgroups run longest rows first.
// k_prefill_select: one workgroup per row emits every score above that bin and
// resolves the bin itself exactly (radix digits over (score, ~index)).
#include "dsa_internal.h"
#include "dsa_common.h"
#include "dsa_select.h"

namespace dsa {

namespace {

constexpr int kPT = 64 * kPrefillRows;   // one wave per query row
constexpr int kStageKeys = 64;
constexpr int kST = 256;                 // select workgroup
constexpr uint32_t kSelListCap = 2048;   // tie-bin entries kept in LDS (global fallback beyond)

template <int D>
constexpr size_t prefill_lds_bytes() {
  return 2 * (size_t)kStageKeys * D * 2 + (size_t)kPrefillRows * (kBins / 2) * 4;
}

template <int HT, int D>
__global__ __launch_bounds__(kPT) void k_prefill_score(PrefillArgs a) {
  constexpr int S = D / 16;                    // k-steps
  constexpr int RB = D * 2;                    // bytes per key row
  constexpr int NC = RB / 16;                  // 16-byte pieces per key row
  constexpr int STAGE = kStageKeys * RB;       // bytes per LDS stage
  constexpr int LOADS = STAGE / 16 / kPT;      // 16-byte loads per thread per stage
  static_assert(LOADS >= 1 && STAGE % (16 * kPT) == 0, "stage size");
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* ktile = smem;                                           // [2][STAGE]
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + 2 * STAGE);  // [rows][kBins / 2]
  __shared__ int s_maxpos;

  const int wv = wave_id(), lane = lane_id();
  const int grp = (int)gridDim.x - 1 - (int)blockIdx.x;            // longest rows first
  const int t = grp * kPrefillRows + wv;
  int pos = -1;
  if (t < a.nq) {
    const int seq = a.q_seq ? a.q_seq[t] : 0;
    const int p = a.q_pos[t];
    if (seq == 0 && p >= 0 && (int64_t)p < a.l_max) pos = p;
  }
  for (int i = threadIdx.x; i < kPrefillRows * (kBins / 2); i += kPT) hist[i] = 0u;
  if (threadIdx.x == 0) s_maxpos = -1;
  __syncthreads();
  if (lane == 0) atomicMax(&s_maxpos, pos);
  __syncthreads();
  const int maxpos = s_maxpos;
  if (maxpos < 0) return;                      // the select kernel pads these rows
  const int n_stages = maxpos / kStageKeys + 1;

  // this wave's query row (zeros for an invalid row)
  const int m = lane & 31, h = lane >> 5;
  bf16x8 qa[HT][S];
  float wr[HT][16];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int row = ht * 32 + m;
    const bool ok = pos >= 0 && row < a.n_heads;
    const uint16_t* src = a.q + ((size_t)t * a.n_heads + (ok ? row : 0)) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < S; ++s) qa[ht][s] = ok ? load_bf16x8(src + 16 * s) : zero_bf16x8();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rs = ht * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      wr[ht][r] = (pos >= 0 && rs < a.n_heads) ? a.w[(size_t)t * a.n_heads + rs] : 0.f;
    }
  }

  // stage loading: thread piece p = threadIdx.x + j * kPT is key p / NC, piece
  // p % NC, stored at LDS slot (piece ^ (key % NC)) of that key's row
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.keys);
  u32x4 pre[LOADS];
  auto fetch = [&](int st) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int p = threadIdx.x + j * kPT;
      int key = st * kStageKeys + p / NC;
      if (key > maxpos) key = maxpos;          // stays inside the cache; never scored
      pre[j] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * RB + (p % NC) * 16);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int p = threadIdx.x + j * kPT;
      const int key = p / NC, pc = p % NC;
      *reinterpret_cast<u32x4*>(ktile + buf * STAGE + key * RB + ((pc ^ (key % NC)) * 16)) = pre[j];
    }
  };

  float* srow = a.scores + (size_t)(t < a.nq ? t : 0) * (size_t)a.row_stride;
  uint32_t* hrow = hist + wv * (kBins / 2);
  fetch(0);
  stash(0);
  __syncthreads();
  for (int st = 0; st < n_stages; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < n_stages;
    if (more) fetch(st + 1);
#pragma unroll
    for (int sub = 0; sub < kStageKeys / 32; ++sub) {
      const int key0 = st * kStageKeys + sub * 32;
      if (key0 <= pos) {                       // wave-uniform
        const int kl = sub * 32 + m;           // key within the stage for this lane's column
        const uint8_t* krow = ktile + buf * STAGE + kl * RB;
        bf16x8 b[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int pc = 2 * s + h;
          b[s] = __builtin_bit_cast(bf16x8,
                                    *reinterpret_cast<const u32x4*>(krow + ((pc ^ (kl % NC)) * 16)));
        }
        f32x16 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[ht][r] = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][s], b[s], acc[ht], 0, 0, 0);
        float p = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int r = 0; r < 16; ++r) p = __builtin_fmaf(wr[ht][r], relu(acc[ht][r]), p);
        p += shfl_xor_f(p, 32);
        const int u = key0 + lane;
        if (lane < 32 && u <= pos) {
          srow[u] = p;
          const uint32_t bin = score_to_key(p) >> kBinShift;
          atomicAdd(hrow + (bin >> 1), 1u << ((bin & 1u) * 16));
        }
      }
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
  }

  // this row's threshold: the 12-bit bin holding its k-th score
  if (pos < 0) return;
  int32_t* meta = a.rowmeta + (size_t)t * 4;
  if (pos + 1 <= a.top_k) {                    // short row: every key is selected
    if (lane == 0) { meta[0] = -1; meta[1] = 0; meta[2] = 0; }
    return;
  }
  // lane l owns bins [kBins - 64 (l + 1), kBins - 64 l), counted from the top
  const int b_hi = kBins - 64 * lane;           // exclusive
  uint32_t mine = 0;
  for (int wd = (b_hi - 64) / 2; wd < b_hi / 2; ++wd) {
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
    for (int b = b_hi - 1; b >= b_hi - 64; --b) {
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

// (score key, index) pairs of one row, generated from the stored scores.
struct RowSource {
  const float* sc;
  uint32_t n;
  template <int NT, class F>
  DSA_DEVICE void for_each(F&& f) const {
    for (uint32_t u = threadIdx.x; u < n; u += NT) f(make_uint2(score_to_key(sc[u]), u));
  }
};

__global__ __launch_bounds__(kST) void k_prefill_select(PrefillArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint2* list = reinterpret_cast<uint2*>(smem);                          // [kSelListCap]
  uint2* tie = list + kSelListCap;                                        // [64]
  uint32_t* hist = reinterpret_cast<uint32_t*>(tie + 64);                 // [1024]
  uint32_t* scratch = hist + 1024;                                        // [64]
  __shared__ uint32_t s_out, s_ln;
  const int t = blockIdx.x;
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
  for (int i = Kt + threadIdx.x; i < a.top_k; i += kST) {
    out_i[i] = -1;
    if (out_s) out_s[i] = -__builtin_inff();
  }
  if (Kt == 0) return;
  const float* sc = a.scores + (size_t)t * (size_t)a.row_stride;
  if (n <= (uint32_t)a.top_k) {                // every key of a short row
    for (uint32_t u = threadIdx.x; u < n; u += kST) {
      out_i[u] = (int32_t)u;
      if (out_s) out_s[u] = key_to_score(score_to_key(sc[u]));
    }
    return;
  }
  const int32_t* meta = a.rowmeta + (size_t)t * 4;
  const int bstar = meta[0];
  const uint32_t above = (uint32_t)meta[1], nb = (uint32_t)meta[2];
  if (threadIdx.x == 0) { s_out = 0; s_ln = 0; }
  __syncthreads();
  const Emitter em{out_i, out_s, &s_out, Kt};
  const bool fits = nb <= kSelListCap;
  // one pass over the row (16-byte loads): emit every score above the bin,
  // collect the bin itself
  constexpr int U = 4;
  const uint32_t n4 = (n + 3) / 4;
  for (uint32_t base = 0; base < n4; base += kST * U) {
    f32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t i4 = base + threadIdx.x + j * kST;
      if (i4 < n4) v[j] = *reinterpret_cast<const f32x4*>(sc + 4 * (size_t)i4);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t i4 = base + threadIdx.x + j * kST;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = 4 * i4 + e;
        const bool ok = i4 < n4 && u < n;
        const uint32_t key = ok ? score_to_key(v[j][e]) : 0u;
        const int b = ok ? (int)(key >> kBinShift) : -1;
        em.put_wave(b > bstar, key, (int32_t)u);
        if (fits) list_put_wave(b == bstar, make_uint2(key, u), list, &s_ln, kSelListCap);
      }
    }
  }
  __syncthreads();
  const uint32_t need = Kt - above;
  if (fits) {
    const uint32_t nl = s_ln < nb ? s_ln : nb;
    finish_bin<kST>(list, nl, need, bstar, em, hist, scratch, tie);
  } else {
    const uint64_t prefix = (uint64_t)bstar << (64 - kBinBits);
    const uint64_t mask = (uint64_t)(kBins - 1) << (64 - kBinBits);
    RowSource src{sc, n};
    radix_finish<kST>(src, prefix, mask, 64 - kBinBits, need, nb, em, hist, scratch);
  }
}

template <int HT, int D>
hipError_t launch_score_t(const PrefillArgs& a, hipStream_t stream) {
  const size_t lds = prefill_lds_bytes<D>();
  auto k = k_prefill_score<HT, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = (a.nq + kPrefillRows - 1) / kPrefillRows;
  hipLaunchKernelGGL(k, dim3(groups), dim3(kPT), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_score(const PrefillArgs& a, hipStream_t stream) {
  if (a.nq <= 0) return hipSuccess;
  if (a.head_dim == 128) return a.n_heads <= 32 ? launch_score_t<1, 128>(a, stream)
                                                : launch_score_t<2, 128>(a, stream);
  if (a.head_dim == 64) return a.n_heads <= 32 ? launch_score_t<1, 64>(a, stream)
                                               : launch_score_t<2, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t stream) {
  if (a.nq <= 0) return hipSuccess;
  const size_t lds = (size_t)kSelListCap * 8 + 64 * 8 + (1024 + 64) * 4;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_prefill_select),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_prefill_select, dim3(a.nq), dim3(kST), lds, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
