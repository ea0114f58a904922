// Sparse attention over the selected index list.
//
// HISA review, key terms and section 3: the selected token indices go, as
// they are, to the downstream Sparse MLA operator; IndexCache review,
// section 1: with k selected tokens per query the core attention costs
// O(L k).  No page gives the operator's formula; the reading taken is
// ordinary scaled-softmax attention restricted to the listed rows, in
// absorbed multi-head latent attention form: every token has one latent row
// c[u] of 576 values, the key of every head, whose first 512 values are the
// value.  Per query t and head h:
//   o[t, h] = sum_i softmax_i(scale * q[t, h] . c[idx_i]) c[idx_i, :512]
// over the list entries inside the query's prefix.
//
// One workgroup = one query x one slice of its list, NW waves of 16 heads
// each.  Per step the workgroup gathers 32 listed rows into LDS (row-major
// for the scores, the value part also transposed for the value product) while
// the next step's rows load into registers.  Each wave forms the 32 x 16
// block S^T = C Q^T on 16x16x32 bf16 MFMAs (its heads' query rows stay in
// registers, the last k-steps in LDS), so a lane owns one head and 8 of the
// step's rows: the running max and sum of the online softmax need no exchange
// across heads.  The
// probabilities, rounded to bf16, are the B operand of O^T += V^T P^T as they
// sit in the lane (the k order of the product is the lane's own row order),
// and O^T (512 x 16 per wave) stays in accumulation registers.  A query whose
// list is split writes its unnormalised slices with their (max, sum); a
// second kernel merges them.  Slices are stored in bf16 (relative 2^-9, like
// the output itself).
#include "dsa_common.h"
#include "dsa_mla.h"

namespace dsa {

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kCh = kMlaDqk / 8;                 // 16-byte chunks per row (72)
constexpr int kVCh = kMlaDv / 8;                 // of them in the value part (64)
constexpr int kPieces = kMlaTile * kCh;          // chunks per step (2304)
constexpr int kS = kMlaDqk / 32;                 // k-steps of the score product (18)
constexpr int kDt = kMlaDv / 16;                 // 16-row value blocks (32)
constexpr int kSR = kS - kMlaQLds;               // query k-steps held in registers

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_sparse_mla(MlaArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int R = (kPieces + NT - 1) / NT;     // chunks per thread per step
  static_assert(NT % kMlaTile == 0, "a thread gathers one row position");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* lc = smem;                                        // [32][kMlaCRow]
  uint16_t* lv = reinterpret_cast<uint16_t*>(smem + kMlaTile * kMlaCRow);   // [512][kMlaVRow/2]
  uint8_t* lq = smem + kMlaTile * kMlaCRow + kMlaDv * kMlaVRow;              // [n_heads][kMlaQRow]
  int32_t* sid = reinterpret_cast<int32_t*>(lq + (size_t)(NW * 16) * kMlaQRow);

  const int t = (int)blockIdx.x / a.splits, sp = (int)blockIdx.x - t * a.splits;
  const int tid = (int)threadIdx.x, lane = lane_id(), g = lane >> 4, col = lane & 15;
  const int head = wave_id() * 16 + col;
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  const bool ok = seq >= 0 && seq < a.n_seq && pos >= 0 && pos < a.l_max;
  const int n_tok = a.tiles_per_split * kMlaTile;
  const int base = sp * n_tok;

  // the slice's row ids (-1: skipped)
  for (int i = tid; i < n_tok; i += NT) {
    const int j = base + i;
    int e = j < a.top_k ? a.idx[(size_t)t * a.top_k + j] : -1;
    sid[i] = (ok && e >= 0 && (int64_t)e <= pos) ? e : -1;
  }
  // this wave's heads' query rows, as the B operand (k = 32 s + 8 g ..): the
  // first kSR k-steps in registers, the rest in LDS where only this lane
  // reads them back
  bf16x8 qb[kSR];
  uint8_t* lq_lane = lq + (size_t)head * kMlaQRow + 16 * g;
  {
    const uint16_t* qr = a.q + ((size_t)t * a.n_heads + head) * kMlaDqk + 8 * g;
#pragma unroll
    for (int s = 0; s < kSR; ++s) qb[s] = load_bf16x8(qr + 32 * s);
#pragma unroll
    for (int s = kSR; s < kS; ++s)
      *reinterpret_cast<bf16x8*>(lq_lane + 64 * (s - kSR)) = load_bf16x8(qr + 32 * s);
  }
  __syncthreads();

  const uint16_t* kv_seq = a.kv + (size_t)(ok ? seq : 0) * (size_t)a.l_max * kMlaDqk;
  const int tok = tid % kMlaTile, c0 = tid / kMlaTile;
  u32x4 pf[R];
  auto prefetch = [&](int tile) {
    const int e = sid[tile * kMlaTile + tok];
    const uint16_t* row = kv_seq + (size_t)(e >= 0 ? e : 0) * kMlaDqk;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = c0 + r * (NT / kMlaTile);
      if (c < kCh) pf[r] = e >= 0 ? *reinterpret_cast<const u32x4*>(row + 8 * c) : u32x4{0, 0, 0, 0};
    }
  };

  f32x4 acc[kDt];
#pragma unroll
  for (int d = 0; d < kDt; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.f;

  prefetch(0);
  for (int tile = 0; tile < a.tiles_per_split; ++tile) {
    // the step's rows into LDS: row-major, and the value part transposed
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = c0 + r * (NT / kMlaTile);
      if (c < kCh) {
        *reinterpret_cast<u32x4*>(lc + tok * kMlaCRow + 16 * c) = pf[r];
        if (c < kVCh) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lv[(8 * c + 2 * i) * (kMlaVRow / 2) + tok] = (uint16_t)(pf[r][i] & 0xFFFFu);
            lv[(8 * c + 2 * i + 1) * (kMlaVRow / 2) + tok] = (uint16_t)(pf[r][i] >> 16);
          }
        }
      }
    }
    __syncthreads();
    if (tile + 1 < a.tiles_per_split) prefetch(tile + 1);

    // S^T = C Q^T: rows 16 c + 4 g + r of the step, column = this lane's head
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const bf16x8 qs = s < kSR ? qb[s < kSR ? s : 0]
                                : *reinterpret_cast<const bf16x8*>(lq_lane + 64 * (s - kSR));
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 ca = *reinterpret_cast<const bf16x8*>(lc + (16 * c + col) * kMlaCRow +
                                                            (32 * s + 8 * g) * 2);
        sacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca, qs, sacc[c], 0, 0, 0);
      }
    }
    // online softmax over the step, in log2 units
    float x[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool v = sid[tile * kMlaTile + 16 * c + 4 * g + r] >= 0;
        x[4 * c + r] = v ? sacc[c][r] * a.scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, x[4 * c + r]);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f;
    bf16x8 pb;
    if (m_new == -__builtin_inff()) {            // nothing valid for this head yet
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)0.f;
    } else {
      alpha = exp2f(m_run - m_new);              // 0 when m_run is -inf
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = exp2f(x[j] - m_new);
        ps += p;
        pb[j] = (__bf16)p;
      }
      l_run = l_run * alpha + ps;
      m_run = m_new;
    }
    // O^T += V^T P^T (A: value rows 16 dt + col, k-slot 8 g + j = step row
    // 16 (j / 4) + 4 g + j % 4, matching where the lane's probabilities sit)
#pragma unroll
    for (int d = 0; d < kDt; ++d) {
      const uint16_t* vr = lv + (16 * d + col) * (kMlaVRow / 2) + 4 * g;
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
      const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[d] = acc[d] * alpha;
      acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[d], 0, 0, 0);
    }
    __syncthreads();
  }

  // the head's sum over the four lane groups
  float l = l_run + shfl_xor_f(l_run, 16);
  l += shfl_xor_f(l, 32);
  // the output, or this slice's output (divided by its own sum) for the merge
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t slot = ((size_t)t * a.splits + sp) * a.n_heads + head;
  uint16_t* o = (a.splits == 1 ? a.out + ((size_t)t * a.n_heads + head) * kMlaDv
                               : a.part_o + slot * kMlaDv) + 4 * g;
#pragma unroll
  for (int d = 0; d < kDt; ++d) {
    bf16x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (__bf16)(acc[d][r] * inv);
    *reinterpret_cast<bf16x4*>(o + 16 * d) = v;
  }
  if (a.splits > 1 && g == 0) a.part_ml[slot] = make_float2(m_run, l);
}

// Merge of a query's slices: with M the largest running max and
// w_s = 2^(m_s - M) l_s, o = sum_s w_s o_s / sum_s w_s, o_s the slice's
// normalised output (zeros when no slice saw a valid row).
// One thread = one head x 8 value columns (16-byte loads and stores).
__global__ __launch_bounds__(256) void k_mla_combine(MlaArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_q = (int64_t)a.n_heads * (kMlaDv / 8);
  if (i >= (int64_t)a.nq * per_q) return;
  const int t = (int)(i / per_q);
  const int rem = (int)(i - (int64_t)t * per_q);
  const int head = rem / (kMlaDv / 8), c8 = rem - head * (kMlaDv / 8);
  float M = -__builtin_inff();
  for (int s = 0; s < a.splits; ++s)
    M = fmaxf(M, a.part_ml[((size_t)t * a.splits + s) * a.n_heads + head].x);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < a.splits; ++s) {
      const size_t slot = ((size_t)t * a.splits + s) * a.n_heads + head;
      const float2 ml = a.part_ml[slot];
      if (ml.x == -__builtin_inff()) continue;
      const float w = exp2f(ml.x - M) * ml.y;
      const bf16x8 os = *reinterpret_cast<const bf16x8*>(a.part_o + slot * kMlaDv + 8 * c8);
      L += w;
#pragma unroll
      for (int r = 0; r < 8; ++r) o[r] += w * (float)os[r];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  bf16x8 v;
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = (__bf16)(o[r] * inv);
  *reinterpret_cast<bf16x8*>(a.out + ((size_t)t * a.n_heads + head) * kMlaDv + 8 * c8) = v;
}

template <int NW>
hipError_t launch_t(const MlaArgs& a, hipStream_t stream) {
  const size_t lds = mla_lds_bytes(a.n_heads, a.tiles_per_split);
  auto k = k_sparse_mla<NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.nq * a.splits), dim3(64 * NW), lds, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.splits > 1) {
    const int64_t n = (int64_t)a.nq * a.n_heads * (kMlaDv / 8);
    hipLaunchKernelGGL(k_mla_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
  if (a.nq < 1 || a.top_k < 1 || a.top_k > kMlaMaxTopK || a.n_heads < 32 || a.n_heads > 128 ||
      a.n_heads % 32 || a.splits < 1 || a.splits > kMlaMaxSplits || a.tiles_per_split < 1 ||
      a.tiles_per_split > kMlaMaxTiles ||
      (int64_t)a.splits * a.tiles_per_split * kMlaTile < a.top_k ||
      (int64_t)a.nq * a.splits > 0x7FFFFFFF ||
      mla_lds_bytes(a.n_heads, a.tiles_per_split) > 160 * 1024 ||
      (a.splits > 1 && (!a.part_o || !a.part_ml)))
    return hipErrorInvalidValue;
  switch (a.n_heads / 32) {
    case 1: return launch_t<2>(a, stream);
    case 2: return launch_t<4>(a, stream);
    case 3: return launch_t<6>(a, stream);
    default: return launch_t<8>(a, stream);
  }
}

}  // namespace dsa
