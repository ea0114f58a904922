// Certified exact top-k of the dense indexer (DoSA review, sections 1 and 3:
// screen with part of the heads, bound the rest, prune, rescore the
// survivors with every head; the page gives no formulas, so the bounds are
// derived here).
//
// Screening set S: the h heads of largest |w_j| * |q_j| (ties: lower j).  For
// every head j outside S, Cauchy-Schwarz gives 0 <= max(0, q_j . k) <=
// |q_j| |k|, so with s_S(u) the exact screened score of key u
//   s_S(u) + |k_u| N-  <=  s(u)  <=  s_S(u) + |k_u| N+,
//   N+ = sum_{j not in S, w_j > 0} w_j |q_j|,  N- = sum_{j not in S, w_j < 0} w_j |q_j|.
// The screening pass (k_score_emit, certified variant) ranks every key by its
// lower bound and stores its upper bound; tau, the k-th largest lower bound,
// is at most the k-th largest score, so a key whose upper bound is below tau
// scores strictly below it and cannot be selected (ties included).  The
// comparison is on order-preserving keys, with an error margin on both bounds
// (kCertRel).
//
// k_certify_heads: one wave per query, one lane per head: |q_j|, the screened
//   heads and {N+, N-, M = sum_j |w_j| |q_j|}.
// k_certify_compact: one workgroup per query x 4096 keys: tau from the
//   screening selection, then every key whose upper bound reaches tau is
//   appended to the query's survivor list, in key order within the workgroup
//   (one device atomic per workgroup).
// k_certify_counts: the survivor counts to the caller.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kCompactItems = 4096;              // keys per compaction workgroup
constexpr int kCT = 256;

DSA_DEVICE bool query_ok(const CertArgs& a, int t, int64_t* pos) {
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  *pos = a.q_pos[t];
  return seq >= 0 && seq < a.n_seq && *pos >= 0 && *pos < a.l_max;
}

__global__ __launch_bounds__(64) void k_certify_heads(CertArgs a) {
  const int t = blockIdx.x, j = threadIdx.x;
  const int H = a.n_heads, D = a.head_dim;
  float nqj = 0.f, wj = 0.f;
  if (j < H) {
    const uint16_t* qr = a.q + ((size_t)t * H + j) * D;
    for (int d = 0; d < D; d += 8) {
      const bf16x8 v = load_bf16x8(qr + d);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)v[e];
        nqj = __builtin_fmaf(x, x, nqj);
      }
    }
    nqj = sqrtf(nqj);
    wj = a.w[(size_t)t * H + j];
  }
  // rank on the order-preserving key of |w_j| |q_j| (a total order, NaN
  // included, so the ranks are a permutation); lanes past H rank last
  const uint32_t cj = j < H ? score_to_key(fabsf(wj) * nqj) : 0u;
  int rank = 0;
  for (int i = 0; i < 64; ++i) {
    const uint32_t ci = (uint32_t)__shfl((int)cj, i, 64);
    rank += (ci > cj) || (ci == cj && i < j);
  }
  const bool in_s = j < H && rank < a.h;
  if (in_s) a.heads[(size_t)t * a.h + rank] = j;
  float np = (j < H && !in_s && wj > 0.f) ? wj * nqj : 0.f;
  float nn = (j < H && !in_s && wj < 0.f) ? wj * nqj : 0.f;
  float m = j < H ? fabsf(wj) * nqj : 0.f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    np += shfl_xor_f(np, o);
    nn += shfl_xor_f(nn, o);
    m += shfl_xor_f(m, o);
  }
  if (j == 0) {
    a.cert[(size_t)t * 4 + 0] = np;
    a.cert[(size_t)t * 4 + 1] = nn;
    a.cert[(size_t)t * 4 + 2] = m;
    a.cert[(size_t)t * 4 + 3] = 0.f;
  }
}

__global__ __launch_bounds__(kCT) void k_certify_compact(CertArgs a) {
  __shared__ uint32_t s_min[kCT / 64];
  __shared__ uint32_t s_pad;
  const int t = blockIdx.x, c = blockIdx.y, tid = (int)threadIdx.x, lane = lane_id();
  int64_t pos;
  if (!query_ok(a, t, &pos)) return;
  const int64_t u0 = (int64_t)c * kCompactItems;
  if (u0 > pos) return;
  // tau: the smallest lower-bound key of the screening selection; a padded
  // slot (fewer valid keys than top_k) keeps every key
  uint32_t mn = 0xFFFFFFFFu;
  bool pad = false;
  for (int i = tid; i < a.top_k; i += kCT) {
    const int32_t id = a.lb_idx[(size_t)t * a.top_k + i];
    if (id < 0) pad = true;
    else {
      const float f = a.lb_score[(size_t)t * a.top_k + i];
      const uint32_t k = f == f ? score_to_key(f) : 1u;         // (NaN ranks lowest)
      mn = k < mn ? k : mn;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t x = (uint32_t)__shfl_xor((int)mn, o, 64);
    mn = x < mn ? x : mn;
  }
  if (tid == 0) s_pad = 0u;
  __syncthreads();
  if (pad) s_pad = 1u;
  if (lane == 0) s_min[tid >> 6] = mn;
  __syncthreads();
  uint32_t tau = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kCT / 64; ++i) tau = s_min[i] < tau ? s_min[i] : tau;
  if (s_pad) tau = 0u;
  // survivors of this workgroup's keys, in key order: thread i takes keys
  // u0 + i * kPer .. + kPer; the counts' block scan and one device atomic per
  // workgroup place them
  const int64_t u1 = (u0 + kCompactItems - 1 < pos ? u0 + kCompactItems - 1 : pos);
  const float* ub = a.ub + (size_t)t * a.l_max;
  int32_t* list = a.list + (size_t)t * a.l_max;
  constexpr int kPer = kCompactItems / kCT;
  const int64_t v0 = u0 + (int64_t)tid * kPer;
  uint32_t keep = 0;                              // bit i: key v0 + i survives
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t u = v0 + i;
    const float x = u <= u1 ? ub[u] : 0.f;
    if (u <= u1 && (x != x || score_to_key(x) >= tau)) keep |= 1u << i;   // NaN: kept
  }
  const uint32_t n = (uint32_t)__popc(keep);
  uint32_t incl = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
    if (lane >= o) incl += y;
  }
  __shared__ uint32_t s_wave[kCT / 64], s_base;
  if (lane == 63) s_wave[tid >> 6] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kCT / 64; ++i) {
    before += i < (tid >> 6) ? s_wave[i] : 0u;
    total += s_wave[i];
  }
  if (tid == 0) s_base = total ? atomicAdd(&a.cnt[t], total) : 0u;
  __syncthreads();
  uint32_t o = s_base + before + incl - n;
  for (int i = 0; i < kPer; ++i)
    if (keep >> i & 1u) list[o++] = (int32_t)(v0 + i);
}

// the survivor counts to the caller (after the compaction, in stream order)
__global__ __launch_bounds__(256) void k_certify_counts(CertArgs a) {
  const int t = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (t < a.nq) a.out_survivors[t] = (int32_t)a.cnt[t];
}

}  // namespace

hipError_t launch_certify_heads(const CertArgs& a, hipStream_t stream) {
  if (a.nq < 1 || a.n_heads < 1 || a.n_heads > 64 || a.h < 1 || a.h > a.n_heads ||
      (a.head_dim != 64 && a.head_dim != 128))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_certify_heads, dim3(a.nq), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_certify_compact(const CertArgs& a, hipStream_t stream) {
  if (a.nq < 1 || a.top_k < 1 || a.l_max < 1) return hipErrorInvalidValue;
  const int64_t chunks = (a.l_max + kCompactItems - 1) / kCompactItems;
  if (chunks > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_certify_compact, dim3(a.nq, (unsigned)chunks), dim3(kCT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_certify_counts(const CertArgs& a, hipStream_t stream) {
  if (a.nq < 1 || !a.out_survivors) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_certify_counts, dim3((unsigned)((a.nq + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
