// Mean-pooled block keys and the per-call preparation kernel.
//
// MISA summary, "method" step 1: the prefix is split into M = ceil(L/B) blocks
// and the router works on mean-pooled indexing keys; HISA review, section 3:
// pooled representative vectors per block of size B.  A block's pooled key is
// the mean of its valid tokens, accumulated in float64 (exact for bf16 inputs
// of ordinary range) and rounded once to bf16, round-to-nearest-even.
#include "dsa_internal.h"
#include "dsa_common.h"

namespace dsa {

namespace {

DSA_DEVICE double bf16_to_f64(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

// float64 -> bf16, correctly rounded (ties to even): round to float32 with
// round-to-odd first (keeps the sticky information), then to bf16 with RNE.
DSA_DEVICE uint16_t f64_to_bf16(double x) {
  float f = (float)x;
  if ((double)f != x) {
    uint32_t u = __float_as_uint(f);
    if (fabs((double)f) > fabs(x)) u -= 1u;  // step back toward zero
    u |= 1u;                                   // inexact -> odd
    f = __uint_as_float(u);
  }
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One wave per (sequence, block).  Lanes split a key row into 16-byte pieces
// (LPR lanes per row) and 64/LPR rows are read per step, so a wave reads
// contiguous 1 KiB runs of the key cache.
template <int D>
__global__ __launch_bounds__(256) void k_mean_pool(const uint16_t* __restrict__ k, int n_seq,
                                                   int64_t l_max, int block, int64_t m_max,
                                                   uint16_t* __restrict__ out) {
  constexpr int LPR = D / 8;          // lanes per key row
  constexpr int RPS = 64 / LPR;       // rows per step
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= (int64_t)n_seq * m_max) return;
  const int lane = threadIdx.x & 63;
  const int64_t s = gw / m_max, b = gw % m_max;
  const int64_t r0 = b * block;
  const int64_t r1 = (r0 + block) < l_max ? (r0 + block) : l_max;
  const int piece = lane % LPR;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* base = k + ((size_t)s * (size_t)l_max) * D + piece * 8;
#pragma unroll 4
  for (int64_t r = r0 + lane / LPR; r < r1; r += RPS) {
    u32x4 v = *reinterpret_cast<const u32x4*>(base + (size_t)r * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_to_f64((uint16_t)(v[e] & 0xFFFFu));
      acc[2 * e + 1] += bf16_to_f64((uint16_t)(v[e] >> 16));
    }
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
  if (lane < LPR) {
    const double n = (double)(r1 - r0);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t lo = f64_to_bf16(acc[2 * e] / n), hi = f64_to_bf16(acc[2 * e + 1] / n);
      o[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(out + ((size_t)s * (size_t)m_max + (size_t)b) * D + piece * 8) = o;
  }
}

// Blocks [0, n_zero_blocks) clear the zero region (and the status words, if
// given); block n_zero_blocks + t pools
// query t's partial last block when its prefix does not end on a block boundary.
__global__ __launch_bounds__(256) void k_prepare(PrepArgs a, int n_zero_blocks) {
  if ((int)blockIdx.x < n_zero_blocks) {
    const size_t stride = (size_t)n_zero_blocks * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < a.zero_words; i += stride)
      a.zero[i] = 0u;
    if (a.status)
      for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < (size_t)a.nq; i += stride)
        a.status[i] = 0;
    return;
  }
  const int t = blockIdx.x - n_zero_blocks;
  if (!a.partial || t >= a.nq) return;
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  if (seq < 0 || seq >= a.n_seq || pos < 0 || pos >= a.l_max) return;
  const int64_t n = (pos + 1) % a.block;
  if (n == 0) return;
  const int64_t r0 = pos + 1 - n;
  const uint16_t* base = a.keys + ((size_t)seq * (size_t)a.l_max + (size_t)r0) * a.head_dim;
  // rows are read eight at a time (the loads in flight together), then added
  // in row order, so the float64 sum is the same as a row-by-row loop's
  for (int e = threadIdx.x; e < a.head_dim; e += 256) {
    double acc = 0.0;
    int64_t r = 0;
    for (; r + 8 <= n; r += 8) {
      uint16_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = base[(size_t)(r + u) * a.head_dim + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += bf16_to_f64(v[u]);
    }
    for (; r < n; ++r) acc += bf16_to_f64(base[(size_t)r * a.head_dim + e]);
    a.partial[(size_t)t * a.head_dim + e] = f64_to_bf16(acc / (double)n);
  }
}

// In-block prefix means of every position: one workgroup per block, one
// thread per dimension, a running float64 sum over the block's rows.
template <int D>
__global__ __launch_bounds__(D) void k_pool_prefix(const uint16_t* __restrict__ k, int64_t l_max,
                                                   int block, uint16_t* __restrict__ out) {
  const int64_t r0 = (int64_t)blockIdx.x * block;
  const int64_t r1 = (r0 + block) < l_max ? (r0 + block) : l_max;
  const int e = threadIdx.x;
  double acc = 0.0;
#pragma unroll 8
  for (int64_t r = r0; r < r1; ++r) {
    acc += bf16_to_f64(k[(size_t)r * D + e]);
    out[(size_t)r * D + e] = f64_to_bf16(acc / (double)(r - r0 + 1));
  }
}

}  // namespace

hipError_t launch_mean_pool(const uint16_t* k, int n_seq, int64_t l_max, int head_dim, int block,
                            uint16_t* out, hipStream_t stream) {
  const int64_t m_max = (l_max + block - 1) / block;
  const int64_t waves = (int64_t)n_seq * m_max;
  const int64_t grid = (waves + 3) / 4;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(k_mean_pool<128>, dim3((unsigned)grid), dim3(256), 0, stream, k, n_seq,
                       l_max, block, m_max, out);
  else if (head_dim == 64)
    hipLaunchKernelGGL(k_mean_pool<64>, dim3((unsigned)grid), dim3(256), 0, stream, k, n_seq,
                       l_max, block, m_max, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prepare(const PrepArgs& a, hipStream_t stream) {
  int nz = (int)((a.zero_words + 255) / 256);
  if (a.status && nz == 0) nz = 1;
  if (nz > 1024) nz = 1024;
  const int np = a.partial ? a.nq : 0;
  if (nz + np == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prepare, dim3(nz + np), dim3(256), 0, stream, a, nz);
  return hipGetLastError();
}

hipError_t launch_pool_prefix(const uint16_t* k, int64_t l_max, int head_dim, int block,
                              uint16_t* out, hipStream_t stream) {
  if (l_max <= 0) return hipSuccess;
  const int64_t nb = (l_max + block - 1) / block;
  if (head_dim == 128) hipLaunchKernelGGL(k_pool_prefix<128>, dim3(nb), dim3(128), 0, stream, k, l_max, block, out);
  else if (head_dim == 64) hipLaunchKernelGGL(k_pool_prefix<64>, dim3(nb), dim3(64), 0, stream, k, l_max, block, out);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsa
