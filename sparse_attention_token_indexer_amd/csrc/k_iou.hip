// Per-query IoU of two token selections: |A & B| / |A | B| over the non-padding
// (>= 0) indices; two empty selections give 1.  The MISA summary ("results")
// and the HISA review (section 3) report selection agreement with the dense
// indexer as this IoU.  Selections hold no duplicates (they are top-k sets).
//
// One workgroup per query: A is bitonic-sorted in LDS, every entry of B is
// found by binary search.
#include "dsa_internal.h"
#include "dsa_common.h"

namespace dsa {

namespace {

constexpr int kIT = 256;
constexpr int kMaxK = 8192;

__global__ __launch_bounds__(kIT) void k_iou(const int32_t* __restrict__ A,
                                             const int32_t* __restrict__ B, int k,
                                             float* __restrict__ out) {
  __shared__ int32_t s[kMaxK];
  __shared__ uint32_t s_na, s_nb, s_hit;
  const int t = blockIdx.x;
  int P = 1;
  while (P < k) P <<= 1;
  if (threadIdx.x == 0) { s_na = 0; s_nb = 0; s_hit = 0; }
  for (int i = threadIdx.x; i < P; i += kIT) {
    int32_t v = i < k ? A[(size_t)t * k + i] : -1;
    s[i] = v >= 0 ? v : 0x7FFFFFFF;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P; i += kIT) {
        int j = i ^ stride;
        if (j > i) {
          bool up = (i & size) == 0;
          int32_t x = s[i], y = s[j];
          if ((x > y) == up) { s[i] = y; s[j] = x; }
        }
      }
      __syncthreads();
    }
  }
  uint32_t na = 0, nb = 0, hit = 0;
  for (int i = threadIdx.x; i < k; i += kIT) {
    if (A[(size_t)t * k + i] >= 0) ++na;
    int32_t v = B[(size_t)t * k + i];
    if (v < 0) continue;
    ++nb;
    int lo = 0, hi = P;
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (s[mid] < v) lo = mid + 1; else hi = mid;
    }
    if (lo < P && s[lo] == v) ++hit;
  }
  atomicAdd(&s_na, na);
  atomicAdd(&s_nb, nb);
  atomicAdd(&s_hit, hit);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t uni = s_na + s_nb - s_hit;
    out[t] = uni ? (float)s_hit / (float)uni : 1.0f;
  }
}

}  // namespace

hipError_t launch_iou(const int32_t* a, const int32_t* b, int nq, int k, float* out,
                      hipStream_t stream) {
  if (k > kMaxK) return hipErrorInvalidValue;
  if (nq == 0) return hipSuccess;
  hipLaunchKernelGGL(k_iou, dim3(nq), dim3(kIT), 0, stream, a, b, k, out);
  return hipGetLastError();
}

}  // namespace dsa
