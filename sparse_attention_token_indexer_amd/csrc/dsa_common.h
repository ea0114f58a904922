// Shared device helpers for the gfx950 DSA indexer kernels.
//
// Score keys: every fp32 score is carried as an order-preserving uint32 "key"
// (larger key = larger score), with -0.0 folded onto +0.0 so both compare
// equal.  Key 0 is below the key of -inf and marks an empty / invalid slot.
// Selections order entries by the 64-bit composite (key << 32) | ~id, so that
// among equal scores the lower id ranks first (lower index wins ties).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#define DSA_DEVICE __device__ __forceinline__

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace dsa {

constexpr int kWave = 64;
constexpr int kBinBits = 12;             // first-level histogram: top 12 key bits
constexpr int kBins = 1 << kBinBits;     // 4096
constexpr int kBinShift = 32 - kBinBits;

DSA_DEVICE uint32_t score_to_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b << 1) == 0u) b = 0u;            // -0.0 -> +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// score_to_key without the -0.0 fold, for scores that cannot be -0.0 (sums
// w * max(0, x) started from +0.0 never are); equal to score_to_key on them.
DSA_DEVICE uint32_t fast_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

DSA_DEVICE float key_to_score(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

DSA_DEVICE uint64_t composite(uint32_t key, int32_t id) {
  return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)id);
}

// max(0, x) in one integer max on the IEEE bit pattern: every negative value
// (sign bit set, -0.0 included) compares below 0 and becomes +0.0, every
// positive value keeps its bits.  (The float max would first canonicalise x.)
DSA_DEVICE float relu(float x) {
  return __int_as_float(__builtin_elementwise_max(__float_as_int(x), 0));
}

// p + W[16*(lane/16) + R] * x: the weight comes from lane R of the lane's own
// 16-lane row (DPP row_newbcast on the first operand), so one VGPR carries 16
// per-row constants for each of the four rows.  Register operands only.
template <int R>
DSA_DEVICE float fmac_rowbcast(float p, float W, float x) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(p)
      : "v"(W), "v"(x), "n"(R));
  return p;
}

// W[16*(lane/16) + R] * x (the first term of a row-broadcast sum; -0.0 when W
// is negative and x is +0.0).
template <int R>
DSA_DEVICE float fmul_rowbcast(float W, float x) {
  float p;
  asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "=v"(p)
      : "v"(W), "v"(x), "n"(R));
  return p;
}

// sum over head tiles ht and accumulator registers r of w(ht, r) * max(0, acc),
// where W[ht] holds, in lane 16*g + r, the weight of the head that register r
// holds in lanes of row group g (see the MFMA layouts in dsa_scorers.h).
template <int HT, int... R>
DSA_DEVICE float weighted_relu_sum(const f32x16 (&acc)[HT], const float (&W)[HT],
                                   std::integer_sequence<int, R...>) {
  float p = 0.f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) ((p = fmac_rowbcast<R>(p, W[ht], relu(acc[ht][R]))), ...);
  return p;
}

template <int N, class F, int... I>
DSA_DEVICE void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// f(integral_constant<0>) .. f(integral_constant<N-1>), in order (unrolled
// steps whose register indices must be compile-time constants)
template <int N, class F>
DSA_DEVICE void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP: shifts by 1, 2, 4
// and 8 lanes within each 16-lane row, then row 0's total added into row 1 and
// row 2's into row 3 (row_bcast:15), then rows 0-1's into rows 2-3
// (row_bcast:31).  Lanes whose source is outside the row read 0.
DSA_DEVICE uint32_t wave_incl_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return (uint32_t)v;
}

// Wave-wide sum / exchange helpers (wave64).
DSA_DEVICE float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

DSA_DEVICE int lane_id() { return (int)(threadIdx.x & 63); }
DSA_DEVICE int wave_id() { return (int)(threadIdx.x >> 6); }

// 16-byte global load of 8 bf16 values.
DSA_DEVICE bf16x8 load_bf16x8(const uint16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

DSA_DEVICE bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// Block-wide exclusive scan helpers over NT threads using LDS scratch[NT/64 + 1].
template <int NT>
DSA_DEVICE uint32_t block_exclusive_sum(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = lane_id(), wv = wave_id();
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wv] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    uint32_t s = scratch[i];
    if (i < wv) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Given a histogram hist[0..nbins) (counts of entries per digit, larger digit =
// better) and need >= 1, find the digit d* such that the number of entries with
// digit > d* is < need <= the number with digit >= d*.  Returns d* and writes
// the count strictly above it to *above.  All threads get the result.
// If the histogram holds fewer than need entries in total, d* = 0 and *above =
// total - hist[0] (caller must avoid this case).
template <int NT>
DSA_DEVICE int block_find_threshold(const uint32_t* hist, int nbins, uint32_t need,
                                    uint32_t* scratch, uint32_t* above) {
  // each thread owns a contiguous run of bins, counted from the top
  const int per = (nbins + NT - 1) / NT;
  const int t = threadIdx.x;
  // thread t owns bins [nbins-1 - t*per - (per-1), nbins-1 - t*per] (top down)
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) {
    int b = nbins - 1 - (t * per + i);
    if (b >= 0) mine += hist[b];
  }
  uint32_t tot;
  uint32_t before = block_exclusive_sum<NT>(mine, scratch, &tot);  // entries in higher bins
  __shared__ int s_d;
  __shared__ uint32_t s_above;
  if (t == 0) { s_d = 0; s_above = tot - hist[0]; }
  __syncthreads();
  if (before < need && before + mine >= need) {
    uint32_t acc = before;
    for (int i = 0; i < per; ++i) {
      int b = nbins - 1 - (t * per + i);
      if (b < 0) break;
      uint32_t h = hist[b];
      if (acc + h >= need) { s_d = b; s_above = acc; break; }
      acc += h;
    }
  }
  __syncthreads();
  *above = s_above;
  int d = s_d;
  __syncthreads();
  return d;
}

}  // namespace dsa
