// Per-wave scorers: each computes the indexer score of 32 keys for one query,
//   s(u) = sum_j w_j * max(0, q_j . k_u)
// (MISA summary, "problem" section: every prefix token is scored through the
// H_I-head indexer; signed heads per the DoSA review, section 3).
//
// Layout facts (gfx950 MFMA, checked on hardware):
//  32x32x16 bf16: lane l holds A[l%32][8*(l/32)+e], B[8*(l/32)+e][l%32];
//                 accumulator r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
//  16x16x32 bf16: lane l holds A[l%16][8*(l/16)+e], B[8*(l/16)+e][l%16];
//                 accumulator r of lane l is D[4*(l/16) + r][l%16].
// Heads are the MFMA rows (A = q), keys the columns (B = k).  The order in which
// the head dimension is fed to the contraction is free (it is a sum): at k-step
// s the two lane halves (or four lane groups) take adjacent 16-byte pieces of
// the key row, so each load instruction reads 32 (64) contiguous bytes of every
// key and the cache lines of a tile are consumed by consecutive instructions.
//
// After score() every lane holds the score of tile key (lane & 31).
#pragma once
#include "dsa_common.h"

namespace dsa {

// H_use <= 32 * HT heads on 32x32x16 MFMAs (HT = 1 or 2), head dim D.
template <int HT, int D>
struct ScorerMfma32 {
  static constexpr int kRows = 1;     // key rows loaded per lane per tile
  static constexpr int S = D / 16;    // k-steps
  static constexpr int kLdsFloats = 0;
  typedef bf16x8 Frag[S];

  bf16x8 qa[HT][S];
  float W[HT];   // row-broadcast weights (see weighted_relu_sum)

  DSA_DEVICE static int row_key(int) { return lane_id() & 31; }

  // (both head-list reads come first, then the weight and query loads with no
  // wait between them)
  DSA_DEVICE void init(const uint16_t* q_t, const float* w_t, const int32_t* heads_t,
                       int h_use, float*) {
    const int lane = lane_id(), m = lane & 31, h = lane >> 5;
    int wsel[HT], qsel[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      // lane 16*g + r: the head slot that accumulator register r holds in
      // lanes of row group g (lane half g/2 = h)
      const int r = lane & 15;
      const int rs = ht * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const int slot = ht * 32 + m;
      wsel[ht] = rs < h_use ? (heads_t ? heads_t[rs] : rs) : -1;
      qsel[ht] = slot < h_use ? (heads_t ? heads_t[slot] : slot) : -1;
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      W[ht] = wsel[ht] >= 0 ? w_t[wsel[ht]] : 0.f;
      const uint16_t* src = q_t + (size_t)(qsel[ht] >= 0 ? qsel[ht] : 0) * D + 8 * h;
#pragma unroll
      for (int s = 0; s < S; ++s) qa[ht][s] = qsel[ht] >= 0 ? load_bf16x8(src + 16 * s) : zero_bf16x8();
    }
  }

  DSA_DEVICE static void load(Frag& b, const uint16_t* const* rows) {
    const uint16_t* src = rows[0] + (lane_id() >> 5) * 8;
#pragma unroll
    for (int s = 0; s < S; ++s) b[s] = load_bf16x8(src + 16 * s);
  }

  DSA_DEVICE float score(const Frag& b) const {
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
    const float p = weighted_relu_sum<HT>(acc, W, std::make_integer_sequence<int, 16>{});
    // the two lane halves' partials of key lane%32 meet in one add (a lane
    // half swap keeps this off the LDS queue)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p),
                                                     false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
};

// H_use <= 16 heads on 16x16x32 MFMAs; two 16-key column blocks per 32-key tile.
template <int D>
struct ScorerMfma16 {
  static constexpr int kRows = 2;
  static constexpr int S = D / 32;
  static constexpr int kLdsFloats = 0;
  typedef bf16x8 Frag[2][S];

  bf16x8 qa[S];
  float wr[4];

  DSA_DEVICE static int row_key(int r) { return r * 16 + (lane_id() & 15); }

  DSA_DEVICE void init(const uint16_t* q_t, const float* w_t, const int32_t* heads_t,
                       int h_use, float*) {
    const int lane = lane_id(), m = lane & 15, g = lane >> 4;
    // head-list reads first, then the loads (see ScorerMfma32::init)
    int wsel[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int rs = 4 * g + r;
      wsel[r] = rs < h_use ? (heads_t ? heads_t[rs] : rs) : -1;
    }
    const int qsel = m < h_use ? (heads_t ? heads_t[m] : m) : -1;
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[r] = wsel[r] >= 0 ? w_t[wsel[r]] : 0.f;
    const uint16_t* src = q_t + (size_t)(qsel >= 0 ? qsel : 0) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < S; ++s) qa[s] = qsel >= 0 ? load_bf16x8(src + 32 * s) : zero_bf16x8();
  }

  DSA_DEVICE static void load(Frag& b, const uint16_t* const* rows) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint16_t* src = rows[c] + 8 * g;
#pragma unroll
      for (int s = 0; s < S; ++s) b[c][s] = load_bf16x8(src + 32 * s);
    }
  }

  DSA_DEVICE float score(const Frag& b) const {
    float p[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], b[c][s], acc, 0, 0, 0);
      float x = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) x = __builtin_fmaf(wr[r], relu(acc[r]), x);
      x += shfl_xor_f(x, 16);
      x += shfl_xor_f(x, 32);
      p[c] = x;
    }
    return ((lane_id() >> 4) & 1) ? p[1] : p[0];
  }

  // squared norm of the key that score() returns the score of in this lane:
  // its values are spread over the four lane groups (lanes m + 16 g)
  DSA_DEVICE static float norm2(const Frag& b) {
    float p[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float x = 0.f;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = (float)b[c][s][e];
          x = __builtin_fmaf(v, v, x);
        }
      x += shfl_xor_f(x, 16);
      x += shfl_xor_f(x, 32);
      p[c] = x;
    }
    return ((lane_id() >> 4) & 1) ? p[1] : p[0];
  }
};

// float32 inputs on the vector ALUs (any H_use <= 64, D = 64 or 128): the
// query rows live in LDS and are read by broadcast; lane (n, h) owns key n and
// the half h of its head dimension.
template <int D>
struct ScorerF32 {
  static constexpr int kRows = 1;
  static constexpr int kLdsFloats = 64 * D + 64;
  typedef float Frag[D / 2];

  const float* sq;   // LDS [h_use][D]
  const float* sw;   // LDS [h_use]
  int h_use;

  DSA_DEVICE static int row_key(int) { return lane_id() & 31; }

  // Collective over the workgroup: copies the (possibly gathered) query rows
  // and weights into LDS.  Callers follow it with a barrier.
  DSA_DEVICE void init(const uint16_t* q_raw, const float* w_t, const int32_t* heads_t,
                       int h, float* lds) {
    const float* q_t = reinterpret_cast<const float*>(q_raw);
    h_use = h;
    float* q_l = lds;
    float* w_l = lds + 64 * D;
    for (int i = threadIdx.x; i < h * D; i += blockDim.x) {
      int slot = i / D, e = i % D;
      int head = heads_t ? heads_t[slot] : slot;
      q_l[i] = q_t[(size_t)head * D + e];
    }
    for (int i = threadIdx.x; i < h; i += blockDim.x) w_l[i] = w_t[heads_t ? heads_t[i] : i];
    sq = q_l;
    sw = w_l;
  }

  DSA_DEVICE static void load(Frag& b, const uint16_t* const* rows) {
    const float* src = reinterpret_cast<const float*>(rows[0]) + (lane_id() >> 5) * (D / 2);
#pragma unroll
    for (int e = 0; e < D / 2; e += 4) {
      f32x4 v = *reinterpret_cast<const f32x4*>(src + e);
      b[e] = v[0]; b[e + 1] = v[1]; b[e + 2] = v[2]; b[e + 3] = v[3];
    }
  }

  DSA_DEVICE float score(const Frag& b) const {
    const int h = lane_id() >> 5;
    float p = 0.f;
    for (int j = 0; j < h_use; ++j) {
      const float* qj = sq + j * D + h * (D / 2);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < D / 2; ++e) d = __builtin_fmaf(qj[e], b[e], d);
      d += shfl_xor_f(d, 32);
      p = __builtin_fmaf(sw[j], relu(d), p);
    }
    return p;
  }
};

}  // namespace dsa
