// Internal (host-side) interface of the HISA kernels (k_hisa.hip) for the
// C-ABI layer.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// HISA: per query, block-pass workgroups score ch1 pooled blocks each and
// token-pass workgroups ch2 token items each (in one grid of `groups`
// workgroups per query that do both, or, with `split`, groups1 block-pass
// items then groups2 token-pass items), then one workgroup per query selects
// the top-k (see k_hisa.hip).
struct HisaArgs {
  const uint16_t* q;           // [nq, n_heads, D] bf16
  const float* w;              // [nq, n_heads]
  const uint16_t* keys;        // [n_seq, l_max, D] bf16
  const uint16_t* pooled;      // [n_seq, m_max, D] bf16
  const uint16_t* partial;     // [nq, D] pooled partial last block (prepare kernel)
  const int32_t* q_seq;        // [nq] or null
  const int32_t* q_pos;        // [nq]
  const int32_t* heads;        // [nq, heads_stride] routed heads (first h_use), or null: all
  int heads_stride, h_use;     // h_use = n_heads without routing
  // MISA routing inside the kernel (route_part non-null, heads null): every
  // workgroup adds the router's per-slice head sums [nq, route_splits,
  // n_heads] in slice order, I_j = |w_j| * sum, and keeps the h_use heads of
  // largest I (ties to the lower index); the first block-pass workgroup of a
  // query reports them (out_heads [nq, h_use], out_importance [nq, n_heads]).
  const float* route_part;
  int route_splits;
  int32_t* out_heads;
  float* out_importance;
  int nq, n_heads, head_dim, n_seq, block, m_blocks, top_k;
  int64_t l_max, m_max;
  int groups;                  // workgroups per query (both passes), or
  int split, groups1, groups2; // with split: block-pass / token-pass items per query
  int ch1, ch2;                // multiples of 32, <= kHisaMaxChunk
  int sblk_n;                  // LDS slots for block ids (>= ch2 / block + 2)
  // workspace
  uint32_t* sync;              // [nq, kHisaSyncWords]  (zeroed before the launch)
  int32_t* bflag;              // [nq, m_blocks] kept block + 1 (zeroed before the launch)
  uint2* cand1;                // [nq, g1, ch1] block candidates (g1 = groups, or groups1)
  uint32_t* cnt1;              // [nq, g1]
  uint32_t* keys2;             // [nq, g2 * ch2] token-pass score keys (g2 = groups, or groups2)
  int32_t* blocks;             // [nq, m_blocks] kept blocks (workspace or the caller's)
  // outputs
  int32_t* out_idx;            // [nq, top_k]
  float* out_score;            // [nq, top_k] or null
  float* out_block_score;      // [nq, m_blocks] or null
  int32_t* out_status;         // [nq] 0 = complete, 1 = a wait timed out (row padded), or null
  // longest wait of a token-pass workgroup for its query's block selection,
  // in ticks of the 100 MHz wall clock
  uint64_t spin_ticks;
};
// default bound of that wait: ~0.67 s
constexpr uint64_t kHisaSpinTicks = 1ull << 26;
constexpr int kHisaBins = 4096;
// per-query sync words: [0] block-pass workgroups arrived, [1] nonzero when a
// token-pass wait of the query timed out
constexpr int kHisaSyncWords = 2;
constexpr int kHisaSyncTimeout = 1;
constexpr int kHisaMaxGroups = 64;
constexpr int kHisaMaxChunk = 2048;
constexpr uint32_t kHisaListCap = 2048;
constexpr uint32_t kHisaCandCap = 2048;   // block candidates selected in LDS
constexpr int kHisaMaxBlocks = 1024;      // m_blocks of the one-kernel path
constexpr int kHisaRegKeys = 8192;        // token items per query (selected in LDS)
// LDS of one workgroup: keys [max(ch1, ch2)], histogram [bins + bins / 16],
// scan scratch [64],
// candidate offsets [g1 + 2] and counts [g1], block ids [sblk_n], the kept blocks and
// their scores [2 * m_blocks], then (8-byte aligned) the tie list
// [kHisaListCap], the brute-force tie slots [64] and the block candidates
// [kHisaCandCap] (pairs).
inline __host__ __device__ int hisa_list_offset_words(const HisaArgs& a) {
  const int g1 = a.split ? a.groups1 : a.groups;
  const int w = (a.ch1 > a.ch2 ? a.ch1 : a.ch2) + kHisaBins + kHisaBins / 16 + 64 + 2 * g1 + 2 +
                a.sblk_n + 2 * a.m_blocks;
  return (w + 1) & ~1;
}
inline size_t hisa_lds_bytes(const HisaArgs& a) {
  return (size_t)hisa_list_offset_words(a) * 4 + ((size_t)kHisaListCap + 64 + kHisaCandCap) * 8;
}
// LDS of the selection kernel (1024 threads): histogram [bins + bins / 4],
// scan scratch [64], kept blocks [m_blocks], then (8-byte aligned) the tie
// list [kHisaListCap], the brute-force tie slots [64], the output staging
// [kHisaCandCap] and the radix finish's spill [kHisaRegKeys] (pairs).
inline __host__ __device__ int hisa_topk_list_offset_words(const HisaArgs& a) {
  const int w = kHisaBins + kHisaBins / 4 + 64 + a.m_blocks;
  return (w + 1) & ~1;
}
inline size_t hisa_topk_lds_bytes(const HisaArgs& a) {
  return (size_t)hisa_topk_list_offset_words(a) * 4 +
         ((size_t)kHisaListCap + 64 + kHisaCandCap + kHisaRegKeys) * 8;
}
// k_hisa, then k_hisa_topk, on `stream`.
hipError_t launch_hisa(const HisaArgs& a, hipStream_t stream);

}  // namespace dsa
