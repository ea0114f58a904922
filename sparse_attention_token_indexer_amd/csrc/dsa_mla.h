// Sparse attention over the selected index list (the operator the indexer's
// output feeds): arguments and limits of the kernels in k_mla.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kMlaDqk = 576;     // latent row: 512 compressed key-value + 64 rotary values
constexpr int kMlaDv = 512;      // value = the first 512 values of the row
constexpr int kMlaTile = 32;     // selected rows per step
constexpr int kMlaMaxSplits = 16;
constexpr int kMlaMaxTiles = 64;     // steps per slice (the slice's row ids stay in LDS)
constexpr int kMlaMaxTopK = kMlaMaxSplits * kMlaMaxTiles * kMlaTile;

struct MlaArgs {
  const uint16_t* q;       // [nq, n_heads, kMlaDqk] bf16
  const uint16_t* kv;      // [n_seq, l_max, kMlaDqk] bf16 latent cache
  const int32_t* q_seq;    // [nq] cache of each query, or null: cache 0
  const int32_t* q_pos;    // [nq] position of each query (prefix = 0..pos)
  const int32_t* idx;      // [nq, top_k] selected rows; entries outside the prefix are skipped
  int nq, n_heads, n_seq, top_k;
  int splits, tiles_per_split;   // the list of each query in `splits` slices of tiles
  int64_t l_max;
  float scale_log2;        // softmax scale * log2(e)
  uint16_t* out;           // [nq, n_heads, kMlaDv] bf16
  uint16_t* part_o;        // [nq, splits, n_heads, kMlaDv] bf16 slices, each divided by its
                           // own sum (splits > 1)
  float2* part_ml;         // [nq, splits, n_heads] (running max in log2 units, sum)
};

// LDS of the attention kernel: three steps of staged rows (32 rows of
// kMlaDqk bf16 each, unpadded: the rows' chunks are swizzled instead), the
// partial score blocks of its waves (4 KiB per wave: 2 per group of 32 heads,
// two groups when 64 divides n_heads), a flag word (and padding), and the
// slice's row ids.
inline size_t mla_lds_bytes(int n_heads, int tiles_per_split) {
  const int waves = n_heads % 64 == 0 ? 4 : 2;
  return (size_t)3 * kMlaTile * kMlaDqk * 2 + (size_t)waves * 4096 + 16 +
         (size_t)tiles_per_split * kMlaTile * 4;
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream);

}  // namespace dsa
