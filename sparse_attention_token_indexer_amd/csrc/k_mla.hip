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
// One workgroup = one query x one slice of its list x one block of 32 G heads
// (G = 2 when 64 divides the head count, else 1), with 2 G waves: the two
// waves kh = 0, 1 of a group of 32 heads split the work in halves.  Wave kh
// forms the partial scores S^T (32 rows x 32 heads) over value entries
// [256 kh, 256 kh + 256) and rotary entries [32 kh, 32 kh + 32) on 32x32x16
// bf16 MFMAs (that part of its heads' query rows stays in registers); the two
// partial blocks are exchanged through LDS and added in both waves (the same
// sum in either order); both waves run the same softmax, and wave kh
// accumulates O^T for value columns [256 kh, 256 kh + 256).  With one wave per
// SIMD each wave has 512 registers.  The head blocks of one (query, slice)
// run on one XCD (workgroup ids 8 apart), so the rows that one gathers reach
// the others from that XCD's L2.
//
// Per step the workgroup gathers 32 listed rows straight into LDS (direct
// 16-byte loads, no register staging; three steps in flight): per row one
// wave-wide load of its 512 value entries from the row's address in scalar
// registers, and per 8 rows one wave-wide load of their 64 rotary entries.  Chunks
// are XOR-swizzled inside each staged row so that both operand reads are free
// of bank conflicts.  The value operand comes from the row-major stage
// through the transposing LDS read (each 16-lane group: 4 rows x 16 columns,
// lane i receiving column i of the 4 rows), in the row order in which the
// lane's probabilities sit.
//
// Softmax reference: each head's probabilities are 2^(x - m) for a fixed
// reference m, its first step's largest score (log2 units), so the
// accumulators are only ever written by MFMAs.  The result, a ratio, does not
// depend on m.  Should a later score exceed m by more than 64 (probabilities
// could overflow), the slice is redone: one pass for every head's largest
// score, then the pass again with that as m.  Probabilities are rounded to
// bf16 for the value product (the sum in the denominator is kept in float32).
// A query whose list is split writes its slices normalised by their own sums,
// with (reference, sum), and a second kernel merges them; slices are stored in
// bf16 (relative 2^-9, like the output itself).
#include "dsa_common.h"
#include "dsa_mla.h"

namespace dsa {

namespace {

typedef __attribute__((address_space(3))) void* lds_vp;
typedef __attribute__((address_space(1))) void* glb_vp;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kRowB = kMlaDqk * 2;                // bytes per latent row (1152)
constexpr int kVCh = kMlaDv / 8;                  // value chunks per row (64)
constexpr int kRCh = (kMlaDqk - kMlaDv) / 8;      // rotary chunks per row (8)
constexpr int kRopeOff = kMlaTile * kVCh * 16;    // rotary region of a stage (32 KiB in)
constexpr int kStageB = kMlaTile * kRowB;         // bytes per stage (36864)
constexpr int kVKS = kMlaDv / 2 / 16;             // value k-steps per wave (16)
constexpr int kKS = kMlaDqk / 2 / 16;             // all k-steps per wave (18)
constexpr int kVB = kMlaDv / 2 / 32;              // 32-column blocks per wave (8)
constexpr float kOverflow = 64.f;                 // largest score above the reference (log2)
static_assert(kVCh == 64 && kRCh == 8 && kMlaTile == 32, "layout");

// The stand-in for rows outside a list: a latent row of zeros (never written).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kRowB];

// Value chunk c of staged row r sits at slot c ^ sv(r) of the row's 64 (a
// permutation inside aligned groups of 16 chunks; rows are 1 KiB apart, so
// slot mod 16 is the chunk's bank quad).  sv is a bijection on the rows' low 4
// bits (score operand: rows 16 h + 0..15, one chunk), and for the rows r0 +
// 0..3 (4 | r0) it sets bits 2-3 of the slot from the row while bits 0-1 keep
// the chunk's (value operand: 4 rows x an aligned quad of chunks).
DSA_DEVICE int sv(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Rotary chunk c of row r sits at slot c ^ sr(r) of the row's 8 (rows 128 B
// apart: rows of one parity share a half of the bank quads, and sr takes 8
// values over the 8 rows of each parity in any aligned 16).
DSA_DEVICE int sr(int r) { return (r >> 1) & 7; }

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLds = 0xC07F;                  // lgkmcnt(0)

// Workgroup barrier after this wave's LDS accesses are done.  Unlike
// __syncthreads it does not wait for the direct loads in flight: the loop
// waits for the ones it needs by count.
DSA_DEVICE void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLds);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

DSA_DEVICE float pair_half(float x, bool sum) {     // x combined with lane ^ 32's
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  const float a = __uint_as_float(sw[0]), b = __uint_as_float(sw[1]);
  return sum ? a + b : fmaxf(a, b);
}

// a wave-uniform address held in scalar registers (so that a load takes it
// as its base and the lane part as a 32-bit offset)
DSA_DEVICE const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

DSA_DEVICE i16x4 read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds_vp)p);
}

template <int G>
__global__ __launch_bounds__(128 * G) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_sparse_mla(MlaArgs a) {
  constexpr int NW = 2 * G, NT = 64 * NW;
  constexpr int RPW = kMlaTile / NW;                       // rows per wave per step
  constexpr int RRW = RPW / 8;                             // rotary loads per wave per step
  static_assert(kMlaTile % (8 * NW) == 0, "rows per wave");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* stage = smem;                                                 // [3][kStageB]
  float* xs = reinterpret_cast<float*>(smem + 3 * kStageB);              // [NW][16][64]
  int32_t* s_flag = reinterpret_cast<int32_t*>(xs + NW * 16 * 64);       // [4]
  int32_t* sid = s_flag + 4;                                             // [slice rows]

  // workgroup -> (query, slice, head block): the head blocks of a (query,
  // slice) take ids 8 apart (one XCD)
  const int hbn = a.n_heads / (32 * G);
  const int bx = (int)blockIdx.x, y8 = bx >> 3;
  const int hb = y8 % hbn;
  const int pair = (y8 / hbn) * 8 + (bx & 7);
  if (pair >= a.nq * a.splits) return;
  const int t = pair / a.splits, sp = pair - t * a.splits;
  // (the wave index in a scalar register: everything derived from it is
  // wave-uniform to the compiler)
  const int tid = (int)threadIdx.x, lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const int kh = wv & 1, kg = lane >> 5, n = lane & 31;
  const int head = 32 * G * hb + 32 * (wv >> 1) + n;
  const int seq = a.q_seq ? a.q_seq[t] : 0;
  const int64_t pos = a.q_pos[t];
  const bool ok = seq >= 0 && seq < a.n_seq && pos >= 0 && pos < a.l_max;
  const int T = a.tiles_per_split;
  const int n_tok = T * kMlaTile;
  const int base = sp * n_tok;

  // the slice's row ids (-1: skipped)
  if (tid == 0) s_flag[0] = 0;
  for (int i = tid; i < n_tok; i += NT) {
    const int j = base + i;
    const int e = j < a.top_k ? a.idx[(size_t)t * a.top_k + j] : -1;
    sid[i] = (ok && e >= 0 && (int64_t)e <= pos) ? e : -1;
  }
  // this wave's part of its heads' query rows, the B operand of the score
  // product (lane (head n, kg)): value entries 256 kh + 16 s + 8 kg .., then
  // rotary entries 512 + 32 kh + 16 s' + 8 kg ..
  bf16x8 qb[kKS];
  {
    const uint16_t* qr = a.q + ((size_t)t * a.n_heads + head) * kMlaDqk + 8 * kg;
#pragma unroll
    for (int s = 0; s < kKS; ++s)
      qb[s] = load_bf16x8(qr + (s < kVKS ? 256 * kh + 16 * s : kMlaDv + 32 * kh + 16 * (s - kVKS)));
  }
  __syncthreads();

  // One step's rows into stage buffer tile % 3: wave wv loads the value
  // chunks of rows r = wv, wv + NW, .., one wave-wide load each (lane l fills
  // slot l with chunk l ^ sv(r)), and the rotary chunks of RRW groups of 8
  // rows.  Rows outside the list load a row of zeros; every load is issued,
  // so the counted waits are exact.
  const uint8_t* kv_seq = reinterpret_cast<const uint8_t*>(a.kv) +
                          (size_t)(ok ? seq : 0) * (size_t)a.l_max * kRowB;
  // the wave's row ids of a step in one LDS read (lane j: row wv + j NW)
  auto row_ids = [&](int tile) {
    return sid[tile * kMlaTile + wv + (lane < RPW ? lane : 0) * NW];
  };
  // value chunks of row wv + j NW (one wave-wide load, the row's address in
  // scalar registers)
  auto issue_row = [&](int idv, int j, uint8_t* dst) {
    const int r = wv + j * NW;
    const int e = __builtin_amdgcn_readlane(idv, j);
    const uint8_t* row = uniform_ptr(e >= 0 ? kv_seq + (size_t)e * kRowB : g_zero_row);
    __builtin_amdgcn_global_load_lds((glb_vp)(row + ((uint32_t)(lane ^ sv(r)) << 4)),
                                     (lds_vp)(dst + 1024 * r), 16, 0, 0);
  };
  // rotary chunks of rows 8 (RRW wv + k) + l / 8 (lane l: slot l % 8, chunk
  // (l % 8) ^ sr(row)), one wave-wide load per 8 rows
  auto issue_rope = [&](int tile, int k, uint8_t* dst) {
    const int rr = 8 * (RRW * wv + k) + (lane >> 3);
    const int e = sid[tile * kMlaTile + rr];
    const uint8_t* src = (e >= 0 ? kv_seq + (size_t)e * kRowB : g_zero_row) + kMlaDv * 2 +
                         (((lane & 7) ^ sr(rr)) << 4);
    __builtin_amdgcn_global_load_lds((glb_vp)src, (lds_vp)(dst + kRopeOff + 1024 * (RRW * wv + k)),
                                     16, 0, 0);
  };
  auto issue = [&](int tile, int b) {
    const int idv = row_ids(tile);
#pragma unroll
    for (int j = 0; j < RPW; ++j) issue_row(idv, j, stage + b * kStageB);
#pragma unroll
    for (int k = 0; k < RRW; ++k) issue_rope(tile, k, stage + b * kStageB);
  };
  // this step's rows have landed (the next step's may still be in flight)
  auto wait_step = [&](int tile) {
    if (tile + 1 < T) __builtin_amdgcn_s_waitcnt(wait_vm(RPW + RRW));
    else __builtin_amdgcn_s_waitcnt(wait_vm(0));
    lds_barrier();
  };
  float* xw = xs + wv * 1024;
  const float* xp = xs + (wv ^ 1) * 1024;
  // the lane's 16 full scores of a step (rows 8 (i / 4) + 4 kg + i % 4, head
  // n; rows outside the list: -inf), unscaled, and the head's largest; stage
  // buffer b holds the step's rows
  auto step_scores = [&](int tile, int b, float (&x)[16]) {
    const uint8_t* st = stage + b * kStageB;
    // the loads of step tile + 2 (into the buffer that step tile - 1 used)
    // are issued between the MFMAs below
    const bool more = tile + 2 < T;
    const int idn = more ? row_ids(tile + 2) : 0;
    uint8_t* dn = stage + (b == 0 ? 2 : b - 1) * kStageB;
    // value chunk 32 kh + 2 s + kg of row n at slot ((2 s + kg) ^ sv(n)) +
    // 32 kh (8 lane addresses for s % 8, the rest immediate); rotary chunk
    // 4 kh + 2 s' + kg at slot that ^ sr(n).  Operands are read kPre k-steps
    // ahead.
    constexpr int kPre = 4;
    const uint8_t* vrow = st + n * 1024 + 512 * kh;
    const int wsv = (sv(n) ^ kg) << 4;
    const uint8_t* rrow = st + kRopeOff + n * 128;
    auto a_of = [&](int s) {
      if (s < kVKS)
        return *reinterpret_cast<const bf16x8*>(vrow + ((32 * (s & 7)) ^ wsv) + 256 * (s >> 3));
      const int c = 4 * kh + 2 * (s - kVKS) + kg;
      return *reinterpret_cast<const bf16x8*>(rrow + ((c ^ sr(n)) << 4));
    };
    auto sphase = [&](auto MORE) {
      constexpr bool kMore = decltype(MORE)::value;
      f32x16 acc_s;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_s[r] = 0.f;
      bf16x8 av[kPre];
#pragma unroll
      for (int s = 0; s < kPre; ++s) av[s] = a_of(s);
#pragma unroll
      for (int s = 0; s < kKS; ++s) {
        const bf16x8 cur = av[s % kPre];
        if (s + kPre < kKS) av[s % kPre] = a_of(s + kPre);
        acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qb[s], acc_s, 0, 0, 0);
        if (kMore && s < RPW) issue_row(idn, s, dn);
        if (kMore && s >= RPW && s < RPW + RRW) issue_rope(tile + 2, s - RPW, dn);
      }
      // keep that order: the first reads, then each MFMA followed by a read
      // (and a row's loads)
      __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
      for (int s = 0; s < kKS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s + kPre < kKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (kMore && s < RPW + RRW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      return acc_s;
    };
    const f32x16 sacc = more ? sphase(std::true_type{}) : sphase(std::false_type{});
    // partial blocks through LDS as [4][64 lanes][4 floats] (16-byte accesses)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f32x4*>(xw + i * 256 + 4 * lane) =
          f32x4{sacc[4 * i], sacc[4 * i + 1], sacc[4 * i + 2], sacc[4 * i + 3]};
    lds_barrier();
    const uint32_t vmask =
        (uint32_t)__ballot(lane < 32 && sid[tile * kMlaTile + (lane & 31)] >= 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(xp + q * 256 + 4 * lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * q + r] = sacc[4 * q + r] + o[r];
    }
    if (vmask != 0xFFFFFFFFu) {                  // (wave-uniform; rare)
      const uint32_t lm = vmask >> (4 * kg);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!((lm >> (8 * (i >> 2) + (i & 3))) & 1u)) x[i] = -__builtin_inff();
    }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
    return pair_half(mx, false);
  };

  f32x16 acc[kVB];
  float m_ref = -__builtin_inff(), l_run = 0.f;
  // value operand (transposing read): lane 4 e + q of 16-lane group g
  // addresses row 16 s + 4 kg + e (+ 8), columns 256 kh + 32 d + 16 (g & 1) +
  // 4 q, i.e. chunk 32 kh + 4 d + cc (cc = 2 (g & 1) + q / 2) at slot
  // ((4 d + cc) ^ sv(row)) + 32 kh, where sv(row) = 4 e + kg (+ 2 for the rows
  // 8 further on)
  const int ve = (lane & 15) >> 2;
  const int vcc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vlo_off = (4 * kg + ve) * 1024 + 512 * kh + 8 * (lane & 1);
  const int slo = (vcc ^ (4 * ve + kg)) << 4, shi = (vcc ^ (4 * ve + kg + 2)) << 4;

  // FIXED: the reference is given (m_ref); otherwise it is each head's first
  // step's largest score, and a score beyond the reference by more than
  // kOverflow (log2 units) flags the workgroup.  References are kept in raw
  // score units: p = 2^(scale_log2 (x - m_ref)).
  const float sl = a.scale_log2;
  const float m_over = kOverflow / sl;
  auto full_pass = [&](bool fixed) {
#pragma unroll
    for (int d = 0; d < kVB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
    l_run = 0.f;
    issue(0, 0);
    if (T > 1) issue(1, 1);
    int b = 0;                                   // stage buffer of the step (tile % 3)
    for (int tile = 0; tile < T; ++tile) {
      b = __builtin_amdgcn_readfirstlane(b);
      wait_step(tile);
      float x[16];
      const float mx = step_scores(tile, b, x);
      if (!fixed) {
        if (m_ref == -__builtin_inff()) m_ref = mx;
        else if (mx > m_ref + m_over) s_flag[0] = 1;
      }
      bf16x8 pb[2];
      float ps = 0.f;
      const float c0 = m_ref == -__builtin_inff() ? 0.f : -sl * m_ref;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // (v_exp_f32: results below 2^-126 flush to zero, which only drops
        // rows weighing less than that against the reference; before the
        // first listed row m_ref is -inf and every x is -inf: p = 0)
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl, c0));
        ps += p;
        pb[i >> 3][i & 7] = (__bf16)p;
      }
      l_run += ps;
      // O^T += V^T P^T: MFMA k-slot 8 kg + j holds step row 16 s + 8 (j / 4)
      // + 4 kg + j % 4, where the lane's probabilities pb[s][j] sit
      // (k-step s outer, value block d inner: consecutive MFMAs are
      // independent; operands read kPre MFMAs ahead)
      const uint8_t* vlo = stage + b * kStageB + vlo_off;
      constexpr int kPre = 4;
      auto v_of = [&](int i) {                    // operand of MFMA i = 8 s + d
        const int s = i / kVB, d = i % kVB;
        const int rs = 16 * s * 1024;
        const i16x4 lo = read_tr(vlo + rs + ((64 * d) ^ slo));
        const i16x4 hi = read_tr(vlo + 8 * 1024 + rs + ((64 * d) ^ shi));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vv[kPre];
#pragma unroll
      for (int i = 0; i < kPre; ++i) vv[i] = v_of(i);
#pragma unroll
      for (int i = 0; i < 2 * kVB; ++i) {
        const bf16x8 cur = vv[i % kPre];
        if (i + kPre < 2 * kVB) vv[i % kPre] = v_of(i + kPre);
        acc[i % kVB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pb[i / kVB], acc[i % kVB], 0,
                                                              0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);
#pragma unroll
      for (int i = 0; i < 2 * kVB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kPre < 2 * kVB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      b = b == 2 ? 0 : b + 1;
    }
  };
  full_pass(false);
  lds_barrier();
  if (s_flag[0]) {
    // every head's largest score over the slice, then the pass again with it
    m_ref = -__builtin_inff();
    issue(0, 0);
    if (T > 1) issue(1, 1);
    int b = 0;
    for (int tile = 0; tile < T; ++tile) {
      b = __builtin_amdgcn_readfirstlane(b);
      wait_step(tile);
      float x[16];
      m_ref = fmaxf(m_ref, step_scores(tile, b, x));
      b = b == 2 ? 0 : b + 1;
    }
    lds_barrier();
    full_pass(true);
  }

  // the head's sum over both halves of the rows
  const float l = pair_half(l_run, true);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t slot = ((size_t)t * a.splits + sp) * a.n_heads + head;
  uint16_t* o = (a.splits == 1 ? a.out + ((size_t)t * a.n_heads + head) * kMlaDv
                               : a.part_o + slot * kMlaDv) + 256 * kh + 4 * kg;
#pragma unroll
  for (int d = 0; d < kVB; ++d)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)(acc[d][4 * q + r] * inv);
      *reinterpret_cast<bf16x4*>(o + 32 * d + 8 * q) = v;
    }
  if (a.splits > 1 && kh == 0 && kg == 0)
    a.part_ml[slot] = make_float2(m_ref == -__builtin_inff() ? m_ref : m_ref * sl, l);
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

template <int G>
hipError_t launch_t(const MlaArgs& a, hipStream_t stream) {
  const size_t lds = mla_lds_bytes(a.n_heads, a.tiles_per_split);
  auto k = k_sparse_mla<G>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // (query, slice) pairs in groups of 8, each group's head blocks 8 ids apart
  const int64_t pairs = (int64_t)a.nq * a.splits;
  const int64_t grid = (pairs + 7) / 8 * 8 * (a.n_heads / (32 * G));
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(128 * G), lds, stream, a);
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
      (int64_t)a.nq * a.splits > 0x3FFFFFF ||
      mla_lds_bytes(a.n_heads, a.tiles_per_split) > 160 * 1024 ||
      (a.splits > 1 && (!a.part_o || !a.part_ml)))
    return hipErrorInvalidValue;
  return a.n_heads % 64 == 0 ? launch_t<2>(a, stream) : launch_t<1>(a, stream);
}

}  // namespace dsa
