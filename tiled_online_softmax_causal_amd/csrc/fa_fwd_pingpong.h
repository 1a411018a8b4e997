// Tiled online-softmax attention forward, 8-wave "ping-pong" kernel for gfx950.
//
// The method is the one of the aiml.sh page "Speed up long contexts with
// FlashAttention" (lab.py, tiled_flash_attention): a block of query rows stays
// on chip while key/value blocks stream through, and every row keeps a running
// maximum, a running sum and an accumulator rescaled when the maximum moves.
// Key blocks wholly above the diagonal are never visited; blocks that straddle
// it are masked per element.  This kernel is that loop laid out for CDNA4.
//
// Work split.  A workgroup owns 256 query rows of one (batch, head) and runs 8
// waves of 32 rows each, two waves per SIMD.  Waves 0-3 (group 0) and 4-7
// (group 1) alternate between two kinds of phase, one phase apart:
//
//     phase 2t     group 0: matrix phase t      group 1: softmax phase t-1
//     phase 2t+1   group 0: softmax phase t     group 1: matrix phase t
//
// where the matrix phase t issues O^T += V_{t-1}^T P_{t-1}^T and then
// S_t^T = K_t Q^T on the matrix cores (32 MFMAs for d = 128) and the softmax
// phase t turns S_t into bf16 probabilities on the vector ALUs.  Every SIMD
// thus holds one wave feeding its matrix core and one wave doing the
// exponentials, the two kinds of work overlap, and one workgroup barrier closes
// each phase.
//
// Data movement.  Group 0 carries the K tiles (64 keys) and group 1 the V
// tiles: K_{t+1} is loaded HBM -> registers during group 0's matrix phase 2t,
// V_t during group 1's softmax phase 2t, and both are written to LDS at the end
// of phase 2t+1 into the half of a double buffer whose previous tile was last
// read in phase 2t-1.  Each wave's loads are spread through its phase's work.
// LDS rows are padded (K by 16 bytes, V by 64 bytes) so the 128-bit K reads
// and the 64-bit transposed V reads are free of bank conflicts on the 64-bank
// LDS, and every read address is one per-lane base plus immediate offsets.
//
// Register layout (v_mfma_f32_32x32x16_bf16).  Scores are formed transposed,
// S^T = K . Q^T, so each lane owns ONE query (column lane%32) and half of the
// tile's keys (rows 8*(r/4) + 4*(lane/32) + r%4 of each 32-key block); row max
// and row sum are lane-local plus one v_permlane32_swap.  The fp32 scores,
// exponentiated and packed to bf16, are already the B operand of
// O^T = V^T . P^T; V^T comes from LDS through ds_read_b64_tr_b16 in the
// matching key order.  The MFMA operands read from LDS run four MFMAs ahead of
// their use (a pinned issue order), so LDS latency hides behind the matrix core.
//
// Softmax.  Base 2: c = scale*log2(e) is folded into one FMA per score and exp
// is v_exp_f32.  The maximum only guards exp2 against overflow, so it is
// maintained lazily: the first tile sets it exactly, later tiles exponentiate
// against the stale value at once, and only if some row's tile sum exceeds
// 2^64 (a score at least ~59 above the stale maximum in base 2) is that tile
// redone with the exact maximum and the accumulator and sum rescaled.  Since
// numerator and denominator share the stale maximum, the result is unchanged;
// probabilities below it underflow exactly as they would against the true one.
// The denominator is an fp32 sum of the fp32 probabilities; only the P.V
// operand is rounded to bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {
namespace pp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupThreads = kThreads / 2;
constexpr int kQW = 32;                 // query rows per wave
constexpr int kBQ = kQW * kWaves;       // query rows per workgroup
constexpr int kBK = 64;                 // keys per tile
constexpr int kAhead = 8;               // MFMAs between an operand's LDS read and its use
constexpr float kOverflowSum = 0x1p64f; // a tile sum above this forces a rescale
constexpr float kLn2 = 0.693147180559945309f;

// LDS tiles are row-major with padded rows.  K rows carry 16 pad bytes: the 16
// rows of one 16-lane group of a 128-bit K read then start on 16 different
// 4-bank groups.  V rows carry 64 pad bytes: the 4 rows x 64 bytes of one
// 32-lane transposed V read then cover all 64 banks once.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "matrix-core path covers D = 64 and 128");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;               // 16-byte chunks per row
  static constexpr int kKStride = kRowBytes + 16;               // LDS bytes per K row
  static constexpr int kVStride = kRowBytes + 64;               // LDS bytes per V row
  static constexpr int kKTileBytes = kBK * kKStride;
  static constexpr int kVTileBytes = kBK * kVStride;
  static constexpr int kLdsBytes = 2 * (kKTileBytes + kVTileBytes);  // K[2], V[2]
  static constexpr int kLoads = kBK * kChunks / kGroupThreads;   // 16-byte loads per thread per tile
  static constexpr int kRowsPerLoad = kGroupThreads / kChunks;   // tile rows covered by one load step
  static_assert(kBK * kChunks % kGroupThreads == 0, "a tile must split evenly over a 4-wave group");
};

__device__ __forceinline__ float max_halves(float x) {
  // lanes l and l^32 hold the two key halves of the same query
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Workgroup barrier that orders LDS only: outstanding global prefetches stay in
// flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup id -> (bh, query block).  Heaviest query blocks first (under the
// causal rule block qb visits qb+1 key ranges).  When the head count is a
// multiple of 8, every query block of a head is placed on one XCD (workgroups
// are dispatched round-robin over the 8 XCDs), so the head's K/V stream is
// shared in that XCD's L2 by the blocks running there at the same time.
__device__ __forceinline__ void schedule_block(int wg, int n_qb, int xcd_group, int& bh, int& qb) {
  if (xcd_group) {
    const int xcd = wg & 7, idx = wg >> 3;
    bh = (idx / n_qb) * 8 + xcd;
    qb = n_qb - 1 - idx % n_qb;
  } else {
    bh = wg / n_qb;
    qb = n_qb - 1 - wg % n_qb;
  }
}

// Issue order of a matrix phase: MFMA items 0..NPV-1 are the P.V products (two
// LDS reads each), items NPV.. the score products (one LDS read each).  The
// reads of item i + kAhead are issued right after MFMA i, and one tile load is
// issued every FSTEP MFMAs while NLOAD remain.
template <int NPV, int N>
constexpr int reads_of(int i) {
  return i < NPV ? 2 : (i < N ? 1 : 0);
}
template <int NPV, int N, int FSTEP, int NLOAD, int I>
__device__ __forceinline__ void schedule_item() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA I
  if constexpr (reads_of<NPV, N>(I + kAhead) > 0)
    __builtin_amdgcn_sched_group_barrier(0x100, reads_of<NPV, N>(I + kAhead), 0);
  if constexpr (NLOAD > 0 && I % FSTEP == 0 && I / FSTEP < NLOAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
}
template <int NPV, int N>
constexpr int first_reads() {
  int r = 0;
  for (int i = 0; i < kAhead; ++i) r += reads_of<NPV, N>(i);
  return r;
}
template <int NPV, int N, int FSTEP, int NLOAD, int... I>
__device__ __forceinline__ void schedule_matrix_phase(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, first_reads<NPV, N>(), 0);
  (schedule_item<NPV, N, FSTEP, NLOAD, I>(), ...);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_pingpong(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int S, int n_qb, float c_log2, int negate_q,
    int xcd_group) {
  using G = Geo<D>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  constexpr int DS = D / 16;  // k-steps of the score MFMA
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int NL = G::kLoads;

  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int grp = wave >> 2;   // 0: matrix phase first, carries K; 1: one phase behind, carries V
  const int col = lane & 31;   // the query this lane owns, within the wave
  const int half = lane >> 5;  // which key half of each 32-key block
  const int u = lane & 15, quad = lane >> 4;

  int bh, qb;
  schedule_block(blockIdx.x, n_qb, xcd_group, bh, qb);
  const size_t head_off = (size_t)bh * S * D;
  const uint16_t* Qh = Q + head_off;
  const int q0 = qb * kBQ;
  const int q0w = q0 + wave * kQW;

  // ---- Q^T operand: lane holds q[q0w + col][16*ds + 8*half + 0..7]
  bf16x8_t qreg[DS];
  {
    const int qrow = min(q0w + col, S - 1);
    const unsigned flip = negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(Qh + (size_t)qrow * D + 16 * ds + 8 * half);
      x ^= (u32x4_t){flip, flip, flip, flip};
      qreg[ds] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
  f32x16_t sacc[2];
  bf16x8_t pb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) pb[ks] = (bf16x8_t){};
  float m_run = -__builtin_inff(), l_run = 0.f;

  const int kv_end = CAUSAL ? min(S, q0 + kBQ) : S;
  const int n_tiles = (kv_end + kBK - 1) / kBK;
  // tiles this wave takes part in (its rows see keys below min(S, q0w + 32))
  const int n_w = q0w >= S ? 0 : (CAUSAL ? min(n_tiles, (min(q0w + kQW, S) - 1) / kBK + 1) : n_tiles);

  // ---- staging: HBM -> registers -> LDS.  Thread gtid of the carrying group
  // owns 16-byte chunks gtid, gtid + 256, ... (row-major) of its tensor's tile.
  // Rows past the end of the sequence re-read row S-1 (their scores are masked).
  const int gtid = tid & (kGroupThreads - 1);
  const int g_row = gtid / G::kChunks, g_chunk = gtid % G::kChunks;
  const uint16_t* const src_g = (grp == 0 ? K : V) + head_off + g_chunk * 8;
  const int stride_g = grp == 0 ? G::kKStride : G::kVStride;
  u32x4_t stg[NL];
  auto fetch_one = [&](int i, int t) {
    const int grow = min(t * kBK + g_row + i * G::kRowsPerLoad, S - 1);
    stg[i] = *reinterpret_cast<const u32x4_t*>(src_g + grow * D);
  };
  auto deposit = [&](char* buf) {
    char* dst = buf + g_row * stride_g + g_chunk * 16;
#pragma unroll
    for (int i = 0; i < NL; ++i) *reinterpret_cast<u32x4_t*>(dst + i * G::kRowsPerLoad * stride_g) = stg[i];
  };
  char* const kbuf0 = lds;
  char* const vbuf0 = lds + 2 * G::kKTileBytes;
  // per-lane read bases: K row col (+32 per key block), 16 bytes per half;
  // V rows 4*half + u/4 (+16 per k-step), columns 16*(quad%2) + 4*(u%4)
  const int k_lane = col * G::kKStride + half * 16;
  const int v_lane = (4 * half + (u >> 2)) * G::kVStride + (16 * (quad & 1) + 4 * (u & 3)) * 2;

  // ---- matrix phase t: O^T += V_{t-1}^T P_{t-1}^T (4 accumulators, k-step
  // outer), then S_t^T = K_t Q^T (2 accumulators, alternating).
  auto matrix_body = [&](auto pv_c, auto sc_c, auto load_c, int t, int t_load) {
    constexpr bool PV = decltype(pv_c)::value, SC = decltype(sc_c)::value, LOAD = decltype(load_c)::value;
    constexpr int NPV = PV ? DB * 4 : 0, NSC = SC ? DS * 2 : 0, N = NPV + NSC;
    constexpr int FSTEP = N / NL > 0 ? N / NL : 1;
    const char* Vl = vbuf0 + ((t - 1) & 1) * G::kVTileBytes + v_lane;
    const char* Kl = kbuf0 + (t & 1) * G::kKTileBytes + k_lane;
    // the matrix-core wave issues first; the softmax wave on the same SIMD
    // fills the issue slots the MFMAs leave free
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < (N > 0 ? N : NL); ++i) {
      if (LOAD && i % FSTEP == 0 && i / FSTEP < NL) fetch_one(i / FSTEP, t_load);
      if (i < NPV) {
        const int ks = i / DB, db = i % DB;
        const char* vp = Vl + 16 * ks * G::kVStride + 64 * db;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vp);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 8 * G::kVStride));
        const bf16x8_t av = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                                    __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], oacc[db], 0, 0, 0);
      } else if (i < N) {
        const int j = i - NPV, ds = j / 2, kb = j % 2;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Kl + 32 * kb * G::kKStride + 32 * ds);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], ds == 0 ? (f32x16_t){} : sacc[kb], 0, 0, 0);
      }
    }
    if constexpr (N > 0)
      schedule_matrix_phase<NPV, N, FSTEP, LOAD ? NL : 0>(std::make_integer_sequence<int, N>{});
    __builtin_amdgcn_s_setprio(0);
  };
  // Group 0 passes load = true: it carries K_{t+1} during matrix phase t.  Every
  // wave runs the same full body in every matrix phase, which keeps the loop's
  // register allocation simple.  Where a product is not needed its result is
  // harmless: at t = 0 the probabilities are zero and the V buffer half read
  // was zero-filled, and once a wave is past its last tile (t > n_w) its
  // skipped softmax phases zero the probabilities, so the P.V product adds
  // exactly 0; scores for t >= n_w are computed but never used.
  auto matrix_phase = [&](int t, auto load_c) {
    const int t_load = min(t + 1, n_tiles - 1);  // the last phase re-reads a tile it does not deposit
    matrix_body(T_{}, T_{}, load_c, t, t_load);
  };

  // ---- softmax phase t: S_t -> bf16 P_t, running max / sum.  Group 1 passes
  // load = true: it carries V_{t+1} during softmax phase t.
  auto softmax_phase = [&](int t, auto load_c) {
    constexpr bool LOAD = decltype(load_c)::value;
    const int t_load = min(t + 1, n_tiles - 1);
    if (t < 0 || t >= n_w) {
      if (LOAD) {
#pragma unroll
        for (int i = 0; i < NL; ++i) fetch_one(i, t_load);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pb[ks] = (bf16x8_t){};
      return;
    }
    if (LOAD) fetch_one(0, t_load);
    const int kv0 = t * kBK;
    const int qi = q0w + col;
    float c_t = c_log2;
    // Tiles that straddle the diagonal or run past S move to the base-2 domain
    // here, so a hidden score is a plain -inf even when the scale is 0.
    if ((CAUSAL && kv0 + kBK - 1 > q0w) || kv0 + kBK > S) {
      c_t = 1.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = kv0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool hidden = (CAUSAL && kj > qi) || kj >= S;
          sacc[kb][r] = hidden ? -__builtin_inff() : sacc[kb][r] * c_log2;
        }
    }
    if (LOAD && NL > 1) fetch_one(1, t_load);
    // exponentiate against the running (possibly stale) maximum; all but the
    // first tile try that directly and fall back to the exact update only when
    // a probability could approach fp32 overflow
    float rs = 0.f;
    auto exponentiate = [&]() {
      const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
      rs = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1, r0 = 8 * (ks & 1);
        bf16x8_t p8;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f32x2_t x = {__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r0 + e], c_t, neg_m)),
                             __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r0 + e + 1], c_t, neg_m))};
          rs += x[0];
          rs += x[1];
          const bf16x2_t b = __builtin_convertvector(x, bf16x2_t);
          p8[e] = b[0];
          p8[e + 1] = b[1];
        }
        pb[ks] = p8;
      }
    };
    bool exact = t == 0;
    if (!exact) {
      exponentiate();
      exact = __builtin_amdgcn_ballot_w64(!(rs <= kOverflowSum)) != 0;
    }
    if (exact) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[kb][r], sacc[kb][r + 1]));
      const float m_new = fmaxf(m_run, max_halves(mx) * c_t);
      const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
      exponentiate();
    }
    if (LOAD) {
#pragma unroll
      for (int i = 2; i < NL; ++i) fetch_one(i, t_load);
    }
    l_run += rs;
  };

  // ---- prologue: K_0 into LDS (group 0 carries K); zero the V buffer half that
  // the first matrix phase reads with zero probabilities
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) fetch_one(i, 0);
    deposit(kbuf0);
  } else {
    char* v1 = vbuf0 + G::kVTileBytes;
    for (int off = gtid * 16; off < G::kVTileBytes; off += kGroupThreads * 16)
      *reinterpret_cast<u32x4_t*>(v1 + off) = (u32x4_t){0u, 0u, 0u, 0u};
  }
  lds_barrier();

  // ---- 2 * (n_tiles + 1) phases, one barrier each.  The two groups run the
  // same phases with their roles swapped; each has its own straight loop.
  if (grp == 0) {
    for (int t = 0; t <= n_tiles; ++t) {
      matrix_phase(t, T_{});  // phase 2t; loads K_{t+1}
      lds_barrier();
      softmax_phase(t, F_{});  // phase 2t + 1
      if (t + 1 < n_tiles) deposit(kbuf0 + ((t + 1) & 1) * G::kKTileBytes);
      lds_barrier();
    }
  } else {
    for (int t = 0; t <= n_tiles; ++t) {
      softmax_phase(t - 1, T_{});  // phase 2t; loads V_t
      lds_barrier();
      matrix_phase(t, F_{});  // phase 2t + 1
      if (t < n_tiles) deposit(vbuf0 + (t & 1) * G::kVTileBytes);
      lds_barrier();
    }
  }

  // ---- epilogue: O = acc / l (bf16, round to nearest even), lse = ln2 * (m + log2 l)
  const int qi = q0w + col;
  const float l_tot = sum_halves(l_run);
  if (qi < S) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = O + head_off + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4_t v4 = {oacc[db][4 * rg + 0] * inv, oacc[db][4 * rg + 1] * inv,
                            oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv};
        *reinterpret_cast<bf16x4_t*>(orow + 32 * db + 8 * rg + 4 * half) = __builtin_convertvector(v4, bf16x4_t);
      }
    if (LSE && half == 0) LSE[(size_t)bh * S + qi] = (m_run + __builtin_log2f(l_tot)) * kLn2;
  }
}

}  // namespace pp
}  // namespace fa
