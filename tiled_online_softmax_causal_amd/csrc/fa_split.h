// Short-sequence attention forward for gfx950: paired query blocks, four key
// streams per workgroup, partial results merged on chip.
//
// The method is the one of the aiml.sh page "Speed up long contexts with
// FlashAttention" (lab.py, tiled_flash_attention): a block of query rows stays
// on chip while key/value tiles stream through, with a running maximum, a
// running sum and a rescaled accumulator per row; key tiles wholly above the
// diagonal are never visited and the diagonal tile is masked per element.
// Online softmax partial results over disjoint key sets combine exactly: with
// maxima m1, m2 and sums l1, l2, m = max(m1, m2), l = 2^(m1-m) l1 + 2^(m2-m)
// l2, O = (2^(m1-m) O1 + 2^(m2-m) O2) / l.  That is what lets several streams
// of one workgroup take disjoint keys of the same rows.
//
// When the sequence is short, 256-row work items cannot fill the 256 CUs
// (b1 h32 S1024: 128 items), and under the causal rule 64- or 128-row blocks
// differ up to 16-fold in work.  Here a work unit is a pair of 64-row query
// blocks of one head, qb and n-1-qb, whose keys add up to about the same count
// for every pair, so b1 h32 S1024 is 256 equal units, one per CU.  A
// workgroup of eight waves (two per SIMD, so one wave's exponentials overlap
// the other's matrix products) runs a unit: wave (rh, st) owns the 32 rows rh
// of the current block and key stream st, keys 32 st .. 32 st + 31 of every
// 128-key tile.  Each step holds one 128-key K and V tile in LDS,
// double-buffered: the copies of step i+1 (HBM -> LDS directly,
// global_load_lds) are issued between the score MFMAs of step i, every LDS
// operand is read a few MFMAs ahead of its use (a pinned issue order), and one
// barrier closes each step.  A block's 64 Q rows are copied once into LDS
// (the four streams share them) and each wave reads its operand from there;
// the second block's rows replace the first's during the first block's second
// step.  The first block's partial results stay in registers while the second
// block's steps run; at the end of the unit the four streams merge the partial
// results of both blocks in two rounds of pairwise exchange through LDS (one
// stage per block, and the maxima and sums in a small area of their own),
// sharing the rounds' barriers; each stream then finishes a quarter of the
// head dimension.  Non-causal units are single blocks (all blocks weigh the
// same).
//
// Register layout as in the other matrix-core kernels: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16, so a lane owns one query (column lane % 32) and the
// row max and sum are lane-local plus one v_permlane32_swap; the fp32 scores,
// exponentiated and packed to bf16, are the B operand of O^T = V^T P^T, with
// V^T read from LDS through ds_read_b64_tr_b16.  The softmax is base 2 with
// c = |scale| log2(e) folded into one FMA per score (a negative scale negates
// Q, exactly, at load).  The running maximum is lazy, as in the ping-pong
// kernel: it starts at one key's score and moves only when a tile's row sum
// would pass 2^64, so the accumulator is almost never rescaled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_common.h"

namespace fa {
namespace split {

using namespace fa::common;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 64;                  // query rows per block
constexpr int kBK = 128;                 // keys per tile (32 per stream)
constexpr float kOverflowSum = 0x1p64f;  // a tile sum above this redoes the tile with the exact maximum

template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "matrix-core path covers D = 64 and 128");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;             // 16-byte chunks per row
  static constexpr int kTileBytes = kBK * kRowBytes;         // one K or V tile
  static constexpr int kStageBytes = 2 * kTileBytes;         // K then V
  static constexpr int kMLBytes = kWaves * 2 * 64 * 4;       // the exchange's maxima and sums (one block)
  static constexpr int kQBytes = kBQ * kRowBytes;             // one block's Q rows
  static constexpr int kLdsBytes = 2 * kStageBytes + 2 * kMLBytes + kQBytes;
  static constexpr int kLoads = kStageBytes / (kThreads * 16);  // 16-byte copies per thread per step
  static constexpr int kQLoads = kQBytes / (kThreads * 16);     // 16-byte copies per thread per Q block
  static constexpr int kRowsPerLoad = kThreads / kChunks;       // tile rows one copy step covers
  // the first exchange round moves half of O^T per wave (16 values per lane and
  // 32-row block of D, D/64 blocks); it must fit one stage
  static_assert(kWaves * (D / 64) * 16 * 64 * 4 <= kStageBytes, "the exchange fits one stage");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  static_assert(kLoads * kThreads * 16 == kStageBytes, "a stage splits evenly over the workgroup");
  static_assert(kQLoads * kThreads * 16 == kQBytes, "a Q block splits evenly over the workgroup");
};

// Work unit u of a head -> its one or two query blocks (64 rows each).
__host__ __device__ inline void unit_blocks(int u, int n_qb, bool causal, int& qa, int& qb) {
  if (causal) {
    qa = n_qb - 1 - u;      // the heavy block first
    qb = qa != u ? u : -1;  // and its light partner (none for the middle block)
  } else {
    qa = u;
    qb = -1;
  }
}
__host__ __device__ inline int units_per_head(int n_qb, bool causal) { return causal ? (n_qb + 1) / 2 : n_qb; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_split(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int S, int n_qb, int BH, float c_log2, int negate_q,
    int xcd_group) {
  using G = Geo<D>;
  constexpr int DS = D / 16;  // k-steps of the score MFMA
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int KS = 2;       // k-steps of the P.V MFMA (32 keys per stream)
  constexpr int NL = G::kLoads;
  constexpr int NS = DS;       // score MFMAs per wave and step
  constexpr int NP = DB * KS;  // P.V MFMAs per wave and step
  static_assert(NL <= NS, "a step's copies fit one per score MFMA");

  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rh = wave & 1;   // which 32 rows of the block
  const int st = wave >> 1;  // which key stream (keys 32 st .. of each tile)
  const int col = lane & 31, half = lane >> 5, u = lane & 15, quad = lane >> 4;

  // ---- the unit: head bh, blocks qa (heavy) and qb2 (light, or none)
  const int U = units_per_head(n_qb, CAUSAL);
  int bh, un;
  if (xcd_group) {  // every unit of a head on one XCD (workgroups go round-robin over the 8 XCDs)
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    bh = (idx / U) * 8 + xcd;
    un = idx % U;
  } else {
    bh = blockIdx.x / U;
    un = blockIdx.x % U;
  }
  bh = __builtin_amdgcn_readfirstlane(bh);
  un = __builtin_amdgcn_readfirstlane(un);
  int qa, qb2;
  unit_blocks(un, n_qb, CAUSAL, qa, qb2);
  auto kv_end_of = [&](int q) { return CAUSAL ? min(S, q * kBQ + kBQ) : S; };
  const int sA = (kv_end_of(qa) + kBK - 1) / kBK;
  const int n_steps = sA + (qb2 >= 0 ? (kv_end_of(qb2) + kBK - 1) / kBK : 0);
  const size_t head = (size_t)bh * S * D;

  // ---- copies: all 512 threads fill a stage (K tile, then V tile).  Thread
  // tid writes 16-byte chunk slots tid, tid + 512, ... (row-major over the
  // swizzled tiles); its source is the logical chunk the swizzle puts in each
  // slot.  Rows past the end of the sequence re-read row S-1 (their scores are
  // masked).
  const int tid = wave * 64 + lane;
  const int c_row0 = tid / G::kChunks, c_pch = tid % G::kChunks;
  auto stage_ptr = [&](int g) { return lds + (g & 1) * G::kStageBytes; };
  char* const q_lds = lds + 2 * G::kStageBytes + 2 * G::kMLBytes;
  // copy j of a tile (K for j < NL/2, else V) into stage dst
  auto copy_step = [&](int j, const uint16_t* kt_src, const uint16_t* vt_src, int rows, char* dst) {
    constexpr int PER = NL / 2;  // copies per tensor
    const int x = j / PER, jj = j % PER;
    const int row = jj * G::kRowsPerLoad + c_row0;
    const int lrow = min(row, rows - 1);  // the chunk keeps its swizzle column
    const unsigned off = (unsigned)(lrow * G::kRowBytes + ((c_pch ^ swz<G::kChunks>(row)) << 4));
    copy16_to_lds(x == 0 ? kt_src : vt_src, off, dst + x * G::kTileBytes + (jj * kThreads + 64 * wave) * 16);
  };

  // ---- Q of block q: the workgroup copies its 64 rows once into LDS (the
  // layout of a K tile: swizzled 16-byte chunks; rows past the end of the
  // sequence re-read row S-1, never stored); each wave then reads its Q^T
  // operand, lane holding q[row][16 ds + 8 half + 0..7]
  struct QOp {
    bf16x8_t r[DS];
  };
  auto copy_q = [&](int q) {
    const uint16_t* src = Q + head;
#pragma unroll
    for (int j = 0; j < G::kQLoads; ++j) {
      const int row = j * G::kRowsPerLoad + c_row0;
      const int grow = min(q * kBQ + row, S - 1);
      const unsigned off = (unsigned)(grow * G::kRowBytes + ((c_pch ^ swz<G::kChunks>(row)) << 4));
      copy16_to_lds(src, off, q_lds + (j * kThreads + 64 * wave) * 16);
    }
  };
  auto read_q = [&]() {
    QOp op;
    const int sq = swz<G::kChunks>(col);
    const char* base = q_lds + (32 * rh + col) * G::kRowBytes;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(base + (((2 * ds + half) ^ sq) << 4));
      if (negate_q) x ^= (u32x4_t){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      op.r[ds] = __builtin_bit_cast(bf16x8_t, x);
    }
    return op;
  };

  // ---- LDS read offsets.  K (A operand of S^T): row 32 st + col, logical
  // chunk 2 ds + half.  V^T (transposed read): rows 32 st + 16 ks + 4 half +
  // u/4 (+8), logical chunk 4 db + 2 (quad % 2) + (u % 4) / 2, byte 8 (u % 2).
  int k_off[DS], v_lo[DB], v_hi[DB];
  {
    const int sk = swz<G::kChunks>(col);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) k_off[ds] = (32 * st + col) * G::kRowBytes + (((2 * ds + half) ^ sk) << 4);
    const int vr = 4 * half + (u >> 2);
    const int s_lo = swz<G::kChunks>(vr), s_hi = swz<G::kChunks>(vr + 8);
    const int cl = 2 * (quad & 1) + ((u & 3) >> 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      v_lo[db] = (32 * st + vr) * G::kRowBytes + (((4 * db + cl) ^ s_lo) << 4) + 8 * (u & 1);
      v_hi[db] = (32 * st + vr + 8) * G::kRowBytes + (((4 * db + cl) ^ s_hi) << 4) + 8 * (u & 1);
    }
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
  float m_run = -__builtin_inff(), l_run = 0.f;

  // ---- one step of block q (tile i of the block, the unit's step g): the
  // stream's 32 keys.  The NL copies of the next step go out one per score
  // MFMA; every LDS operand is read kAhead MFMAs before its use.  The issue
  // order is pinned (sched_barrier between items): the compiler would
  // otherwise wait for each read right before its MFMA.  `compute` false:
  // only the copies (the stream has no key of the block in this tile).
  constexpr int kAhead = 4;
  auto step = [&](const QOp& qop, int q, int i, int g, const uint16_t* kn, const uint16_t* vn, int rows_n,
                  bool compute) __attribute__((always_inline)) {
    char* const dst = stage_ptr(g + 1);
    if (!compute) {
#pragma unroll
      for (int j = 0; j < NL; ++j) copy_step(j, kn, vn, rows_n, dst);
      return;
    }
    const char* Kl = stage_ptr(g);
    const char* Vl = Kl + G::kTileBytes;
    f32x16_t sacc;
    bf16x8_t ka[NS];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) ka[k] = *reinterpret_cast<const bf16x8_t*>(Kl + k_off[k]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k], qop.r[k], k == 0 ? (f32x16_t){} : sacc, 0, 0, 0);
      if (k < NL) copy_step(k, kn, vn, rows_n, dst);
      if (k + kAhead < NS) ka[k + kAhead] = *reinterpret_cast<const bf16x8_t*>(Kl + k_off[k + kAhead]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V^T operands, read while the softmax runs
    bf16x8_t va[NP];
    auto read_v = [&](int k) __attribute__((always_inline)) {
      const int ks = k / DB, db = k % DB;
      const char* vp = Vl + 16 * ks * G::kRowBytes;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + v_lo[db]));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + v_hi[db]));
      va[k] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2,
                                      3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int k = 0; k < kAhead; ++k) read_v(k);
    __builtin_amdgcn_sched_barrier(0);

    const int kv0 = i * kBK + 32 * st;  // the stream's first key
    const int q0w = q * kBQ + 32 * rh;
    const int qi = q0w + col;
    const bool masked = (CAUSAL && kv0 + 31 > q0w) || kv0 + 32 > S;
    float c_t = c_log2;
    if (masked) {
      c_t = 1.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = kv0 + 8 * (r >> 2) + 4 * half + (r & 3);
        const bool hidden = (CAUSAL && kj > qi) || kj >= S;
        sacc[r] = hidden ? -__builtin_inff() : sacc[r] * c_log2;
      }
    }
    // Lazy running maximum (it only guards exp2 against overflow): a lane
    // starts it at the score of the first key of the stream's first tile, or of
    // the first tile where it sees one, and exponentiates every tile against
    // the running value (0 while it is still -inf: every score it has is then
    // -inf too).  Only if some row's tile sum passes 2^64 is the tile redone
    // against its exact maximum (the scores are still in sacc), rescaling O
    // and l.
    if (m_run == -__builtin_inff()) m_run = max_halves(sacc[0] * c_t);
    float rs;
    bf16x8_t pb[KS];
    auto exponentiate = [&]() __attribute__((always_inline)) {
      const float m_ref = m_run == -__builtin_inff() ? 0.f : m_run;
      rs = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r0 = 8 * ks;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f32x2_t x = {__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r0 + e], c_t, -m_ref)),
                             __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r0 + e + 1], c_t, -m_ref))};
          rs += x[0];
          rs += x[1];
          const bf16x2_t b = __builtin_convertvector(x, bf16x2_t);
          pb[ks][e] = b[0];
          pb[ks][e + 1] = b[1];
        }
      }
    };
    exponentiate();
    if (__builtin_amdgcn_ballot_w64(!(rs <= kOverflowSum)) != 0) {
      float mx = fmaxf(sacc[0], sacc[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = max3(mx, sacc[r], sacc[r + 1]);
      const float m_new = fmaxf(m_run, max_halves(mx) * c_t);
      const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
      exponentiate();
    }
    l_run += rs;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int ks = k / DB, db = k % DB;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[k], pb[ks], oacc[db], 0, 0, 0);
      if (k + kAhead < NP) read_v(k + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the end of the unit: the four streams' partial results of each of
  // its NB blocks merge in two rounds of pairwise exchange through LDS (block
  // b through stage b, all copies landed and consumed by then, and its own
  // maxima/sums area), the rounds of both blocks sharing their barriers.
  // Round 1 pairs streams st and st^1; each keeps half of the 32-row blocks of
  // O^T (st even: the lower half) and sends the other half.  Round 2 pairs st
  // and st^2, which kept the same half; each keeps one block (the lower if
  // st < 2) and finishes it: merges, normalises, stores (at d = 64, one block
  // per half: streams 0 and 1 finish it, 2 and 3 only send).  The stream and
  // the block are compile-time indices so that the accumulators are addressed
  // statically and stay in registers.  The first block's partial results wait
  // in registers (acc_a) while the second block's steps run.
  struct Partial {
    f32x16_t o[DB];
    float m, l;
  };
  Partial acc_a;
  auto finish_st = [&](auto st_c, auto nb_c, int q0, int q1) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    constexpr int NB = decltype(nb_c)::value;
    constexpr int H = DB / 2;                  // blocks kept after round 1
    constexpr int KEEP1 = (ST & 1) * H;        // first block kept after round 1
    constexpr int SEND1 = ((ST & 1) ^ 1) * H;  // first block sent in round 1
    constexpr int H2 = H / 2 > 0 ? H / 2 : 1;  // blocks kept (and sent) in round 2
    constexpr int KEEP2 = H / 2 > 0 ? KEEP1 + (ST >> 1) * H2 : KEEP1;
    constexpr int SEND2 = H / 2 > 0 ? KEEP1 + ((ST >> 1) ^ 1) * H2 : KEEP1;
    constexpr bool FINISHES = H / 2 > 0 || (ST >> 1) == 0;
    constexpr int P1 = ST ^ 1, P2 = ST ^ 2;
    // block b's accumulator, maximum and sum: the saved first block when there
    // are two, else the running ones
    auto o_of = [&](auto b_c) __attribute__((always_inline)) -> f32x16_t* {
      if constexpr (NB == 2 && decltype(b_c)::value == 0) return acc_a.o; else return oacc;
    };
    auto m_of = [&](auto b_c) __attribute__((always_inline)) -> float& {
      if constexpr (NB == 2 && decltype(b_c)::value == 0) return acc_a.m; else return m_run;
    };
    auto l_of = [&](auto b_c) __attribute__((always_inline)) -> float& {
      if constexpr (NB == 2 && decltype(b_c)::value == 0) return acc_a.l; else return l_run;
    };
    auto each_block = [&](auto&& f) __attribute__((always_inline)) {
      f(std::integral_constant<int, 0>{});
      if constexpr (NB == 2) f(std::integral_constant<int, 1>{});
    };
    auto xb_of = [&](auto b_c) { return reinterpret_cast<float*>(lds + decltype(b_c)::value * G::kStageBytes); };
    auto ml_of = [&](auto b_c) {
      return reinterpret_cast<float*>(lds + 2 * G::kStageBytes + decltype(b_c)::value * G::kMLBytes);
    };
    // round 1: send half of O^T and (m, l) to stream P1
    each_block([&](auto b_c) __attribute__((always_inline)) {
      float* mine = xb_of(b_c) + (size_t)wave * H * 16 * 64;
      f32x16_t* o = o_of(b_c);
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(16 * h + r) * 64 + lane] = o[SEND1 + h][r];
      ml_of(b_c)[(wave * 2 + 0) * 64 + lane] = m_of(b_c);
      ml_of(b_c)[(wave * 2 + 1) * 64 + lane] = l_of(b_c);
    });
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    phase_barrier();
    each_block([&](auto b_c) __attribute__((always_inline)) {
      const int pw = 2 * P1 + rh;  // the partner wave
      const float* theirs = xb_of(b_c) + (size_t)pw * H * 16 * 64;
      const float m_o = ml_of(b_c)[(pw * 2 + 0) * 64 + lane], l_o = ml_of(b_c)[(pw * 2 + 1) * 64 + lane];
      float& m_s = m_of(b_c);
      float& l_s = l_of(b_c);
      f32x16_t* o = o_of(b_c);
      const float m = fmaxf(m_s, m_o);
      const float a_s = m_s == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_s - m);
      const float a_o = m_o == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_o - m);
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[KEEP1 + h][r] = o[KEEP1 + h][r] * a_s + theirs[(16 * h + r) * 64 + lane] * a_o;
      l_s = l_s * a_s + l_o * a_o;
      m_s = m;
    });
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    phase_barrier();
    // round 2: send a kept block and (m, l) to stream P2
    each_block([&](auto b_c) __attribute__((always_inline)) {
      float* mine = xb_of(b_c) + (size_t)wave * H2 * 16 * 64;
      f32x16_t* o = o_of(b_c);
#pragma unroll
      for (int h = 0; h < H2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(16 * h + r) * 64 + lane] = o[SEND2 + h][r];
      ml_of(b_c)[(wave * 2 + 0) * 64 + lane] = m_of(b_c);
      ml_of(b_c)[(wave * 2 + 1) * 64 + lane] = l_of(b_c);
    });
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    phase_barrier();
    each_block([&](auto b_c) __attribute__((always_inline)) {
      const int pw = 2 * P2 + rh;
      const float* theirs = xb_of(b_c) + (size_t)pw * H2 * 16 * 64;
      const float m_o = ml_of(b_c)[(pw * 2 + 0) * 64 + lane], l_o = ml_of(b_c)[(pw * 2 + 1) * 64 + lane];
      const float m_s = m_of(b_c), l_s = l_of(b_c);
      f32x16_t* o = o_of(b_c);
      const float m = fmaxf(m_s, m_o);  // finite: every row sees a key in some stream
      const float a_s = m_s == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_s - m);
      const float a_o = m_o == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_o - m);
      const float l_tot = sum_halves(a_s * l_s + a_o * l_o);
      const float inv_s = a_s / l_tot, inv_o = a_o / l_tot;
      const int q = decltype(b_c)::value == 0 ? q0 : q1;
      const int qi = q * kBQ + 32 * rh + col;
      uint16_t* const orow = O + head + (size_t)min(qi, S - 1) * D;
      if constexpr (FINISHES) {
#pragma unroll
        for (int h = 0; h < H2; ++h) {
          const int db = KEEP2 + h;
#pragma unroll
          for (int rg = 0; rg < 4; rg += 2) {
            f32x4_t v0, v1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v0[e] = o[KEEP2 + h][4 * rg + e] * inv_s + theirs[(16 * h + 4 * rg + e) * 64 + lane] * inv_o;
              v1[e] = o[KEEP2 + h][4 * rg + 4 + e] * inv_s + theirs[(16 * h + 4 * rg + 4 + e) * 64 + lane] * inv_o;
            }
            // columns 32 db + 8 rg + 4 half + 0..3 (a0) and the same for rg + 1
            // (a1); lanes l and l^32 swap so that each stores a whole 16-byte piece
            const u32x2_t a0 = __builtin_bit_cast(u32x2_t, __builtin_convertvector(v0, bf16x4_t));
            const u32x2_t a1 = __builtin_bit_cast(u32x2_t, __builtin_convertvector(v1, bf16x4_t));
            u32x2_t got;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const unsigned send = half ? a0[e] : a1[e];
              const auto p = __builtin_amdgcn_permlane32_swap(send, send, false, false);
              got[e] = half ? p[0] : p[1];
            }
            const u32x4_t piece =
                half ? (u32x4_t){got[0], got[1], a1[0], a1[1]} : (u32x4_t){a0[0], a0[1], got[0], got[1]};
            if (qi < S) *reinterpret_cast<u32x4_t*>(orow + 32 * db + 8 * (rg + half)) = piece;
          }
        }
      }
      if (LSE && ST == 0 && half == 0 && qi < S) LSE[(size_t)bh * S + qi] = (m + __builtin_log2f(l_tot)) * common::kLn2;
    });
  };
  auto finish = [&](auto nb_c, int q0, int q1) __attribute__((always_inline)) {
    switch (st) {
      case 0: finish_st(std::integral_constant<int, 0>{}, nb_c, q0, q1); break;
      case 1: finish_st(std::integral_constant<int, 1>{}, nb_c, q0, q1); break;
      case 2: finish_st(std::integral_constant<int, 2>{}, nb_c, q0, q1); break;
      default: finish_st(std::integral_constant<int, 3>{}, nb_c, q0, q1); break;
    }
  };

  // the tile (of the head) of the unit's step g, clamped to a valid one past the end
  auto tile_of_step = [&](int g) { return g < sA ? g : (g < n_steps ? g - sA : 0); };
  auto copy_src = [&](int g, const uint16_t*& kp, const uint16_t*& vp, int& rows) {
    const int t = tile_of_step(g);
    kp = K + head + (size_t)t * kBK * D;
    vp = V + head + (size_t)t * kBK * D;
    rows = S - t * kBK;
  };

  // ---- prologue: the tile of step 0 and the first block's Q
  {
    const uint16_t *kp, *vp;
    int rows;
    copy_src(0, kp, vp, rows);
#pragma unroll
    for (int j = 0; j < NL; ++j) copy_step(j, kp, vp, rows, stage_ptr(0));
    copy_q(qa);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
  phase_barrier();

  // the steps of one block (its Q operand fixed), then the block's merge
  // The second block's Q replaces the first's in LDS once every wave has read
  // it (after the first step's barrier); the copy completes under the waits of
  // the next barrier, or of the one before the second block when the first
  // block has a single step.
  auto run_block = [&](int q, int g0, int g1) __attribute__((always_inline)) {
    const QOp qop = read_q();
    const int kv_end = kv_end_of(q);
    for (int g = g0; g < g1; ++g) {
      const int i = g - g0;
      const bool have = i * kBK + 32 * st < kv_end;  // the stream has keys of the block in this tile
      const uint16_t *kn, *vn;
      int rows_n;
      copy_src(g + 1, kn, vn, rows_n);
      step(qop, q, i, g, kn, vn, rows_n, have);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
      phase_barrier();
      if (g == 0 && qb2 >= 0) copy_q(qb2);
    }
  };
  run_block(qa, 0, sA);
  if (qb2 >= 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc_a.o[db] = oacc[db];
      oacc[db] = (f32x16_t){};
    }
    acc_a.m = m_run;
    acc_a.l = l_run;
    m_run = -__builtin_inff();
    l_run = 0.f;
    if (sA == 1) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
      phase_barrier();
    }
    run_block(qb2, sA, n_steps);
    finish(std::integral_constant<int, 2>{}, qa, qb2);
  } else {
    finish(std::integral_constant<int, 1>{}, qa, qa);
  }
}

}  // namespace split
}  // namespace fa
