// Backward pass of the tiled attention forward on the gfx950 matrix cores
// (bf16 in and out, fp32 accumulation).
//
// The pages stop at the forward of the aiml.sh page "Speed up long contexts
// with FlashAttention" (lab.py, tiled_flash_attention); this is its gradient,
// computed the same tiled way: the probabilities are recomputed tile by tile
// from Q, K and the log-sum-exp the forward saved, so no S x S matrix reaches
// memory here either.  Per (batch, head), with P = softmax(scale * Q K^T) under
// the causal rule and an upstream gradient dO:
//
//     delta_i = dO_i . O_i
//     dP = dO V^T,  dS = P * (dP - delta)
//     dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO
//
// Two kernels, so that every output row has one writer and no atomics are
// needed:
//   attn_bwd_dq    a workgroup owns 128 query rows (32 per wave) and streams
//                  64-key K/V tiles: S^T = K Q^T and dP^T = V dO^T, then
//                  dQ^T += K^T dS^T.  It also writes delta for the second kernel.
//   attn_bwd_dkdv  a workgroup owns 128 keys (32 per wave; their K rows in LDS,
//                  their V rows in registers) and streams 32- or 64-row Q/dO
//                  tiles: X = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//                  dK^T += Q^T dS.
// Both recompute P and dP, which costs two extra products per tile over a
// one-kernel design with atomic dQ updates.
//
// Layouts are those of the 4-wave forward kernel (fa_mfma_bf16.h): a 32-row
// operand held in registers has one row per lane (row = lane % 32, 8 columns per
// lane and k-step); accumulators put one row of the result per lane as well
// (column = lane % 32), so the elementwise softmax-gradient work is lane-local;
// the bf16 probabilities or dS of a 16-row k-step are the B operand of the next
// MFMA as they sit in the accumulator registers, and the A operand that pairs
// with them (K^T, dO^T or Q^T) is read transposed from LDS (ds_read_b64_tr_b16)
// in the matching row order.
#pragma once

#include <utility>

#include "fa_common.h"
#include "fa_mfma_bf16.h"

namespace fa {
namespace bwd {

constexpr int kRows = 32 * kWaves;  // query rows (dQ kernel) or keys (dK/dV kernel) per workgroup
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// Issue order of a run of N steps of M MFMAs, each step taking R LDS reads for
// its A operands: first PRE other reads (row values the run's elementwise work
// needs) and the reads of the first A steps, then each step's MFMAs followed by
// the reads of step i + A.  Left to itself the compiler reads each operand
// right before its MFMA and waits for it there, so every MFMA pays the LDS
// latency; A steps of lead hide it.
template <int N, int M, int R, int A, int PRE, int... I>
__device__ __forceinline__ void pipeline_reads(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, PRE + R * (N < A ? N : A), 0);  // DS reads
  ((__builtin_amdgcn_sched_group_barrier(0x008, M, 0),                         // MFMAs of step I
    (I + A < N ? __builtin_amdgcn_sched_group_barrier(0x100, R, 0) : void())), ...);
}
template <int N, int M, int R, int A, int PRE = 0>
__device__ __forceinline__ void pipeline_reads() {
  pipeline_reads<N, M, R, A, PRE>(std::make_integer_sequence<int, N>{});
}

// Copy ROWS rows of X starting at r0 (rows past S re-read row S-1) into a
// swizzled LDS tile, HBM -> LDS directly (global_load_lds, no register
// staging): thread tid fills the tile's 16-byte slots tid, tid + 256, ...
// with the logical chunk the swizzle puts there.  The copies are not tracked
// by the compiler; the caller waits (s_waitcnt vmcnt(0)) before the barrier
// that publishes the tile.
template <int D, int ROWS>
__device__ __forceinline__ void copy_tile(const uint16_t* __restrict__ X, int r0, int S, char* tile, int tid) {
  constexpr int kChunks = D / 8;
  constexpr int L = ROWS * kChunks / kThreads;
  static_assert(ROWS * kChunks % kThreads == 0, "a tile must split evenly over the workgroup");
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int cidx = i * kThreads + tid;
    const int row = cidx / kChunks, pch = cidx % kChunks;
    const int lch = pch ^ lds_swizzle<D>(row);
    common::copy16_to_lds(X + (size_t)min(r0 + row, S - 1) * D + lch * 8, tile + (i * kThreads + wave * 64) * 16);
  }
}

// A 32-row operand in registers: lane holds X[row][16*ds + 8*half + 0..7].
template <int D>
__device__ __forceinline__ void load_row_operand(bf16x8_t (&r)[D / 16], const uint16_t* __restrict__ X,
                                                 size_t row_off, int half) {
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    r[ds] = *reinterpret_cast<const bf16x8_t*>(X + row_off + 16 * ds + 8 * half);
}

// A operand "rows of a tile", k = d: lane holds T[32*rb + lane%32][16*ds + 8*half + 0..7].
template <int D>
__device__ __forceinline__ bf16x8_t tile_rows(const char* T, int rb, int ds, int col, int half) {
  return *reinterpret_cast<const bf16x8_t*>(T + lds_chunk_offset<D>(32 * rb + col, 2 * ds + half));
}

// A operand "tile transposed", m = d (block db), k = tile rows of k-step ks in
// the order the accumulator registers hold them (16*ks + 4*half + 0..3, then +8).
template <int D>
__device__ __forceinline__ bf16x8_t tile_transposed(const char* T, int db, int ks, int lane) {
  const int half = lane >> 5, u = lane & 15, grp = lane >> 4;
  const int vcol = 32 * db + 16 * (grp & 1) + 4 * (u & 3);
  const int vchunk = vcol >> 3, vbyte = (vcol & 7) * 2;
  const int vrow0 = 16 * ks + 4 * half + (u >> 2);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(T + lds_chunk_offset<D>(vrow0, vchunk) + vbyte));
  const s16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(T + lds_chunk_offset<D>(vrow0 + 8, vchunk) + vbyte));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4,
                                 5, 6, 7);
}

// The bf16 B operand of k-step ks (16 rows) from two 32-row accumulators.
__device__ __forceinline__ bf16x8_t pack_kstep(const f32x16_t* acc, int ks) {
  const int b = ks >> 1, r0 = 8 * (ks & 1);
  f32x8_t x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = acc[b][r0 + e];
  return __builtin_convertvector(x, bf16x8_t);
}

// Store a transposed accumulator (32-row blocks of d, one output row per lane)
// as bf16 row `row` of Y, times `mul`.
template <int D>
__device__ __forceinline__ void store_row(uint16_t* __restrict__ Y, size_t row_off, const f32x16_t (&acc)[D / 32],
                                          float mul, int half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4_t v4 = {acc[db][4 * rg] * mul, acc[db][4 * rg + 1] * mul, acc[db][4 * rg + 2] * mul,
                          acc[db][4 * rg + 3] * mul};
      *reinterpret_cast<bf16x4_t*>(Y + row_off + 32 * db + 8 * rg + 4 * half) = __builtin_convertvector(v4, bf16x4_t);
    }
}

// ---------------------------------------------------------------- dQ (and delta)
template <int D, bool CAUSAL, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void attn_bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    uint16_t* __restrict__ dQ, float* __restrict__ Delta, int S, int n_qb, int BH, float scale, int xcd_group) {
  using G = TileGeo<D>;
  constexpr int DS = D / 16, DB = D / 32, KB = kBK / 32, KS = kBK / 16;
  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const BlockCoord bc = schedule_block(blockIdx.x, n_qb, BH, xcd_group);
  const size_t head = (size_t)bc.bh * S * D;
  const int q0 = bc.qb * kRows, q0w = q0 + 32 * wave;
  const int qi = q0w + col, qr = min(qi, S - 1);

  // Q^T and dO^T operands of the lane's query; delta = dO . O over the bf16 values
  bf16x8_t qreg[DS], doreg[DS];
  load_row_operand<D>(qreg, Q, head + (size_t)qr * D, half);
  load_row_operand<D>(doreg, dO, head + (size_t)qr * D, half);
  float dpart = 0.f;
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    const bf16x8_t o8 = *reinterpret_cast<const bf16x8_t*>(O + head + (size_t)qr * D + 16 * ds + 8 * half);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)doreg[ds][e], (float)o8[e], dpart);
  }
  const float delta = wave_sum_halves(dpart);
  if (half == 0 && qi < S) Delta[(size_t)bc.bh * S + qi] = delta;
  const float lse2 = LSE[(size_t)bc.bh * S + qr] * kLog2e;  // P = exp2(s * c2 - lse2)
  const float c2 = scale * kLog2e;

  f32x16_t qacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) qacc[db] = (f32x16_t){};

  const int kv_end = CAUSAL ? min(S, q0 + kRows) : S;
  const int n_tiles = (kv_end + kBK - 1) / kBK;
  copy_tile<D, kBK>(K + head, 0, S, lds, tid);
  copy_tile<D, kBK>(V + head, 0, S, lds + G::kTileBytes, tid);
  __builtin_amdgcn_s_waitcnt(common::waitcnt_vm<0>());
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBK;
    const bool has_next = t + 1 < n_tiles;
    if (has_next) {  // into the other stage, last read before the previous barrier
      char* nx = lds + ((t + 1) & 1) * G::kStageBytes;
      copy_tile<D, kBK>(K + head, kv0 + kBK, S, nx, tid);
      copy_tile<D, kBK>(V + head, kv0 + kBK, S, nx + G::kTileBytes, tid);
    }
    const char* Kl = lds + (t & 1) * G::kStageBytes;
    const char* Vl = Kl + G::kTileBytes;

    const bool live = (!CAUSAL || kv0 <= q0w + 31) && q0w < S;
    if (live) {
      // S^T = K Q^T and dP^T = V dO^T (keys down the registers, one query per lane)
      f32x16_t sacc[KB], pacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = (f32x16_t){};
        pacc[kb] = (f32x16_t){};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_rows<D>(Kl, kb, ds, col, half), qreg[ds], sacc[kb], 0, 0, 0);
          pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_rows<D>(Vl, kb, ds, col, half), doreg[ds], pacc[kb], 0, 0, 0);
        }
      }
      pipeline_reads<KB * DS, 2, 2, 2>();
      __builtin_amdgcn_sched_barrier(0);
      // dS = P * (dP - delta); hidden keys (above the diagonal or past S) give 0
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = kv0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool hidden = (CAUSAL && kj > qi) || kj >= S;
          const float p = hidden ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c2, -lse2));
          sacc[kb][r] = p * (pacc[kb][r] - delta);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t dsb = pack_kstep(sacc, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          qacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_transposed<D>(Kl, db, ks, lane), dsb, qacc[db], 0, 0, 0);
      }
      pipeline_reads<KS * DB, 1, 2, 4>();
    }
    __builtin_amdgcn_s_waitcnt(common::waitcnt_vm<0>());  // the next tile has landed
    __syncthreads();
  }
  if (qi < S) store_row<D>(dQ, head + (size_t)qi * D, qacc, scale, half);
}

// ---------------------------------------------------------------- dK and dV
// QT query rows per streamed tile (32 or 64): the shorter tile needs half the
// accumulator registers for X and dP, at twice the barriers.
template <int D, int QT>
struct QTileGeo {
  static constexpr int kTileBytes = QT * D * 2;
  static constexpr int kStageBytes = 2 * kTileBytes;  // Q tile then dO tile
  static constexpr int kLdsBytes = 2 * kStageBytes;   // two stages
};

template <int D, bool CAUSAL, int QT, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void attn_bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int S, int n_kb, int BH, float scale, int xcd_group) {
  using G = QTileGeo<D, QT>;
  constexpr int DS = D / 16, DB = D / 32, QB = QT / 32, KS = QT / 16;
  static_assert(QT == 32 || QT == 64, "query tiles of 32 or 64 rows");
  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];
  __shared__ __attribute__((aligned(16))) float rows[2][2][QT];  // per stage: lse * log2(e), delta
  // the workgroup's 128 K rows (swizzled like the tiles): the B operand of
  // X = Q K^T, read from LDS each tile instead of held in registers
  __shared__ __attribute__((aligned(16))) char kl[kRows * D * 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  // heaviest first: under the causal rule key block kb is read by the query
  // tiles from its own onwards, so the first key blocks carry the most work
  const BlockCoord bc = schedule_block(blockIdx.x, n_kb, BH, xcd_group);
  const int kblk = n_kb - 1 - bc.qb;
  const size_t head = (size_t)bc.bh * S * D;
  const size_t hrow = (size_t)bc.bh * S;
  const int j0 = kblk * kRows, j0w = j0 + 32 * wave;
  const int kj = j0w + col, kr = min(kj, S - 1);

  // K^T and V^T operands of the lane's key (the B side of X = Q K^T, dP = dO V^T)
  bf16x8_t vreg[DS];
  load_row_operand<D>(vreg, V, head + (size_t)kr * D, half);
  copy_tile<D, kRows>(K + head, j0, S, kl, tid);
  const float c2 = scale * kLog2e;

  f32x16_t dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = (f32x16_t){};
    dvacc[db] = (f32x16_t){};
  }

  const int n_qt = (S + QT - 1) / QT;
  const int t0 = CAUSAL ? j0 / QT : 0;  // the first query tile that sees a key of this block
  // per-row values of a tile: threads 0..QT-1 lse * log2(e), QT..2QT-1 delta
  auto row_value = [&](int q0n) {
    const size_t r = hrow + min(q0n + tid % QT, S - 1);
    return tid < QT ? LSE[r] * kLog2e : (tid < 2 * QT ? Delta[r] : 0.f);
  };
  auto copy_stage = [&](int q0n, int stage) {
    char* st = lds + stage * G::kStageBytes;
    copy_tile<D, QT>(Q + head, q0n, S, st, tid);
    copy_tile<D, QT>(dO + head, q0n, S, st + G::kTileBytes, tid);
  };
  copy_stage(t0 * QT, 0);
  float rv = row_value(t0 * QT);
  if (tid < 2 * QT) rows[0][tid / QT][tid % QT] = rv;
  __builtin_amdgcn_s_waitcnt(common::waitcnt_vm<0>());
  __syncthreads();

  for (int t = t0; t < n_qt; ++t) {
    const int q0 = t * QT, st = (t - t0) & 1;
    const bool has_next = t + 1 < n_qt;
    if (has_next) {  // into the other stage, last read before the previous barrier
      copy_stage(q0 + QT, st ^ 1);
      rv = row_value(q0 + QT);
    }
    const char* Ql = lds + st * G::kStageBytes;
    const char* dOl = Ql + G::kTileBytes;

    const bool live = (!CAUSAL || q0 + QT - 1 >= j0w) && j0w < S;
    if (live) {
      // X = Q K^T and dP = dO V^T (queries down the registers, one key per lane)
      f32x16_t xacc[QB], pacc[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        xacc[qb] = (f32x16_t){};
        pacc[qb] = (f32x16_t){};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          xacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_rows<D>(Ql, qb, ds, col, half),
                                                              tile_rows<D>(kl, wave, ds, col, half), xacc[qb], 0, 0, 0);
          pacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_rows<D>(dOl, qb, ds, col, half), vreg[ds], pacc[qb], 0, 0, 0);
        }
      }
      pipeline_reads<QB * DS, 2, 3, 1>();
      __builtin_amdgcn_sched_barrier(0);
      // P and dS = P * (dP - delta); hidden pairs (key above the query, or a
      // query row past S) give 0
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row4 = 32 * qb + 8 * g + 4 * half;
          const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(&rows[st][0][row4]);
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&rows[st][1][row4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e, qi = q0 + row4 + e;
            const bool hidden = (CAUSAL && kj > qi) || qi >= S;
            const float p = hidden ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(xacc[qb][r], c2, -l4[e]));
            pacc[qb][r] = p * (pacc[qb][r] - d4[e]);
            xacc[qb][r] = p;
          }
        }
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t pb = pack_kstep(xacc, ks);
        const bf16x8_t dsb = pack_kstep(pacc, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_transposed<D>(dOl, db, ks, lane), pb, dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_transposed<D>(Ql, db, ks, lane), dsb, dkacc[db], 0, 0, 0);
        }
      }
      pipeline_reads<KS * DB, 2, 4, 1>();
    }
    if (has_next && tid < 2 * QT) rows[st ^ 1][tid / QT][tid % QT] = rv;
    __builtin_amdgcn_s_waitcnt(common::waitcnt_vm<0>());  // the next tiles have landed
    __syncthreads();
  }
  if (kj < S) {
    store_row<D>(dK, head + (size_t)kj * D, dkacc, scale, half);
    store_row<D>(dV, head + (size_t)kj * D, dvacc, 1.f, half);
  }
}

}  // namespace bwd
}  // namespace fa
