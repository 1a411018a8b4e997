// Tiled online-softmax attention forward on the gfx950 matrix cores (bf16 in, fp32 state).
//
// The method is the one of the aiml.sh page "Speed up long contexts with
// FlashAttention" (lab.py, tiled_flash_attention): query row blocks stay on
// chip, key/value blocks stream through, and each row keeps a running maximum,
// a running sum and an accumulator that is rescaled whenever the maximum grows.
// Key blocks wholly above the diagonal are never visited; blocks that straddle
// it are masked per element.  What changes for CDNA4:
//
//  * Both contractions run on v_mfma_f32_32x32x16_bf16.  The score tile is
//    formed transposed, S^T = K . Q^T, so the accumulator layout puts ONE QUERY
//    PER LANE (column = lane % 32) and keys down the 16 accumulator registers
//    (row = 8*(r/4) + 4*(lane/32) + r%4).  Row max and row sum are then
//    reductions over a lane's own registers plus one v_permlane32_swap between
//    the two half-waves, instead of cross-lane shuffles per element.
//  * The probabilities never leave registers: the accumulator registers of
//    S^T, packed to bf16, are exactly the B operand of O^T = V^T . P^T for the
//    next MFMA (lane holds 8 consecutive k-slots of one query).  The key
//    order inside a k-step (4*(lane/32) + {0..3}, then 8 + ...) is matched on
//    the V side by ds_read_b64_tr_b16, which reads V row-major from LDS and
//    returns it transposed: within each 16-lane group, lane t receives
//    element t%4 of the 4-element rows addressed by lanes t/4, t/4+4, t/4+8,
//    t/4+12.
//  * Each wave owns NSUB x 32 queries, so that every K and V operand read
//    from LDS feeds NSUB MFMAs.  The library instantiates NSUB = 1 only: 128
//    query rows per 4-wave workgroup, two workgroups per CU (this kernel is the
//    128-row tiling; the 256-row ping-pong kernel is the hot path).
//  * K and V tiles are staged HBM -> registers -> LDS (global loads into
//    VGPRs, then LDS stores), double buffered, one barrier per tile; the
//    ping-pong and short-sequence kernels copy HBM -> LDS directly instead.
//    LDS rows are XOR-swizzled in 16-byte chunks,
//    chunk' = chunk ^ f(row) with f(row) = 4*(row%4) + (row/4)%4, so the 16
//    lanes of a 128-bit K read (16 consecutive rows) and the 32 lanes of a
//    64-bit transposed V read (4 rows x 64 bytes) hit distinct banks of a
//    64-bank LDS.
//  * The softmax runs in the base-2 domain: c = scale * log2(e) is folded into
//    one FMA per score, exp is v_exp_f32, and the log-sum-exp is converted back
//    to natural log at the end.  A negative scale is handled by negating Q at
//    load (exact in bf16) and using |c|.
//  * The O^T rescale by alpha is skipped when no lane's maximum moved (then
//    alpha == 1 exactly, so the result is bit-identical).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;  // keys per tile
constexpr float kLn2 = 0.693147180559945309f;

// Geometry of one K or V tile of BK keys in LDS for head dim D (bf16).
template <int D, int BK = kBK>
struct TileGeo {
  static_assert(D == 64 || D == 128, "matrix-core path covers D = 64 and 128");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row (8 or 16)
  static constexpr int kTileBytes = BK * kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;  // K tile then V tile
  static constexpr int kLdsBytes = 2 * kStageBytes;   // two stages
  static constexpr int kLoadsPerThread = BK * kChunks / kThreads;  // per tensor
  static_assert(BK * kChunks % kThreads == 0, "tile must split evenly over the workgroup");
};

// XOR key of a row's 16-byte chunks, masked to the row's chunk count.
template <int D>
__device__ __forceinline__ int lds_swizzle(int row) {
  return (((row & 3) << 2) | ((row >> 2) & 3)) & (TileGeo<D>::kChunks - 1);
}

// Byte offset of logical 16-byte chunk `chunk` of row `row` in a swizzled tile.
template <int D>
__device__ __forceinline__ int lds_chunk_offset(int row, int chunk) {
  return row * TileGeo<D>::kRowBytes + ((chunk ^ lds_swizzle<D>(row)) << 4);
}

__device__ __forceinline__ float wave_max_halves(float x) {
  // lanes 0-31 and 32-63 hold the two key halves of the same 32 queries
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float wave_sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Maps a workgroup id to (bh, query block).  Heaviest query blocks first (under
// the causal rule block qb visits qb+1 key ranges).  When the head count allows,
// every query block of a head lands on the same XCD (workgroups are dispatched
// round-robin over the 8 XCDs), so that head's K/V prefix is fetched into that
// XCD's L2 once and shared by the blocks running there together.
struct BlockCoord {
  int bh, qb;
};
__device__ __forceinline__ BlockCoord schedule_block(int wg, int n_qb, int BH, int xcd_group) {
  BlockCoord c;
  if (xcd_group) {
    const int xcd = wg & 7, idx = wg >> 3;
    c.bh = (idx / n_qb) * 8 + xcd;
    c.qb = n_qb - 1 - idx % n_qb;
  } else {
    c.bh = wg / n_qb;
    c.qb = n_qb - 1 - wg % n_qb;
  }
  return c;
}

template <int D, int BK = kBK>
struct TileStager {
  static constexpr int L = TileGeo<D, BK>::kLoadsPerThread;
  u32x4_t kr[L], vr[L];

  // HBM -> registers.  Thread tid owns LDS chunks tid, tid+256, ... (row-major
  // over the swizzled tile), so its source is the logical chunk that lands there.
  // Rows past the end of the sequence re-read row S-1 (masked later).
  __device__ __forceinline__ void load(const uint16_t* __restrict__ Kh, const uint16_t* __restrict__ Vh,
                                       int kv0, int S, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int cidx = i * kThreads + tid;
      const int row = cidx / TileGeo<D>::kChunks;
      const int pch = cidx % TileGeo<D>::kChunks;
      const int lch = pch ^ lds_swizzle<D>(row);
      const int grow = min(kv0 + row, S - 1);
      const size_t off = (size_t)grow * D + lch * 8;
      kr[i] = *reinterpret_cast<const u32x4_t*>(Kh + off);
      vr[i] = *reinterpret_cast<const u32x4_t*>(Vh + off);
    }
  }
  __device__ __forceinline__ void store(char* stage, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int cidx = i * kThreads + tid;
      *reinterpret_cast<u32x4_t*>(stage + cidx * 16) = kr[i];
      *reinterpret_cast<u32x4_t*>(stage + TileGeo<D, BK>::kTileBytes + cidx * 16) = vr[i];
    }
  }
};

// BK: keys per tile.  64-key tiles fit two workgroups per CU (two waves per
// SIMD); 128-key tiles take 128 KB of LDS, so one.
template <int D, int NSUB, bool CAUSAL, int BK = kBK>
__global__ __launch_bounds__(kThreads, (NSUB == 1 && BK == 64 ? 2 : 1)) void attn_fwd_mfma_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int S, int n_qb, int BH, float c_log2,
    int negate_q, int xcd_group) {
  using G = TileGeo<D, BK>;
  constexpr int QW = 32 * NSUB;      // queries per wave
  constexpr int BQ = QW * kWaves;    // queries per workgroup
  constexpr int DS = D / 16;         // k-steps of the score MFMA
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int KB = BK / 32;       // 32-key blocks of S^T
  constexpr int KS = BK / 16;       // k-steps of the PV MFMA

  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query within a 32-query sub-block
  const int half = lane >> 5;

  const BlockCoord bc = schedule_block(blockIdx.x, n_qb, BH, xcd_group);
  const size_t head_off = (size_t)bc.bh * S * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;
  const int q0 = bc.qb * BQ;
  const int q0w = q0 + wave * QW;  // first query of this wave

  // Q^T operand: lane holds q[query = q0w + 32*sb + col][16*ds + 8*half + 0..7]
  bf16x8_t qreg[NSUB][DS];
#pragma unroll
  for (int sb = 0; sb < NSUB; ++sb) {
    const int qrow = min(q0w + 32 * sb + col, S - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(Qh + (size_t)qrow * D + 16 * ds + 8 * half);
      if (negate_q) x ^= (u32x4_t){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qreg[sb][ds] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t oacc[NSUB][DB];
  float m_run[NSUB], l_run[NSUB];
#pragma unroll
  for (int sb = 0; sb < NSUB; ++sb) {
    m_run[sb] = -__builtin_inff();
    l_run[sb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[sb][db] = (f32x16_t){};
  }

  const int kv_end = CAUSAL ? min(S, q0 + BQ) : S;
  const int n_tiles = (kv_end + BK - 1) / BK;

  TileStager<D, BK> stager;
  stager.load(Kh, Vh, 0, S, tid);
  stager.store(lds, tid);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * BK;
    const bool has_next = t + 1 < n_tiles;
    if (has_next) stager.load(Kh, Vh, kv0 + BK, S, tid);

    const char* Kl = lds + (t & 1) * G::kStageBytes;
    const char* Vl = Kl + G::kTileBytes;

    // A wave whose queries all lie before this tile's first key has nothing to do.
    const bool wave_live = (!CAUSAL || kv0 <= q0w + QW - 1) && q0w < S;
    if (wave_live) {
      // ---- S^T = K . Q^T for each sub-block and 32-key block
      f32x16_t sacc[NSUB][KB];
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[sb][kb] = (f32x16_t){};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = 32 * kb + col;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8_t a =
              *reinterpret_cast<const bf16x8_t*>(Kl + lds_chunk_offset<D>(row, 2 * ds + half));
#pragma unroll
          for (int sb = 0; sb < NSUB; ++sb)
            sacc[sb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[sb][ds], sacc[sb][kb], 0, 0, 0);
        }
      }

      // ---- mask: only tiles that straddle the diagonal or run past S.  These
      // tiles are moved to the base-2 domain here (c_t = 1 afterwards), so a
      // hidden score is a plain -inf even when the scale is 0.
      const bool need_mask = (CAUSAL && kv0 + BK - 1 > q0w) || (kv0 + BK > S);
      float c_t = c_log2;
      if (need_mask) {
        c_t = 1.f;
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
          const int qi = q0w + 32 * sb + col;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kj = kv0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
              const bool hidden = (CAUSAL && kj > qi) || kj >= S;
              sacc[sb][kb][r] = hidden ? -__builtin_inff() : sacc[sb][kb][r] * c_log2;
            }
        }
      }

      // ---- online softmax (base 2), lane-local per query
      bf16x8_t pb[NSUB][KS];
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][kb][r]);
        mx = wave_max_halves(mx);
        const float m_new = fmaxf(m_run[sb], mx * c_t);
        const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[sb] - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sb][kb][r], c_t, -m_use));
            sacc[sb][kb][r] = p;
            rs += p;
          }
        l_run[sb] = l_run[sb] * alpha + rs;
        if (__builtin_amdgcn_ballot_w64(m_new != m_run[sb])) {
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[sb][db] *= alpha;
        }
        m_run[sb] = m_new;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int kb = ks >> 1, r0 = 8 * (ks & 1);
          f32x8_t p8;
#pragma unroll
          for (int e = 0; e < 8; ++e) p8[e] = sacc[sb][kb][r0 + e];
          pb[sb][ks] = __builtin_convertvector(p8, bf16x8_t);
        }
      }

      // ---- O^T += V^T . P^T ; V^T operand via transposed LDS reads
      const int u = lane & 15, grp = lane >> 4;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int vcol = 32 * db + 16 * (grp & 1) + 4 * (u & 3);
        const int vchunk = vcol >> 3, vbyte = (vcol & 7) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int vrow0 = 16 * ks + 4 * half + (u >> 2);
          const int vrow1 = vrow0 + 8;
          typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(Vl + lds_chunk_offset<D>(vrow0, vchunk) + vbyte));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(Vl + lds_chunk_offset<D>(vrow1, vchunk) + vbyte));
          const bf16x4_t lo4 = __builtin_bit_cast(bf16x4_t, lo);
          const bf16x4_t hi4 = __builtin_bit_cast(bf16x4_t, hi);
          const bf16x8_t av = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int sb = 0; sb < NSUB; ++sb)
            oacc[sb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[sb][ks], oacc[sb][db], 0, 0, 0);
        }
      }
    }

    if (has_next) stager.store(lds + ((t + 1) & 1) * G::kStageBytes, tid);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (bf16, round to nearest even), lse = ln2 * (m + log2 l)
#pragma unroll
  for (int sb = 0; sb < NSUB; ++sb) {
    const int qi = q0w + 32 * sb + col;
    const float l_tot = wave_sum_halves(l_run[sb]);
    if (qi < S) {
      const float inv = 1.0f / l_tot;
      uint16_t* orow = O + head_off + (size_t)qi * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          f32x4_t v4 = {oacc[sb][db][4 * rg + 0] * inv, oacc[sb][db][4 * rg + 1] * inv,
                        oacc[sb][db][4 * rg + 2] * inv, oacc[sb][db][4 * rg + 3] * inv};
          const bf16x4_t b4 = __builtin_convertvector(v4, bf16x4_t);
          *reinterpret_cast<bf16x4_t*>(orow + 32 * db + 8 * rg + 4 * half) = b4;
        }
      if (LSE && half == 0) LSE[(size_t)bc.bh * S + qi] = (m_run[sb] + log2f(l_tot)) * kLn2;
    }
  }
}

}  // namespace fa
