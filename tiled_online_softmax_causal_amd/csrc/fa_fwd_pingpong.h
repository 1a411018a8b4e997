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
// where the matrix phase t issues O^T += V_{t-1}^T P_{t-1}^T and
// S_t^T = K_t Q^T on the matrix cores (32 MFMAs for d = 128) and the softmax
// phase t turns S_t into bf16 probabilities on the vector ALUs.  Every SIMD
// thus always holds one wave feeding its matrix core and one wave doing the
// exponentials, the two kinds of work overlap, and one workgroup barrier closes
// each phase.
//
// Data movement.  K and V tiles (64 keys) are fetched HBM -> registers at the
// start of an even phase and written to LDS at the end of the following odd
// phase, two phases after the fetch, into the other half of a double buffer
// (so up to ~2 phases of load latency are hidden).  LDS rows are XOR-swizzled
// in 16-byte chunks, chunk' = chunk ^ (2*(row%4) + (row/4)%2): the 8 lanes of a
// 128-bit K read and the 16 lanes of a 64-bit transposed V read then hit
// distinct banks.
//
// Register layout (v_mfma_f32_32x32x16_bf16).  Scores are formed transposed,
// S^T = K . Q^T, so each lane owns ONE query (column lane%32) and half of the
// tile's keys (rows 8*(r/4) + 4*(lane/32) + r%4 of each 32-key block); row
// max and row sum are lane-local plus one v_permlane32_swap.  The fp32 scores,
// exponentiated and packed to bf16, are already the B operand of
// O^T = V^T . P^T; V^T comes from LDS through ds_read_b64_tr_b16 in the
// matching key order.
//
// Softmax.  Base 2: c = scale*log2(e) is folded into one FMA per score and exp
// is v_exp_f32.  The running maximum is moved lazily: only when a tile's
// maximum exceeds it by more than 8 (a factor 256) are the accumulator and the
// sum rescaled.  Otherwise the stale maximum stays, probabilities may reach
// 256, and since numerator and denominator share it the result is unchanged.
// The denominator is an fp32 sum of the fp32 probabilities (the log-sum-exp
// keeps fp32 accuracy); only the P.V operand is rounded to bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr int kQW = 32;                 // query rows per wave
constexpr int kBQ = kQW * kWaves;       // query rows per workgroup
constexpr int kBK = 64;                 // keys per tile
constexpr float kLazyRescale = 8.0f;    // log2 of the growth that forces a rescale
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "matrix-core path covers D = 64 and 128");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
  static constexpr int kTileBytes = kBK * kRowBytes;       // one K or V tile
  static constexpr int kChunksPerThread = kBK * kChunks / kThreads;
  static_assert(kBK * kChunks % kThreads == 0, "a tile must split evenly over the workgroup");
};

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

template <int D>
__device__ __forceinline__ int chunk_offset(int row, int chunk) {
  return row * Geo<D>::kRowBytes + ((chunk ^ swz(row)) << 4);
}

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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_pingpong(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int S, int n_qb, float c_log2, int negate_q,
    int xcd_group) {
  using G = Geo<D>;
  constexpr int DS = D / 16;  // k-steps of the score MFMA
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int NC = G::kChunksPerThread;

  __shared__ __attribute__((aligned(16))) char lds[4 * G::kTileBytes];  // K[2], V[2]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int grp = wave >> 2;   // 0: matrix phase first, 1: one phase behind
  const int col = lane & 31;   // the query this lane owns, within the wave
  const int half = lane >> 5;  // which key half of each 32-key block
  const int u = lane & 15, quad = lane >> 4;

  int bh, qb;
  schedule_block(blockIdx.x, n_qb, xcd_group, bh, qb);
  const size_t head_off = (size_t)bh * S * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;
  const int q0 = qb * kBQ;
  const int q0w = q0 + wave * kQW;

  // ---- Q^T operand: lane holds q[q0w + col][16*ds + 8*half + 0..7]
  bf16x8_t qreg[DS];
  {
    const int qrow = min(q0w + col, S - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(Qh + (size_t)qrow * D + 16 * ds + 8 * half);
      if (negate_q) x ^= (u32x4_t){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
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

  // ---- staging: HBM -> registers -> LDS.  Thread tid owns LDS chunks tid,
  // tid + 512, ...; its source is the logical chunk that the swizzle puts there.
  // Rows past the end of the sequence re-read row S-1 (their scores are masked).
  u32x4_t kst[NC], vst[NC];
  auto fetch = [&](u32x4_t* dst, const uint16_t* src, int t) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int slot = i * kThreads + tid;
      const int row = slot / G::kChunks;
      const int lch = (slot % G::kChunks) ^ swz(row);
      const int grow = min(t * kBK + row, S - 1);
      dst[i] = *reinterpret_cast<const u32x4_t*>(src + (size_t)grow * D + lch * 8);
    }
  };
  auto deposit = [&](char* buf, const u32x4_t* src) {
#pragma unroll
    for (int i = 0; i < NC; ++i) *reinterpret_cast<u32x4_t*>(buf + (i * kThreads + tid) * 16) = src[i];
  };
  char* const kbuf0 = lds;
  char* const vbuf0 = lds + 2 * G::kTileBytes;

  // ---- matrix phase t: O^T += V_{t-1}^T P_{t-1}^T, then S_t^T = K_t Q^T
  auto matrix_phase = [&](int t) {
    if (t >= 1 && t - 1 < n_w) {
      const char* Vl = vbuf0 + ((t - 1) & 1) * G::kTileBytes;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int vcol = 32 * db + 16 * (quad & 1) + 4 * (u & 3);
        const int vchunk = vcol >> 3, vbyte = (vcol & 7) * 2;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int vrow0 = 16 * ks + 4 * half + (u >> 2);
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(Vl + chunk_offset<D>(vrow0, vchunk) + vbyte));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(Vl + chunk_offset<D>(vrow0 + 8, vchunk) + vbyte));
          const bf16x8_t av = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                                      __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], oacc[db], 0, 0, 0);
        }
      }
    }
    if (t < n_w) {
      const char* Kl = kbuf0 + (t & 1) * G::kTileBytes;
      sacc[0] = (f32x16_t){};
      sacc[1] = (f32x16_t){};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Kl + chunk_offset<D>(32 * kb + col, 2 * ds + half));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], sacc[kb], 0, 0, 0);
        }
    }
  };

  // ---- softmax phase t: S_t -> bf16 P_t, running max / sum
  auto softmax_phase = [&](int t) {
    if (t < 0 || t >= n_w) return;
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
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[kb][r], sacc[kb][r + 1]));
    const float mt = max_halves(mx) * c_t;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazyRescale)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
    float rs = 0.f;
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
    l_run += rs;
  };

  // ---- prologue: K_0 into LDS
  if (n_tiles > 0) {
    fetch(kst, Kh, 0);
    deposit(kbuf0, kst);
  }
  lds_barrier();

  // ---- 2 * (n_tiles + 1) phases, one barrier each.  The two groups run the
  // same phases with their roles swapped; each has its own straight loop.
  if (grp == 0) {
    for (int t = 0; t <= n_tiles; ++t) {
      if (t + 1 < n_tiles) fetch(kst, Kh, t + 1);
      if (t < n_tiles) fetch(vst, Vh, t);
      matrix_phase(t);  // phase 2t
      lds_barrier();
      softmax_phase(t);  // phase 2t + 1
      if (t + 1 < n_tiles) deposit(kbuf0 + ((t + 1) & 1) * G::kTileBytes, kst);
      if (t < n_tiles) deposit(vbuf0 + (t & 1) * G::kTileBytes, vst);
      lds_barrier();
    }
  } else {
    for (int t = 0; t <= n_tiles; ++t) {
      if (t + 1 < n_tiles) fetch(kst, Kh, t + 1);
      if (t < n_tiles) fetch(vst, Vh, t);
      softmax_phase(t - 1);  // phase 2t
      lds_barrier();
      matrix_phase(t);  // phase 2t + 1
      if (t + 1 < n_tiles) deposit(kbuf0 + ((t + 1) & 1) * G::kTileBytes, kst);
      if (t < n_tiles) deposit(vbuf0 + (t & 1) * G::kTileBytes, vst);
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
