// Dense, materialising attention forward for gfx950: the standard algorithm
// that the tiled method replaces, run on the GPU as a baseline.
//
// The aiml.sh page "Speed up long contexts with FlashAttention" (lab.py,
// standard_attention) computes every score row s_ij = scale * q_i . k_j, takes
// the row's softmax and then the weighted sum of V rows; its traffic model
// (run-output.txt, hbm_traffic_sweep) charges the N x N score and probability
// matrices to HBM.  These three kernels do exactly that, one pass each:
//
//   dense_scores   S = scale * Q K^T        -> fp32 S x S per head (HBM)
//   dense_softmax  P = softmax(S) per row   -> bf16 S x S per head (HBM), lse
//   dense_pv       O = P V                  -> bf16 [S, D]
//
// Under the causal rule only key tiles at or below the diagonal are computed,
// stored and read (128 x 128 tiles), so the materialised work is the causal
// half plus the diagonal tiles.  Scores and the softmax state are fp32; P is
// normalised, then rounded to bf16 as the P.V operand, like the tiled path.
//
// Workspace layout per (batch, head) of a chunk: the fp32 score matrix, S rows
// of `pitch` floats, then the bf16 probability matrix, S rows of `pitch`
// elements, where pitch = S rounded up to a multiple of 8, so that 16-byte
// accesses stay aligned and a row's padding holds zeros.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"

namespace fa {
namespace dense {

using namespace fa::common;

constexpr int kTile = 128;       // query and key tile (rows of S per block)
constexpr int kThreads = 256;    // 4 waves of 32 rows
constexpr int kRowsPerWave = 32;

__host__ __device__ inline int64_t pitch_of(int64_t S) { return (S + 7) & ~int64_t(7); }

// Workspace bytes for one (batch, head): fp32 scores + bf16 probabilities.
__host__ __device__ inline int64_t head_bytes(int64_t S) { return pitch_of(S) * S * 6; }

// ---------------------------------------------------------------- S = scale * Q K^T
//
// Block: one 128 x 128 tile (query tile qt, key tile kt) of one head.  Wave w
// owns query rows 32w..32w+31 of the tile.  The MFMA A operand is Q (lane l:
// row l%32, dims 16*ds + 8*(l/32) + 0..7, kept in registers) and B is K^T read
// from LDS (lane l: key l%32 of a 32-key block, the same 8 dims), so lane l of
// the result holds keys l%32 of rows 8*(r/4) + 4*(l/32) + r%4: a store of one
// accumulator register writes 32 consecutive floats of two score rows.
template <int D>
struct ScoresGeo {
  static constexpr int kRowBytes = D * 2 + 16;  // padded: conflict-free 128-bit reads of 16 rows
  static constexpr int kLdsBytes = kTile * kRowBytes;
  static constexpr int kChunks = D / 8;         // 16-byte chunks per K row
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void dense_scores(const uint16_t* __restrict__ Q,
                                                         const uint16_t* __restrict__ K,
                                                         float* __restrict__ Sm, int S, int n_qt,
                                                         int64_t pitch, float scale) {
  using G = ScoresGeo<D>;
  constexpr int DS = D / 16;
  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;

  // block -> (head, query tile, key tile); causal blocks enumerate kt <= qt
  const int n_pairs = CAUSAL ? n_qt * (n_qt + 1) / 2 : n_qt * n_qt;
  const int bh = blockIdx.x / n_pairs;
  const int p = blockIdx.x % n_pairs;
  int qt, kt;
  if (CAUSAL) {
    qt = (int)((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
    while ((qt + 1) * (qt + 2) / 2 <= p) ++qt;
    while (qt * (qt + 1) / 2 > p) --qt;
    kt = p - qt * (qt + 1) / 2;
  } else {
    qt = p / n_qt;
    kt = p % n_qt;
  }
  const size_t head = (size_t)bh * S * D;
  const int q0 = qt * kTile, k0 = kt * kTile;

  // K tile -> LDS (rows past S re-read row S-1; their scores are not stored)
  for (int c = tid; c < kTile * G::kChunks; c += kThreads) {
    const int r = c / G::kChunks, ch = c % G::kChunks;
    const int gr = min(k0 + r, S - 1);
    *reinterpret_cast<u32x4_t*>(lds + r * G::kRowBytes + ch * 16) =
        *reinterpret_cast<const u32x4_t*>(K + head + (size_t)gr * D + ch * 8);
  }
  // Q operand straight from HBM
  bf16x8_t qreg[DS];
  {
    const int qrow = min(q0 + kRowsPerWave * wave + col, S - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qreg[ds] = *reinterpret_cast<const bf16x8_t*>(Q + head + (size_t)qrow * D + 16 * ds + 8 * half);
  }
  __syncthreads();

  f32x16_t acc[kTile / 32];
#pragma unroll
  for (int kb = 0; kb < kTile / 32; ++kb) {
    acc[kb] = (f32x16_t){};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8_t b =
          *reinterpret_cast<const bf16x8_t*>(lds + (32 * kb + col) * G::kRowBytes + (16 * ds + 8 * half) * 2);
      acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qreg[ds], b, acc[kb], 0, 0, 0);
    }
  }

  float* const Sh = Sm + (size_t)bh * S * pitch;
#pragma unroll
  for (int kb = 0; kb < kTile / 32; ++kb) {
    const int key = k0 + 32 * kb + col;
    if (key >= S) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = q0 + kRowsPerWave * wave + 8 * (r >> 2) + 4 * half + (r & 3);
      if (qi < S) Sh[(size_t)qi * pitch + key] = acc[kb][r] * scale;
    }
  }
}

// ---------------------------------------------------------------- P = softmax(S), lse
//
// One wave per score row i (keys 0..i under the causal rule, else 0..S-1):
// one pass for the row's maximum and sum (online, per lane, then merged across
// the wave), one pass writing P = exp(s - m) / l in bf16.  The row is then
// zero-filled up to the end of its diagonal key tile (causal) or to the pitch,
// so the P.V kernel can read whole 8-key groups without masking.
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) void dense_softmax(const float* __restrict__ Sm, uint16_t* __restrict__ Pm,
                                                          float* __restrict__ LSE, int S, int64_t pitch,
                                                          int64_t n_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int i = (int)(row % S);
  const int len = CAUSAL ? i + 1 : S;
  const float* srow = Sm + row * pitch;  // rows of all heads are consecutive
  uint16_t* prow = Pm + row * pitch;

  float m = -__builtin_inff(), l = 0.f;
  for (int j = lane; j < len; j += 64) {
    const float x = srow[j];
    if (x > m) {
      l = l * __expf(m - x) + 1.f;
      m = x;
    } else {
      l += __expf(x - m);
    }
  }
  // merge the lanes' (m, l)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const float mn = fmaxf(m, mo);
    l = (m == -__builtin_inff() ? 0.f : l * __expf(m - mn)) + (mo == -__builtin_inff() ? 0.f : lo * __expf(mo - mn));
    m = mn;
  }
  const float inv = 1.f / l;
  for (int j = lane; j < len; j += 64)
    prow[j] = __builtin_bit_cast(uint16_t, (__bf16)(__expf(srow[j] - m) * inv));
  const int64_t pad_end = CAUSAL ? min(pitch, (int64_t)(i / kTile + 1) * kTile) : pitch;
  for (int64_t j = len + lane; j < pad_end; j += 64) prow[j] = 0;
  if (LSE && lane == 0) LSE[row] = m + __logf(l);
}

// ---------------------------------------------------------------- O = P V
//
// Block: 128 query rows of one head, wave w owns rows 32w..32w+31 and walks
// the key tiles (up to the diagonal under the causal rule).  O^T = V^T . P^T:
// the A operand V^T comes from the V tile in LDS through ds_read_b64_tr_b16
// (lane l: dims l%32 of a 32-dim block, keys 8*(l/32) + 0..7 of a 16-key
// step), the B operand P^T is read from HBM (lane l: row l%32, the same 8
// keys, one 16-byte load).  The V tile uses the XOR-swizzled row layout of the
// tiled kernel.
template <int D>
struct PvGeo {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kLdsBytes = kTile * kRowBytes;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void dense_pv(const uint16_t* __restrict__ Pm, const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O, int S, int n_qt, int64_t pitch) {
  using G = PvGeo<D>;
  constexpr int DB = D / 32;
  constexpr int KS = kTile / 16;
  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int u = lane & 15, quad = lane >> 4;
  const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const size_t head = (size_t)bh * S * D;
  const int qi = qt * kTile + kRowsPerWave * wave + col;
  const uint16_t* prow = Pm + ((size_t)bh * S + min(qi, S - 1)) * pitch;

  // transposed-read offsets: lane (group quad, index u) addresses key row
  // 8*half + u/4 (+4 for the upper four keys) and dims 32*db + 16*(quad%2) + 4*(u%4)
  int v_lo[DB], v_hi[DB];
  {
    const int r_lo = 8 * half + (u >> 2), r_hi = r_lo + 4;
    const int c_l = 2 * (quad & 1) + ((u & 3) >> 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      v_lo[db] = r_lo * G::kRowBytes + (((4 * db + c_l) ^ swz<G::kChunks>(r_lo)) << 4) + 8 * (u & 1);
      v_hi[db] = r_hi * G::kRowBytes + (((4 * db + c_l) ^ swz<G::kChunks>(r_hi)) << 4) + 8 * (u & 1);
    }
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
  const int n_kt = CAUSAL ? qt + 1 : n_qt;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * kTile;
    __syncthreads();  // the previous tile's reads are done
    for (int c = tid; c < kTile * G::kChunks; c += kThreads) {
      const int r = c / G::kChunks, ch = c % G::kChunks;
      const int gr = min(k0 + r, S - 1);  // past S: finite values, multiplied by P = 0
      *reinterpret_cast<u32x4_t*>(lds + r * G::kRowBytes + ((ch ^ swz<G::kChunks>(r)) << 4)) =
          *reinterpret_cast<const u32x4_t*>(V + head + (size_t)gr * D + ch * 8);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int key = k0 + 16 * ks + 8 * half;  // this lane's 8 keys of P
      const bf16x8_t pb = key < pitch ? *reinterpret_cast<const bf16x8_t*>(prow + key) : (bf16x8_t){};
      const char* vp = lds + 16 * ks * G::kRowBytes;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + v_lo[db]));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + v_hi[db]));
        const bf16x8_t av = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                                    __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, oacc[db], 0, 0, 0);
      }
    }
  }

  if (qi < S) {
    uint16_t* orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4_t v4 = {oacc[db][4 * rg + 0], oacc[db][4 * rg + 1], oacc[db][4 * rg + 2], oacc[db][4 * rg + 3]};
        *reinterpret_cast<bf16x4_t*>(orow + 32 * db + 8 * rg + 4 * half) = __builtin_convertvector(v4, bf16x4_t);
      }
  }
}

}  // namespace dense
}  // namespace fa
