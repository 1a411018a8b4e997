// Tiled online-softmax attention forward in fp32 vector arithmetic.
//
// The fp32 path (and bf16 with small head dims).  One lane owns one query row
// and walks the key/value tiles exactly as the aiml.sh page "Speed up long
// contexts with FlashAttention" describes the method (lab.py,
// tiled_flash_attention): 64-row query blocks, 32-key tiles staged in LDS
// (every lane of the wave reads the same K/V row, an LDS broadcast), the
// causal rule ending the walk at the block's last row, a per-row running
// maximum / sum / accumulator, and a row with no visible key in a tile left
// untouched.  Scores, softmax and accumulation are fp32; each q.k is summed in
// four partial sums and then scaled once by scale * log2(e) (exp in base 2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

constexpr int kValuBQ = 64;   // queries per workgroup (one wave)
constexpr int kValuBK = 32;   // keys per tile

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kValuBQ) void attn_fwd_valu(const T* __restrict__ Q, const T* __restrict__ K,
                                                         const T* __restrict__ V, T* __restrict__ O,
                                                         float* __restrict__ LSE, int S, int n_qb,
                                                         float c_log2) {
  __shared__ float ks[kValuBK][D];
  __shared__ float vs[kValuBK][D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / n_qb;
  const int qb = n_qb - 1 - blockIdx.x % n_qb;  // heaviest blocks first
  const int q0 = qb * kValuBQ;
  const int qi = q0 + tid;
  const size_t head_off = (size_t)bh * S * D;

  float qr[D], acc[D];
  {
    const T* src = Q + head_off + (size_t)min(qi, S - 1) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      qr[c] = to_f32<T>(src[c]);
      acc[c] = 0.f;
    }
  }
  float m = -__builtin_inff(), l = 0.f;

  const int kv_end = CAUSAL ? min(S, q0 + kValuBQ) : S;
  for (int kv0 = 0; kv0 < kv_end; kv0 += kValuBK) {
    __syncthreads();
    for (int idx = tid; idx < kValuBK * D; idx += kValuBQ) {
      const int r = idx / D, c = idx % D;
      const size_t g = head_off + (size_t)min(kv0 + r, S - 1) * D + c;
      ks[r][c] = to_f32<T>(K[g]);
      vs[r][c] = to_f32<T>(V[g]);
    }
    __syncthreads();

    float s[kValuBK];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kValuBK; ++j) {
      // q.k in four interleaved partial sums (shorter rounding chains), then
      // one multiply by scale*log2(e) into the base-2 domain
      float x4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D; ++c) x4[c & 3] = __builtin_fmaf(qr[c], ks[j][c], x4[c & 3]);
      const float x = ((x4[0] + x4[1]) + (x4[2] + x4[3])) * c_log2;
      const int kj = kv0 + j;
      const bool visible = kj < S && (!CAUSAL || kj <= qi);
      s[j] = visible ? x : -__builtin_inff();
      tmax = fmaxf(tmax, s[j]);
    }
    if (tmax == -__builtin_inff()) continue;  // no visible key in this tile for this row
    const float m_new = fmaxf(m, tmax);
    const float alpha = (m == -__builtin_inff()) ? 0.f : exp2f(m - m_new);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kValuBK; ++j) {
      s[j] = exp2f(s[j] - m_new);
      rs += s[j];
    }
    l = l * alpha + rs;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float a = acc[c] * alpha;
#pragma unroll
      for (int j = 0; j < kValuBK; ++j) a = __builtin_fmaf(s[j], vs[j][c], a);
      acc[c] = a;
    }
    m = m_new;
  }

  if (qi < S) {
    const float inv = 1.0f / l;
    T* dst = O + head_off + (size_t)qi * D;
#pragma unroll
    for (int c = 0; c < D; ++c) dst[c] = from_f32<T>(acc[c] * inv);
    if (LSE) LSE[(size_t)bh * S + qi] = (m + log2f(l)) * 0.693147180559945309f;
  }
}

}  // namespace fa
