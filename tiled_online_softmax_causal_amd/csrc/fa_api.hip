// C ABI of the attention forward library: argument checks, kernel choice,
// causal tile scheduling and launch.  Declarations and the contract are in
// include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "fa_bwd.h"
#include "fa_dense.h"
#include "fa_fwd_pingpong.h"
#include "fa_mfma_bf16.h"
#include "fa_split.h"
#include "fa_valu.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNumXcd = 8;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t mfma_block_q(int variant) {
  if (variant == FA_VARIANT_SPLIT) return fa::split::kBQ;
  return variant == FA_VARIANT_MFMA_B256 || variant == FA_VARIANT_MFMA_B256_K128 ? fa::pp::kBQ : 4 * 32;
}

int64_t mfma_block_k(int variant) {
  if (variant == FA_VARIANT_SPLIT) return fa::split::kBK;
  return variant == FA_VARIANT_MFMA_B256_K128 || variant == FA_VARIANT_MFMA_B128_K128 ? 128 : fa::kBK;
}

// Whether a variant runs (D, dtype, S).  The ping-pong kernels copy whole key
// tiles (a last tile cut short is copied as the sequence's last BK rows), so
// they take S >= BK.
bool variant_covers(int variant, int64_t D, fa_dtype dtype, int64_t S) {
  switch (variant) {
    case FA_VARIANT_MFMA_B256:
    case FA_VARIANT_MFMA_B256_K128:
      return dtype == FA_DTYPE_BF16 && (D == 64 || D == 128) &&
             S >= (variant == FA_VARIANT_MFMA_B256_K128 ? 128 : 64);
    case FA_VARIANT_MFMA_B128:
    case FA_VARIANT_MFMA_B128_K128:
    case FA_VARIANT_SPLIT:
      return dtype == FA_DTYPE_BF16 && (D == 64 || D == 128);
    case FA_VARIANT_VALU:
      return (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_FP32) && (D == 16 || D == 32 || D == 64 || D == 128);
    default:
      return false;
  }
}

// Shape-only choice (for the 256 CUs of an MI355X): bf16 with D 64/128 runs
// on the matrix cores, in 256-row workgroups (one per CU) with 128-key tiles
// unless that leaves CUs idle (fewer 256-row items than CUs) or S < 128 (the
// kernel takes whole 128-key tiles).  Then the split kernel runs pairs of
// 64-row blocks with four key streams per workgroup while its units (about
// one per 128 rows of a head) fit on the CUs at once.  Between the two
// (measured at 1152 <= S <= 7000 over several head counts) the 128-row kernel
// was the slowest of the three: at d = 128 the 256-row kernel is taken below
// S = 2048 and the split kernel (in more than one round of units) from there,
// at d = 64 the split kernel throughout; the 128-row kernel only below 128
// keys.
int select_variant(int64_t B, int64_t H, int64_t S, int64_t D, fa_dtype dtype) {
  if (dtype == FA_DTYPE_BF16 && (D == 64 || D == 128)) {
    constexpr int64_t kCUs = 256;
    // at d = 64 one 256-row item per CU (items == CUs) still ran 10-14% slower
    // than the split kernel's two rounds of units; from 384 items on it ran faster
    const int64_t items = B * H * ceil_div(S, mfma_block_q(FA_VARIANT_MFMA_B256_K128));
    if (S >= 128 && (D == 64 ? items > kCUs : items >= kCUs)) {
      // rows shorter than 384 keys with at most 384 heads: the 128-row kernel
      // (two workgroups per CU, no ping-pong start-up per item) ran 4-30%
      // faster (b4 h80 and b8 h48 at S 128-320); with 512 heads at S 256 it
      // ran 16% slower
      if (S < 384 && B * H <= 384) return FA_VARIANT_MFMA_B128;
      return FA_VARIANT_MFMA_B256_K128;
    }
    if (B * H * ceil_div(S, 2 * fa::split::kBQ) <= kCUs) return FA_VARIANT_SPLIT;
    if (S < 128) return FA_VARIANT_MFMA_B128;
    return D == 64 || S >= 2048 ? FA_VARIANT_SPLIT : FA_VARIANT_MFMA_B256_K128;
  }
  if (variant_covers(FA_VARIANT_VALU, D, dtype, S)) return FA_VARIANT_VALU;
  return -1;
}

template <int D, int NSUB, int BK = fa::kBK>
hipError_t launch_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                       int64_t S, int causal, float scale, hipStream_t stream) {
  const int64_t bq = 4 * 32 * NSUB;
  const int64_t n_qb = ceil_div(S, bq);
  const int64_t grid = BH * n_qb;
  const int xcd_group = (BH % kNumXcd) == 0;
  const float c = std::fabs(scale) * kLog2e;
  const int negate_q = scale < 0.f;
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  auto* O = static_cast<uint16_t*>(o);
  if (causal)
    hipLaunchKernelGGL((fa::attn_fwd_mfma_bf16<D, NSUB, true, BK>), dim3((unsigned)grid), dim3(fa::kThreads), 0,
                       stream, Q, K, V, O, lse, (int)S, (int)n_qb, (int)BH, c, negate_q, xcd_group);
  else
    hipLaunchKernelGGL((fa::attn_fwd_mfma_bf16<D, NSUB, false, BK>), dim3((unsigned)grid), dim3(fa::kThreads), 0,
                       stream, Q, K, V, O, lse, (int)S, (int)n_qb, (int)BH, c, negate_q, xcd_group);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// The schedule of the ping-pong grid (fa_schedule.h).  With more items than
// CUs the grid is resident (one workgroup per CU walking a static list).  The
// list order is the head-major snake unless the block-major one models at
// least 3% less time for the busiest workgroup: head-major keeps an XCD's
// workgroups on fewer heads' K/V at once.  The choice is cached per shape.
fa::sched::Plan make_plan(int64_t BH, int64_t n_qb, int64_t grid, int64_t S, int causal, int BK, bool balanced) {
  namespace sc = fa::sched;
  const int64_t n_items = BH * n_qb;
  sc::Plan p{sc::kOne, (int)grid, (int)n_qb, (int)BH, 0};
  if (grid >= n_items) return p;
  const bool grouped = BH % kNumXcd == 0 && grid % kNumXcd == 0;
  const int hx = (int)(BH / kNumXcd);
  p.hs = grouped ? hx : 0;
  // The order is chosen on the full static lists, the same with or without the
  // balanced schedule's pool.
  struct Key {
    int64_t BH, n_qb, grid, S;
    int causal, BK, grouped, pad;
  };
  thread_local Key last{-1, 0, 0, 0, 0, 0, 0, 0};
  thread_local int last_order = sc::kXcdHead;
  const Key key{BH, n_qb, grid, S, causal, BK, grouped, 0};
  if (std::memcmp(&key, &last, sizeof key) == 0) {
    p.order = last_order;
  } else {
    // per-item overhead: about 2.3 key tiles of 128 keys
    const double item_cost = 2.3 * 128.0 / BK;
    sc::Plan head = p, block = p;
    head.order = grouped ? sc::kXcdHead : sc::kFlatHead;
    block.order = grouped ? sc::kXcdBlock : sc::kFlatBlock;
    const double th = sc::plan_makespan(head, (int)S, fa::pp::kBQ, BK, causal != 0, item_cost);
    const double tb = sc::plan_makespan(block, (int)S, fa::pp::kBQ, BK, causal != 0, item_cost);
    p.order = tb < 0.97 * th ? block.order : head.order;
    last = key;
    last_order = p.order;
  }
  // the balanced schedule pools the last eighth of each XCD's heads
  if (balanced) p.hs = hx - std::max(1, hx / 8);
  return p;
}

// The ping-pong kernel holds a whole CU (LDS), so with more work items than
// CUs it runs resident: one workgroup per CU walking its items, instead of a
// grid of one workgroup per item that the dispatcher refills as they finish.
// With a schedule workspace (sched) and heads grouped per XCD, the resident
// grid balances the last part of its work across XCDs (the balanced schedule
// in fa_fwd_pingpong.h); otherwise the schedule is static.
template <int D, int BK>
hipError_t launch_pingpong(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                           int64_t S, int causal, float scale, unsigned* sched, hipStream_t stream) {
  const int64_t n_qb = ceil_div(S, fa::pp::kBQ);
  const int64_t n_items = BH * n_qb;
  const int cus = device_cus();
  const int64_t grid = cus >= 8 && n_items > cus ? cus : n_items;
  // balanced: a resident grid over whole XCDs with at least 8 heads per XCD
  const bool balanced = sched && BH % kNumXcd == 0 && grid < n_items && grid % kNumXcd == 0 &&
                        grid <= fa::pp::kSchedMaxGrid && BH >= 8 * kNumXcd;
  const fa::sched::Plan plan = make_plan(BH, n_qb, grid, S, causal, BK, balanced);
  const float c = scale * kLog2e;  // the kernel takes a scale of either sign
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  auto* O = static_cast<uint16_t*>(o);
  const dim3 g((unsigned)grid), b(fa::pp::kThreads);
  const int s = (int)S;
  if (balanced) {
    if (causal)
      hipLaunchKernelGGL((fa::pp::attn_fwd_pingpong<D, BK, true, true>), g, b, 0, stream, Q, K, V, O, lse, s, c, plan,
                         sched);
    else
      hipLaunchKernelGGL((fa::pp::attn_fwd_pingpong<D, BK, false, true>), g, b, 0, stream, Q, K, V, O, lse, s, c, plan,
                         sched);
  } else if (causal) {
    hipLaunchKernelGGL((fa::pp::attn_fwd_pingpong<D, BK, true, false>), g, b, 0, stream, Q, K, V, O, lse, s, c, plan,
                       nullptr);
  } else {
    hipLaunchKernelGGL((fa::pp::attn_fwd_pingpong<D, BK, false, false>), g, b, 0, stream, Q, K, V, O, lse, s, c, plan,
                       nullptr);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t S,
                        int causal, float scale, hipStream_t stream) {
  namespace sp = fa::split;
  const int64_t n_qb = ceil_div(S, sp::kBQ);
  const int64_t grid = BH * sp::units_per_head((int)n_qb, causal != 0);
  const int xcd_group = (BH % kNumXcd) == 0;
  const float c = std::fabs(scale) * kLog2e;
  const int negate_q = scale < 0.f;
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  auto* O = static_cast<uint16_t*>(o);
  if (causal)
    hipLaunchKernelGGL((sp::attn_fwd_split<D, true>), dim3((unsigned)grid), dim3(sp::kThreads), 0, stream, Q, K, V,
                       O, lse, (int)S, (int)n_qb, (int)BH, c, negate_q, xcd_group);
  else
    hipLaunchKernelGGL((sp::attn_fwd_split<D, false>), dim3((unsigned)grid), dim3(sp::kThreads), 0, stream, Q, K, V,
                       O, lse, (int)S, (int)n_qb, (int)BH, c, negate_q, xcd_group);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t S,
                       int causal, float scale, hipStream_t stream) {
  const int64_t n_qb = ceil_div(S, fa::kValuBQ);
  const int64_t grid = BH * n_qb;
  const float c = scale * kLog2e;
  const auto* Q = static_cast<const T*>(q);
  const auto* K = static_cast<const T*>(k);
  const auto* V = static_cast<const T*>(v);
  auto* O = static_cast<T*>(o);
  if (causal)
    hipLaunchKernelGGL((fa::attn_fwd_valu<T, D, true>), dim3((unsigned)grid), dim3(fa::kValuBQ), 0, stream, Q, K,
                       V, O, lse, (int)S, (int)n_qb, c);
  else
    hipLaunchKernelGGL((fa::attn_fwd_valu<T, D, false>), dim3((unsigned)grid), dim3(fa::kValuBQ), 0, stream, Q, K,
                       V, O, lse, (int)S, (int)n_qb, c);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_valu_d(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t S,
                         int64_t D, int causal, float scale, hipStream_t stream) {
  switch (D) {
    case 16: return launch_valu<T, 16>(q, k, v, o, lse, BH, S, causal, scale, stream);
    case 32: return launch_valu<T, 32>(q, k, v, o, lse, BH, S, causal, scale, stream);
    case 64: return launch_valu<T, 64>(q, k, v, o, lse, BH, S, causal, scale, stream);
    default: return launch_valu<T, 128>(q, k, v, o, lse, BH, S, causal, scale, stream);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_dense(const void* q, const void* k, const void* v, void* o, float* lse, int64_t nb, int64_t S,
                        float scale, float* smat, uint16_t* pmat, hipStream_t stream) {
  namespace dn = fa::dense;
  const int n_qt = (int)ceil_div(S, dn::kTile);
  const int64_t pitch = dn::pitch_of(S);
  const int64_t n_pairs = CAUSAL ? (int64_t)n_qt * (n_qt + 1) / 2 : (int64_t)n_qt * n_qt;
  hipLaunchKernelGGL((dn::dense_scores<D, CAUSAL>), dim3((unsigned)(nb * n_pairs)), dim3(dn::kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), smat, (int)S, n_qt, pitch,
                     scale);
  const int64_t n_rows = nb * S;
  hipLaunchKernelGGL((dn::dense_softmax<CAUSAL>), dim3((unsigned)ceil_div(n_rows, dn::kThreads / 64)),
                     dim3(dn::kThreads), 0, stream, smat, pmat, lse, (int)S, pitch, n_rows);
  hipLaunchKernelGGL((dn::dense_pv<D, CAUSAL>), dim3((unsigned)(nb * n_qt)), dim3(dn::kThreads), 0, stream, pmat,
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), (int)S, n_qt, pitch);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int64_t BH, int64_t S, float scale,
                      float* delta, hipStream_t stream) {
  namespace bw = fa::bwd;
  const int64_t nb = ceil_div(S, bw::kRows);  // query blocks (dQ) and key blocks (dK/dV) per head
  const int64_t grid = BH * nb;
  const int xcd_group = (BH % kNumXcd) == 0;
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  const auto* dO = static_cast<const uint16_t*>(dout);
  // two workgroups per CU (two waves per SIMD), so one wave's exponentials and
  // dS products overlap the other's MFMAs.  At d = 128 the key-side kernel fits
  // that register budget only with 32-row query tiles.
  constexpr int kOcc = 2, kQT = D == 128 ? 32 : 64;
  hipLaunchKernelGGL((bw::attn_bwd_dq<D, CAUSAL, kOcc>), dim3((unsigned)grid), dim3(fa::kThreads), 0, stream, Q, K, V,
                     static_cast<const uint16_t*>(o), dO, lse, static_cast<uint16_t*>(dq), delta, (int)S, (int)nb,
                     (int)BH, scale, xcd_group);
  hipLaunchKernelGGL((bw::attn_bwd_dkdv<D, CAUSAL, kQT, kOcc>), dim3((unsigned)grid), dim3(fa::kThreads), 0, stream, Q, K, V,
                     dO, lse, delta, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), (int)S, (int)nb,
                     (int)BH, scale, xcd_group);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int fa_fwd_select_variant(int64_t B, int64_t H, int64_t S, int64_t D, fa_dtype dtype) {
  if (B < 1 || H < 1 || S < 1) return -1;
  return select_variant(B, H, S, D, dtype);
}

int64_t fa_fwd_tiles_per_head(int64_t S, int causal, int variant) {
  int64_t bq, bk;
  if (variant == FA_VARIANT_MFMA_B256 || variant == FA_VARIANT_MFMA_B128 ||
      variant == FA_VARIANT_MFMA_B256_K128 || variant == FA_VARIANT_SPLIT || variant == FA_VARIANT_MFMA_B128_K128) {
    bq = mfma_block_q(variant);
    bk = mfma_block_k(variant);
  } else if (variant == FA_VARIANT_VALU) {
    bq = fa::kValuBQ;
    bk = fa::kValuBK;
  } else {
    return 0;
  }
  if (S < 1) return 0;
  int64_t tiles = 0;
  for (int64_t q0 = 0; q0 < S; q0 += bq) {
    const int64_t kv_end = causal ? (q0 + bq < S ? q0 + bq : S) : S;
    tiles += ceil_div(kv_end, bk);
  }
  return tiles;
}

}  // extern "C"

namespace {

// Host-side checks of a forward call (nothing is enqueued); on success the
// variant to run (AUTO resolved) is stored in *variant.
fa_status validate_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int64_t B,
                       int64_t H, int64_t S, int64_t D, float scale, fa_dtype dtype, int* variant) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || S < 1 || D < 1) return FA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARGUMENT;
  if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARGUMENT;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  // in-kernel offsets within one head are 32-bit; the grid is one dimension
  if (S * D >= (int64_t(1) << 31) || B > INT32_MAX / H) return FA_ERR_UNSUPPORTED;
  int var = *variant == FA_VARIANT_AUTO ? select_variant(B, H, S, D, dtype) : *variant;
  if (!variant_covers(var, D, dtype, S)) return FA_ERR_UNSUPPORTED;
  const int64_t bq = var == FA_VARIANT_VALU ? fa::kValuBQ : mfma_block_q(var);
  if (B * H * ceil_div(S, bq) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  *variant = var;
  return FA_OK;
}

// The forward with a given variant; sched is the balanced schedule's workspace or NULL.
fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t S, int64_t D, int causal, float scale, fa_dtype dtype, int variant, unsigned* sched,
                   void* stream) {
  const fa_status valid = validate_fwd(q, k, v, o, lse, B, H, S, D, scale, dtype, &variant);
  if (valid != FA_OK) return valid;
  const int64_t BH = B * H;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (variant == FA_VARIANT_VALU) {
    err = dtype == FA_DTYPE_FP32 ? launch_valu_d<float>(q, k, v, o, lse, BH, S, D, causal, scale, st)
                                 : launch_valu_d<uint16_t>(q, k, v, o, lse, BH, S, D, causal, scale, st);
  } else if (variant == FA_VARIANT_MFMA_B256_K128) {
    err = D == 128 ? launch_pingpong<128, 128>(q, k, v, o, lse, BH, S, causal, scale, sched, st)
                   : launch_pingpong<64, 128>(q, k, v, o, lse, BH, S, causal, scale, sched, st);
  } else if (variant == FA_VARIANT_SPLIT) {
    err = D == 128 ? launch_split<128>(q, k, v, o, lse, BH, S, causal, scale, st)
                   : launch_split<64>(q, k, v, o, lse, BH, S, causal, scale, st);
  } else if (variant == FA_VARIANT_MFMA_B256) {
    err = D == 128 ? launch_pingpong<128, 64>(q, k, v, o, lse, BH, S, causal, scale, sched, st)
                   : launch_pingpong<64, 64>(q, k, v, o, lse, BH, S, causal, scale, sched, st);
  } else if (variant == FA_VARIANT_MFMA_B128_K128) {
    err = D == 128 ? launch_mfma<128, 1, 128>(q, k, v, o, lse, BH, S, causal, scale, st)
                   : launch_mfma<64, 1, 128>(q, k, v, o, lse, BH, S, causal, scale, st);
  } else {
    err = D == 128 ? launch_mfma<128, 1>(q, k, v, o, lse, BH, S, causal, scale, st)
                   : launch_mfma<64, 1>(q, k, v, o, lse, BH, S, causal, scale, st);
  }
  if (err != hipSuccess) {
    g_last_hip_error = static_cast<int>(err);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

// The allocation-free entry point's scheduling scratch: one 8 KB array per
// device, at file scope, held until the process ends.  Host code never uses
// its name as an address: the device address comes from hipGetSymbolAddress,
// once per device, with that device current.
__device__ __align__(256) unsigned scratch[fa::pp::kSchedBytes / 4];

namespace {

__global__ void zero_words(unsigned* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
unsigned* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address; at the first call on a device it is
// looked up and cleared by a fill kernel on `stream` (stream-ordered, and a
// kernel rather than a memset, so a caller may capture it in a graph).
hipError_t device_scratch(hipStream_t stream, unsigned** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zero_words, dim3(1), dim3(256), 0, stream, static_cast<unsigned*>(p),
                       fa::pp::kSchedBytes / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<unsigned*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

fa_status fa_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                         int64_t S, int64_t D, int causal, float scale, fa_dtype dtype, int variant,
                         void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, variant, nullptr, stream);
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                 int64_t S, int64_t D, int causal, float scale, fa_dtype dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, FA_VARIANT_AUTO, nullptr, stream);
}

int64_t fa_fwd_workspace_bytes(void) { return fa::pp::kSchedBytes; }

fa_status fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                    int64_t S, int64_t D, int causal, float scale, fa_dtype dtype, void* workspace,
                    int64_t workspace_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 8) || workspace_bytes < fa::pp::kSchedBytes) return FA_ERR_INVALID_ARGUMENT;
  return fwd_impl(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, FA_VARIANT_AUTO,
                  static_cast<unsigned*>(workspace), stream);
}

fa_status fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                         int64_t S, int64_t D, int causal, float scale, fa_dtype dtype, void* stream) {
  int variant = FA_VARIANT_AUTO;
  const fa_status valid = validate_fwd(q, k, v, o, lse, B, H, S, D, scale, dtype, &variant);
  if (valid != FA_OK) return valid;  // a rejected call enqueues nothing, not even the scratch's first clear
  unsigned* ws = nullptr;
  const hipError_t e = device_scratch(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return fwd_impl(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, FA_VARIANT_AUTO, ws, stream);
}

int64_t fa_dense_workspace_bytes(int64_t S) { return S < 1 ? 0 : fa::dense::head_bytes(S); }

fa_status fa_dense_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                       int64_t S, int64_t D, int causal, float scale, fa_dtype dtype, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  namespace dn = fa::dense;
  if (!q || !k || !v || !o || !workspace) return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || S < 1 || D < 1) return FA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(workspace, 16))
    return FA_ERR_INVALID_ARGUMENT;
  if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARGUMENT;
  if (dtype != FA_DTYPE_BF16 || (D != 64 && D != 128)) return FA_ERR_UNSUPPORTED;
  if (S * D >= (int64_t(1) << 31) || B > INT32_MAX / H) return FA_ERR_UNSUPPORTED;
  const int64_t per_head = dn::head_bytes(S);
  if (workspace_bytes < per_head) return FA_ERR_INVALID_ARGUMENT;
  const int64_t BH = B * H;
  const int64_t n_qt = ceil_div(S, dn::kTile);
  const int64_t n_pairs = causal ? n_qt * (n_qt + 1) / 2 : n_qt * n_qt;
  // heads per chunk: what the workspace holds, within a one-dimensional grid
  int64_t nb = workspace_bytes / per_head;
  nb = nb < BH ? nb : BH;
  const int64_t grid_cap = INT32_MAX / (n_pairs > 4 ? n_pairs : 4);
  nb = nb < grid_cap ? nb : grid_cap;
  if (nb < 1) return FA_ERR_UNSUPPORTED;
  const int64_t pitch = dn::pitch_of(S);
  float* smat = static_cast<float*>(workspace);
  uint16_t* pmat = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + nb * S * pitch * 4);

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t head_elems = S * D;
  for (int64_t h0 = 0; h0 < BH; h0 += nb) {
    const int64_t n = BH - h0 < nb ? BH - h0 : nb;
    const auto* qh = static_cast<const uint16_t*>(q) + h0 * head_elems;
    const auto* kh = static_cast<const uint16_t*>(k) + h0 * head_elems;
    const auto* vh = static_cast<const uint16_t*>(v) + h0 * head_elems;
    auto* oh = static_cast<uint16_t*>(o) + h0 * head_elems;
    float* lh = lse ? lse + h0 * S : nullptr;
    hipError_t err;
    if (D == 128)
      err = causal ? launch_dense<128, true>(qh, kh, vh, oh, lh, n, S, scale, smat, pmat, st)
                   : launch_dense<128, false>(qh, kh, vh, oh, lh, n, S, scale, smat, pmat, st);
    else
      err = causal ? launch_dense<64, true>(qh, kh, vh, oh, lh, n, S, scale, smat, pmat, st)
                   : launch_dense<64, false>(qh, kh, vh, oh, lh, n, S, scale, smat, pmat, st);
    if (err != hipSuccess) {
      g_last_hip_error = static_cast<int>(err);
      return FA_ERR_HIP;
    }
  }
  return FA_OK;
}

int64_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S) {
  return (B < 1 || H < 1 || S < 1) ? 0 : B * H * S * (int64_t)sizeof(float);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t S, int64_t D, int causal, float scale,
                 fa_dtype dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || S < 1 || D < 1) return FA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(workspace, 4))
    return FA_ERR_INVALID_ARGUMENT;
  if (dtype != FA_DTYPE_BF16 || (D != 64 && D != 128)) return FA_ERR_UNSUPPORTED;
  if (S * D >= (int64_t(1) << 31) || B > INT32_MAX / H) return FA_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  if (BH * ceil_div(S, fa::bwd::kRows) > INT32_MAX || BH * S >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa_bwd_workspace_bytes(B, H, S)) return FA_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* delta = static_cast<float*>(workspace);
  hipError_t err;
  if (D == 128)
    err = causal ? launch_bwd<128, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, S, scale, delta, st)
                 : launch_bwd<128, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, S, scale, delta, st);
  else
    err = causal ? launch_bwd<64, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, S, scale, delta, st)
                 : launch_bwd<64, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, S, scale, delta, st);
  if (err != hipSuccess) {
    g_last_hip_error = static_cast<int>(err);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

const char* fa_status_str(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype, head dim, variant or size";
    case FA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

const char* fa_version(void) { return "fa_mi355x 0.1.0 gfx950"; }

}  // extern "C"
