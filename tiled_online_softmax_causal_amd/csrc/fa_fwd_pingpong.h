// Tiled online-softmax attention forward, 8-wave "ping-pong" kernel for gfx950.
//
// The method is the one of the aiml.sh page "Speed up long contexts with
// FlashAttention" (lab.py, tiled_flash_attention): a block of query rows stays
// on chip while key/value blocks stream through, and every row keeps a running
// maximum, a running sum and an accumulator rescaled when the maximum moves.
// Key blocks wholly above the diagonal are never visited; blocks that straddle
// it are masked per element.  This kernel is that loop laid out for CDNA4.
//
// Work split.  A work item is 256 query rows of one (batch, head); a
// workgroup runs 8 waves of 32 rows each, two waves per SIMD.  With more items
// than CUs the grid is one workgroup per CU, each walking a list of items, and
// the key tiles of its items, item after item, form one tile sequence
// T = 0 .. N-1 that the phases run through without a break.  Waves 0-3
// (group 0) and 4-7 (group 1) alternate between two kinds of phase, one phase
// apart:
//
//     phase 2T     group 0: matrix phase T      group 1: softmax of tile T-1
//     phase 2T+1   group 0: softmax of tile T   group 1: matrix phase T
//
// where the matrix phase T issues O^T += V_{T-1}^T P_{T-1}^T and then
// S_T^T = K_T Q^T on the matrix cores (32 MFMAs per 64 keys for d = 128) and
// the softmax of tile T turns S_T into bf16 probabilities on the vector ALUs.
// Every SIMD thus holds one wave feeding its matrix core and one wave doing the
// exponentials, the two kinds of work overlap, and one workgroup barrier closes
// each phase.  At an item boundary one matrix phase finishes an item (its last
// P.V product) and starts the next (its first scores); the softmax of an
// item's first tile writes out the previous item before its own work, and the
// softmax of an item's last tile loads the next item's Q.  A key tile is
// BK = 64 or 128 keys; the longer tile halves the barriers and per-phase
// bookkeeping per unit of work.
//
// Data movement.  Group 0 carries the K tiles and group 1 the V tiles, copied
// HBM -> LDS directly (global_load_lds, no register staging) into a 3-slot K
// ring and a 2-slot V ring (160 KB of LDS for d = 128 and 128-key tiles).  A
// group issues its copies during its softmax phase, one between each pair of
// exponential steps, so the copies trickle into the CU's memory pipeline
// instead of arriving as one burst that would stall the issuing waves: K_{T+2}
// in phase 2T+1 and V_T in phase 2T, two phases before their first reader.
// The rings number tiles along the sequence, so the last copies of an item
// bring in the next item's first tiles.
// LDS rows are XOR-swizzled in 16-byte chunks so the 128-bit K reads and the
// 64-bit transposed V reads are free of bank conflicts on the 64-bank LDS.
//
// Register layout (v_mfma_f32_32x32x16_bf16).  Scores are formed transposed,
// S^T = K . Q^T, so each lane owns ONE query (column lane%32) and half of the
// tile's keys (rows 8*(r/4) + 4*(lane/32) + r%4 of each 32-key block); row max
// and row sum are lane-local plus one v_permlane32_swap.  The fp32 scores,
// exponentiated and packed to bf16, are already the B operand of
// O^T = V^T . P^T; V^T comes from LDS through ds_read_b64_tr_b16 in the
// matching key order.  The MFMA operands read from LDS run five MFMAs ahead
// of their use (a pinned issue order), so LDS latency hides behind the matrix
// core.
//
// Softmax.  Base 2: c = scale*log2(e) (of either sign) is folded into one FMA
// per score and exp is v_exp_f32.  The maximum only guards exp2 against
// overflow, so it is maintained lazily: an item starts it at the score of a
// key every row sees (key 0), every tile exponentiates against the running
// value at once, and only if some row's tile sum passes 2^64 is the tile
// redone with the exact maximum (its scores recomputed from the K tile still
// in LDS) and the accumulator and sum rescaled.  Numerator and denominator
// share the running value, so the result is that of the exact update up to
// rounding; a probability underflows only where it would also underflow
// against the true maximum.  The bf16 probabilities are written over the
// fp32 scores they come from.  The denominator is an fp32 sum of the fp32
// probabilities; only the P.V operand is rounded to bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_common.h"
#include "fa_schedule.h"

namespace fa {
namespace pp {

using namespace fa::common;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupThreads = kThreads / 2;
constexpr int kQW = 32;                 // query rows per wave
constexpr int kBQ = kQW * kWaves;       // query rows per workgroup
constexpr int kAhead = 5;               // MFMAs between an operand's LDS read and its use
constexpr float kOverflowSum = 0x1p64f; // a tile sum above this redoes the tile with the exact maximum
// Balanced schedule's workspace (32-bit words): 8 pool counters 128 bytes apart
// (64-bit front/back pairs at words 0, 32, ..., 224), a count of finished
// workgroups (word 256), then one 8-byte broadcast slot per workgroup from
// word 288.  It is zero between calls.
constexpr int kSchedBytes = 8192;
constexpr int kSchedDone = 256;
constexpr int kSchedSlots = 288;
constexpr int kSchedMaxGrid = (kSchedBytes / 4 - kSchedSlots) / 2;

// LDS tiles are row-major, D*2 bytes per row, with the 16-byte chunks of each
// row XOR-swizzled by swz(row) (masked to the row's chunk count).  For d = 128
// the 16 rows of one 16-lane group of a 128-bit K read get 16 different keys,
// and the 4 rows x 4 chunks of one 32-lane transposed V read land in 16
// different chunk columns, so neither read has bank conflicts on the 64-bank
// LDS.  Rows stay contiguous, as the direct global->LDS loads need.
template <int D, int BK>
struct Geo {
  static_assert(D == 64 || D == 128, "matrix-core path covers D = 64 and 128");
  static_assert(BK == 64 || BK == 128, "key tiles of 64 or 128 keys");
  static constexpr int kStagesK = 3;                            // depth of the K ring
  static constexpr int kStagesV = 2;                            // depth of the V ring
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;               // 16-byte chunks per row
  static constexpr int kTileBytes = BK * kRowBytes;             // one K or V tile
  static constexpr int kLdsBytes = (kStagesK + kStagesV) * kTileBytes;
  static constexpr int kLoads = BK * kChunks / kGroupThreads;    // 16-byte loads per thread per tile
  static constexpr int kRowsPerLoad = kGroupThreads / kChunks;   // tile rows covered by one load step
  static_assert(BK * kChunks % kGroupThreads == 0, "a tile must split evenly over a 4-wave group");
  static_assert(kLdsBytes <= 160 * 1024, "rings must fit the 160 KB LDS");
};

// Issue order of a matrix phase: MFMA items 0..NPV-1 are the P.V products (two
// LDS reads each), items NPV.. the score products (one LDS read each).  The
// reads of item i + kAhead are issued right after MFMA i.
template <int NPV, int N>
constexpr int reads_of(int i) {
  return i < NPV ? 2 : (i < N ? 1 : 0);
}
template <int NPV, int N, int I>
__device__ __forceinline__ void schedule_item() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA I
  if constexpr (reads_of<NPV, N>(I + kAhead) > 0)
    __builtin_amdgcn_sched_group_barrier(0x100, reads_of<NPV, N>(I + kAhead), 0);
}
template <int NPV, int N>
constexpr int first_reads() {
  int r = 0;
  for (int i = 0; i < kAhead; ++i) r += reads_of<NPV, N>(i);
  return r;
}
template <int NPV, int N, int... I>
__device__ __forceinline__ void schedule_matrix_phase(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, first_reads<NPV, N>(), 0);
  (schedule_item<NPV, N, I>(), ...);
}

template <int D, int BK, bool CAUSAL, bool BALANCED>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_pingpong(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int S, float c_log2, fa::sched::Plan plan,
    unsigned* __restrict__ sched) {
  using G = Geo<D, BK>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  constexpr int DS = D / 16;   // k-steps of the score MFMA
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int KB = BK / 32;  // 32-key blocks of S^T
  constexpr int KS = BK / 16;  // k-steps of the P.V MFMA
  constexpr int NL = G::kLoads;
  static_assert(NL <= KS && KS % NL == 0, "copies are spread over the exponential steps");

  __shared__ __attribute__((aligned(16))) char lds[G::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  // the lane's index recomputed from the hardware, so that no thread index is
  // held in a register through the whole kernel
  auto lane_id = []() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); };
  const int grp = wave >> 2;   // 0: matrix phase first, carries K; 1: one phase behind, carries V
  const int col = lane & 31;   // the query this lane owns, within the wave
  const int half = lane >> 5;  // which key half of each 32-key block
  const int u = lane & 15, quad = lane >> 4;

  // ---- work items and the flattened tile sequence.  The workgroup walks its
  // items (bh, query block) in order (one item when the grid has one
  // workgroup per item); their key tiles, item after item, form one sequence
  // T = 0 .. N-1 that the ping-pong pipeline runs without a break: the matrix
  // phase that finishes an item (its last P.V product) also starts the next
  // (its first scores), and the softmax phase of an item's first tile first
  // writes out the previous item.  The K and V rings number tiles by T.
  struct Item {
    int bh, qb, n_tiles, k;
    bool valid;
  };
  struct Span {
    int n_w, t_mask, t_last;
  };
  const int n_qb = plan.n_qb;
  //
  // Balanced schedule (a resident grid of G = 8P workgroups, heads grouped per
  // XCD, at least 8 heads per XCD).  Each XCD runs at its own clock under load,
  // and a static schedule ends with the slowest XCD.  So the last eighth of
  // every XCD's heads (hp of its hx heads) form a pool instead of being
  // scheduled in advance.  A workgroup that has finished its static items
  // claims pool items one at a time.  It takes its own XCD's pool from the
  // front, head after head, heaviest query block first, so that the XCD's
  // workgroups share each head's K/V in their L2.  Once that pool is empty it
  // takes other XCDs' pools from the back, where their lightest items are,
  // which read the least K/V from outside its L2.  Front and back counts of a
  // pool share one 64-bit word, so one atomic add claims an item and never
  // one that the other end has taken.  Each claimed item runs as a pipeline
  // of its own.  Which workgroup computes an item does not change its
  // arithmetic, so the outputs equal the static schedule's bit for bit.
  // sched: 8 front/back counters 128 bytes apart, a done count, then one
  // (bh, qb) slot per workgroup.  The counters start at zero, and the last
  // workgroup to finish zeroes them again for the next call.
  auto make_item = [&](int b, int q, int k) -> Item {
    const int kv_end = CAUSAL ? min(S, q * kBQ + kBQ) : S;
    return Item{b, q, (kv_end + BK - 1) / BK, k, true};
  };
  // the k-th item of this workgroup's static list (fa_schedule.h); in the
  // balanced schedule the list covers the XCD's heads in front of its pool and
  // is one of the two XCD orders (a smaller function: fewer live registers)
  auto static_item = [&](int k) -> Item {
    int b = 0, q = 0;
    if (BALANCED ? !fa::sched::static_item_xcd(plan, blockIdx.x, k, b, q)
                 : !fa::sched::static_item(plan, blockIdx.x, k, b, q))
      return Item{0, 0, 1, k, false};
    return make_item(b, q, k);
  };
  // The next pool item for this workgroup (-1 when every pool is empty).  One
  // thread takes it from the counters and writes it to the workgroup's slot;
  // the barriers around it make every wave finish the previous segment first
  // and read the slot after the write has completed.
  auto claim = [&]() -> Item {
    unsigned* const slot = sched + kSchedSlots + 2 * blockIdx.x;
    phase_barrier();
    if (wave == 0 && lane_id() == 0) {
      const int x = blockIdx.x & 7;
      int b = -1, q = 0;
      const int len = fa::sched::pool_len(plan);
      for (int d = 0; d < 8 && b < 0; ++d) {
        const int y = (x + d) & 7;
        const unsigned long long old = __hip_atomic_fetch_add(reinterpret_cast<unsigned long long*>(&sched[32 * y]),
                                                              d == 0 ? 1ull : 1ull << 32, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT);
        const int front = (int)(unsigned)old, back = (int)(unsigned)(old >> 32);
        if (front + back < len) fa::sched::pool_item(plan, y, d == 0 ? front : len - 1 - back, b, q);
      }
      __hip_atomic_store(slot, (unsigned)b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(slot + 1, (unsigned)q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
    }
    phase_barrier();
    const int b = __builtin_amdgcn_readfirstlane((int)__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const int q = __builtin_amdgcn_readfirstlane((int)__hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return b < 0 ? Item{0, 0, 1, 0, false} : make_item(b, q, 0);
  };
  // One segment: the pipeline over an item list from its first item `first`:
  // the static list, or (SINGLE) one claimed item.  The static schedule runs
  // one segment; the balanced one runs the static part, then one segment per
  // claimed item.
  auto run_segment = [&](const Item first, auto single_c) {
    constexpr bool SINGLE = decltype(single_c)::value;
    auto item_at = [&](int k) -> Item {
      if constexpr (SINGLE) {
        // opaque at every use, so that nothing derived from the one item is
        // hoisted out of the tile loop into registers held through it
        int bh = first.bh, qb = first.qb, nt = first.n_tiles;
        asm volatile("" : "+s"(bh), "+s"(qb), "+s"(nt));
        return k == 0 ? Item{bh, qb, nt, 0, true} : Item{0, 0, 1, k, false};
      } else {
        return static_item(k);
      }
    };
    Item cur = first;
    // The lane's indices, made opaque per segment: the offsets derived from
    // them are then formed in each segment instead of being shared by all
    // segments and held in registers through the static one.
    int tid_s = wave * 64 + lane_id();
    asm volatile("" : "+v"(tid_s));
    const int lane = tid_s & 63, col = lane & 31, half = lane >> 5, u = lane & 15, quad = lane >> 4;

    // ---- Q^T operand of an item: lane holds q[q0w + col][16*ds + 8*half + 0..7].
    // Nothing but the score MFMAs reads it, so a load issued early in a phase
    // is waited for only where those MFMAs need it.
    bf16x8_t qreg[DS];
    auto load_q = [&](const Item& it) {
      const int qrow = min(it.qb * kBQ + wave * kQW + col, S - 1);
      const uint16_t* src = Q + (size_t)it.bh * S * D + (size_t)qrow * D + 8 * half;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) qreg[ds] = *reinterpret_cast<const bf16x8_t*>(src + 16 * ds);
    };
    load_q(cur);

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
    // Scores and probabilities share registers: the bf16 probabilities of
    // k-step ks (keys 16*ks.., 8 per lane) are written over the first four of
    // the eight fp32 scores they come from, sacc[ks/2][8*(ks%2) + 0..3], and are
    // read from there as the B operand of the P.V MFMA before the next score
    // MFMAs overwrite the accumulator.
    f32x16_t sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = (f32x16_t){};
    auto p_operand = [&](int ks) {
      const f32x16_t& a = sacc[ks >> 1];
      const int r0 = 8 * (ks & 1);
      const f32x4_t w = {a[r0], a[r0 + 1], a[r0 + 2], a[r0 + 3]};
      return __builtin_bit_cast(bf16x8_t, w);
    };
    auto set_p = [&](int ks, bf16x8_t p8) {
      const f32x4_t w = __builtin_bit_cast(f32x4_t, p8);
      const int r0 = 8 * (ks & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) sacc[ks >> 1][r0 + j] = w[j];
    };
    float m_run = -__builtin_inff(), l_run = 0.f;

    // ---- staging: HBM -> LDS directly (global_load_lds, 16 bytes per lane).
    // Thread gtid of the carrying group fills 16-byte slots gtid, gtid + 256, ...
    // (row-major) of its tensor's tile; the source is the logical chunk that the
    // swizzle puts in that slot.  Every copy moves BK whole rows: a last tile cut
    // short by the end of the sequence is copied as the sequence's last BK rows
    // (keys S-BK .. S-1, so no row past S is read), and the keys it repeats from
    // the tile before are masked (the launch takes S >= BK).  K tile T lives in
    // K slot T % 3, V tile T in V slot T % 2.
    const int gtid = tid_s & (kGroupThreads - 1);
    const int gwave = wave & 3;
    const int g_row = gtid / G::kChunks;
    const int g_lch = (gtid % G::kChunks) ^ swz<G::kChunks>(g_row);  // same for every load step
    char* const kbuf0 = lds;
    char* const vbuf0 = lds + G::kStagesK * G::kTileBytes;
    auto kslot = [](int T) { return (T + G::kStagesK) % G::kStagesK; };
    auto vslot = [](int T) { return (T + G::kStagesV) % G::kStagesV; };
    // One tile copy: its first source row (wave-uniform) and the ring slot.
    struct Copy {
      const uint16_t* tile;
      char* slot;
    };
    // The copy cursor walks this group's tensor along the tile sequence; past
    // its end it keeps re-reading the last tile into the next slots, which keeps
    // the wait counts uniform.  Within an item it only adds: the tile address,
    // the rows left before the end of the sequence and the ring slot offset
    // move by fixed steps (no per-tile multiply or modulo in the softmax wave).
    const uint16_t* const c_tensor = grp == 0 ? K : V;
    char* const c_ring = grp == 0 ? kbuf0 : vbuf0;
    const int c_ring_bytes = (grp == 0 ? G::kStagesK : G::kStagesV) * G::kTileBytes;
    const uint16_t* c_src = c_tensor + (size_t)cur.bh * S * D;
    int c_k = cur.k, c_left = cur.n_tiles, c_rows = S, c_slot = 0;
    auto next_copy = [&]() -> Copy {
      // (c_rows < BK only for a last tile; S >= BK keeps the shifted start in the head)
      const Copy c{c_rows >= BK ? c_src : c_src - (BK - c_rows) * D, c_ring + c_slot};
      c_slot = c_slot + G::kTileBytes == c_ring_bytes ? 0 : c_slot + G::kTileBytes;
      if (c_left > 1) {
        --c_left;
        c_src += BK * D;
        c_rows -= BK;
      } else {
        const Item nx = item_at(c_k + 1);
        if (nx.valid) {
          c_k = nx.k;
          c_left = nx.n_tiles;
          c_rows = S;
          c_src = c_tensor + (size_t)nx.bh * S * D;
        }
      }
      return c;
    };
    // Load steps 2j and 2j + 1 of a copy, issued as one pair: 16 bytes per lane
    // from a 32-bit per-lane byte offset off the tile base.  The group's 256
    // lanes cover 4096 bytes per step, in the source and in LDS alike, so the
    // two steps of a pair share one offset register and one M0 value.
    static_assert(G::kRowsPerLoad * G::kRowBytes == 4096 && kGroupThreads * 16 == 4096, "steps 4096 bytes apart");
    static_assert(NL % 2 == 0, "copy steps go in pairs");
    const unsigned g_off = (unsigned)(g_row * G::kRowBytes + g_lch * 16);
    auto copy_pair = [&](int j, const Copy& c, unsigned off0) {
      const int i = 2 * j + 1;
      copy16x2_to_lds(c.tile, off0 + (unsigned)(i * 4096), c.slot + (i * kGroupThreads + gwave * 64) * 16);
    };

    // per-lane read offsets within a tile.  K: row 32*kb + col, logical chunk
    // 2*ds + half.  V (transposed read): rows 16*ks + 4*half + u/4 (+8 for the
    // upper k-slots), logical chunk 4*db + 2*(quad%2) + (u%4)/2, byte 8*(u%2).
    int k_off[DS], v_off_lo[DB], v_off_hi[DB];
    {
      const int sk = swz<G::kChunks>(col);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) k_off[ds] = col * G::kRowBytes + (((2 * ds + half) ^ sk) << 4);
      const int vr = 4 * half + (u >> 2);
      const int s_lo = swz<G::kChunks>(vr), s_hi = swz<G::kChunks>(vr + 8);
      const int c_l = 2 * (quad & 1) + ((u & 3) >> 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        v_off_lo[db] = vr * G::kRowBytes + (((4 * db + c_l) ^ s_lo) << 4) + 8 * (u & 1);
        v_off_hi[db] = (vr + 8) * G::kRowBytes + (((4 * db + c_l) ^ s_hi) << 4) + 8 * (u & 1);
      }
    }

    // ---- matrix phase T: O^T += V_{T-1}^T P_{T-1}^T (DB accumulators, k-step
    // outer), then S_T^T = K_T Q^T (KB accumulators, alternating).
    auto matrix_phase = [&](int T) {
      constexpr int NPV = DB * KS, NSC = DS * KB, NM = NPV + NSC;
      // slot bases as opaque wave-uniform values: the compiler would otherwise
      // strength-reduce T % 3 into one induction register per read address
      const char* Vl = vbuf0 + __builtin_amdgcn_readfirstlane(vslot(T - 1) * G::kTileBytes);
      const char* Kl = kbuf0 + __builtin_amdgcn_readfirstlane(kslot(T) * G::kTileBytes);
      // the matrix-core wave issues first; the softmax wave on the same SIMD
      // fills the issue slots the MFMAs leave free
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if (i < NPV) {
          const int ks = i / DB, db = i % DB;
          const char* vp = Vl + 16 * ks * G::kRowBytes;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + v_off_lo[db]));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + v_off_hi[db]));
          const bf16x8_t av = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                                      __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, p_operand(ks), oacc[db], 0, 0, 0);
        } else {
          const int j = i - NPV, ds = j / KB, kb = j % KB;
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Kl + 32 * kb * G::kRowBytes + k_off[ds]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], ds == 0 ? (f32x16_t){} : sacc[kb], 0, 0, 0);
        }
      }
      schedule_matrix_phase<NPV, NM>(std::make_integer_sequence<int, NM>{});
      __builtin_amdgcn_s_setprio(0);
    };
    // Every matrix phase runs the same full body, which keeps the loop's
    // register allocation simple.  Where a product is not needed its result is
    // harmless: in phase 0 the probabilities are zero and the V ring slot read
    // was zero-filled, and for a tile a wave does not see (past its rows'
    // diagonal) its softmax phase zeroes the probabilities, so the P.V product
    // adds exactly 0; the scores of phase N (past the last tile) are never used.

    // ---- epilogue of an item: O = acc / l (bf16, round to nearest even),
    // lse = ln2 * (m + log2 l); then the state starts over for the next item.
    // In the accumulator layout lanes l and l^32 hold the two 8-byte halves of
    // each 16-byte piece of one row; one v_permlane32_swap per dword hands each
    // lane a whole piece of its own and its partner's, so every store writes 32
    // contiguous bytes of each of 32 rows (8 stores instead of 16 of 16 bytes).
    auto finish_item = [&](const Item& it) {
      const int qi = it.qb * kBQ + wave * kQW + col;
      const float l_tot = sum_halves(l_run);
      // v_rcp_f32 (about 1 ulp) rather than a correctly rounded division: the
      // products are rounded to bf16; rows past S (l = 0) are not stored
      const float inv = __builtin_amdgcn_rcpf(l_tot);
      uint16_t* const orow = O + (size_t)it.bh * S * D + (size_t)min(qi, S - 1) * D;
      // all pieces first, then the stores under one branch (rows past S store
      // nothing): the pieces' multiply / convert / swap chains then overlap
      u32x4_t piece[DB][2];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; rg += 2) {
          const f32x4_t v0 = {oacc[db][4 * rg + 0] * inv, oacc[db][4 * rg + 1] * inv,
                              oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv};
          const f32x4_t v1 = {oacc[db][4 * rg + 4] * inv, oacc[db][4 * rg + 5] * inv,
                              oacc[db][4 * rg + 6] * inv, oacc[db][4 * rg + 7] * inv};
          // a0: columns 32db + 8rg + 4half + 0..3, a1: the same for rg + 1
          const u32x2_t a0 = __builtin_bit_cast(u32x2_t, __builtin_convertvector(v0, bf16x4_t));
          const u32x2_t a1 = __builtin_bit_cast(u32x2_t, __builtin_convertvector(v1, bf16x4_t));
          // the lower half-wave keeps piece rg and needs its partner's a0; the
          // upper keeps piece rg + 1 and needs its partner's a1.  Swapping the
          // upper lanes of a0 with the lower lanes of a1 gives both at once:
          // afterwards a0 holds (own a0 | partner's a1) and a1 holds (partner's
          // a0 | own a1) in the (lower | upper) half-wave, so every lane's piece
          // is a0 then a1, with no per-lane selects.
          u32x2_t x0, x1;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const auto p = __builtin_amdgcn_permlane32_swap(a0[e], a1[e], false, false);
            x0[e] = p[0];
            x1[e] = p[1];
          }
          piece[db][rg / 2] = (u32x4_t){x0[0], x0[1], x1[0], x1[1]};
        }
      if (qi < S) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rg = 0; rg < 4; rg += 2)
            *reinterpret_cast<u32x4_t*>(orow + 32 * db + 8 * (rg + half)) = piece[db][rg / 2];
      }
      if (LSE && half == 0 && qi < S) LSE[(size_t)it.bh * S + qi] = (m_run + __builtin_log2f(l_tot)) * common::kLn2;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
      m_run = -__builtin_inff();
      l_run = 0.f;
    };

    // Per-item, per-wave tile bounds of the softmax phases: the wave's rows see
    // keys only in tiles t < n_w (keys below min(S, q0w + 32)); tiles
    // t >= t_mask straddle the diagonal or run past S and are masked per
    // element; t_last is the tile in whose phase the next item's Q is loaded
    // (-1: no next item).
    auto span_of = [&](const Item& it, const Item& nx) -> Span {
      const int q0w = it.qb * kBQ + wave * kQW;
      const int n_w = q0w >= S ? 0 : (CAUSAL ? min(it.n_tiles, (min(q0w + kQW, S) - 1) / BK + 1) : it.n_tiles);
      const int t_mask = CAUSAL ? min((q0w + 1) / BK, S / BK) : S / BK;
      return Span{n_w, t_mask, nx.valid ? it.n_tiles - 1 : -1};
    };

    // ---- softmax phase for tile t of item `it` (flattened index T): S -> bf16
    // P, running max / sum.  The NL load steps of copy cp are issued along the
    // way, one per KS / NL exponential steps (pinned there by a scheduling
    // barrier).  When `next_q` is set the next item's Q operand has already been
    // loaded over this item's (its latency hidden by this phase), and the rare
    // recompute below reloads this item's first.
    auto softmax_phase = [&](const Item& it, int t, int T, const Copy& cp, bool next_q, const Item& nx,
                             const Span& sp) {
      const int q0w = it.qb * kBQ + wave * kQW;
      // the copy offsets are formed here, not hoisted out of the loop, where
      // they would hold registers through the matrix phase
      unsigned off0 = g_off;
      asm volatile("" : "+v"(off0));
      // copy modes: 0 none, 1 the tile's copy steps (a pair after every second
      // step's exponentials)
      auto copy_at = [&](int ks, auto mode_c) {
        if (decltype(mode_c)::value != 0 && ks % (KS / NL) == 0 && (ks / (KS / NL)) % 2 == 1) {
          copy_pair(ks / (KS / NL) / 2, cp, off0);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      using WithCopies = std::integral_constant<int, 1>;
      if (t >= sp.n_w) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) set_p(ks, (bf16x8_t){});
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) copy_at(ks, WithCopies{});
        return;
      }
      const int kv0 = t * BK;
      // keys in the tile's LDS rows: kv0 .. kv0 + BK - 1, or S - BK .. S - 1 for a
      // last tile cut short by S (those below kv0 repeat the tile before)
      const int kv_row0 = min(kv0, S - BK);
      const int qi = q0w + col;
      // Tiles that straddle the diagonal or run past S move to the base-2 domain
      // here, so a hidden score is a plain -inf even when the scale is 0.
      bool masked = t >= sp.t_mask;
      const float c_t = masked ? 1.f : c_log2;
      // Element (kb, r) sits in LDS row j = 32 kb + 8 (r / 4) + 4 half + r % 4,
      // key kv_row0 + j.  It is visible from key kv0 (below it a last tile cut
      // short by S repeats the tile before) up to the row's diagonal qi
      // (causal).  With d = kv0 - kv_row0 and c = 32 kb + 8 (r / 4) + r % 4,
      // that is 0 <= c + 4 half - d <= qi - kv0: one unsigned compare, as a
      // negative left side wraps above any bound (qi >= kv0 in every tile a
      // wave takes part in).
      auto apply_mask = [&]() {
        const int b = 4 * half - (kv0 - kv_row0);
        const unsigned hi = CAUSAL ? (unsigned)(qi - kv0) : (unsigned)BK;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
            const bool hidden = (unsigned)(c + b) > hi;
            sacc[kb][r] = hidden ? -__builtin_inff() : sacc[kb][r] * c_log2;
          }
      };
      if (masked) apply_mask();
      // exponentiate against the running maximum (the copies interleaved in
      // copy mode 1); rs is the lane's share of the tile's row sum
      float rs = 0.f;
      auto exponentiate = [&](auto mode_c) {
        const float neg_m = m_run == -__builtin_inff() ? 0.f : -m_run;
        rs = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int kb = ks >> 1, r0 = 8 * (ks & 1);
          bf16x8_t p8;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const f32x2_t x = {__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r0 + e], c_t, neg_m)),
                               __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r0 + e + 1], c_t, neg_m))};
            rs = ks == 0 && e == 0 ? x[0] : rs + x[0];
            rs += x[1];
            const bf16x2_t b = __builtin_convertvector(x, bf16x2_t);
            p8[e] = b[0];
            p8[e + 1] = b[1];
          }
          set_p(ks, p8);
          copy_at(ks, mode_c);
        }
      };
      // The running maximum only guards exp2 against overflow.  An item starts
      // it at the scaled score of key 0, which every row sees (keys 0 and 4 in
      // the two half-waves), and every tile exponentiates against it at once;
      // only if some row's tile sum then passes 2^64 (a score about 64 above
      // the running value, base 2) is the tile redone: its scores, which the
      // probabilities have overwritten, are recomputed from K_T (still in its
      // LDS slot: K_{T+3} is copied two phases later), the maximum is taken
      // exactly, and O and l are rescaled.
      // (the maximum of the scaled scores: the scale may be negative)
      auto take_exact_max = [&]() {
        float mxk[KB];  // one three-input max chain per 32-key block
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          mxk[kb] = fmaxf(sacc[kb][0] * c_t, sacc[kb][1] * c_t);
#pragma unroll
          for (int r = 2; r < 16; r += 2) mxk[kb] = max3(mxk[kb], sacc[kb][r] * c_t, sacc[kb][r + 1] * c_t);
        }
        float mx = mxk[0];
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, mxk[kb]);
        const float m_new = fmaxf(m_run, max_halves(mx));
        const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      };
      // item start: O and l are zero, so no rescale
      if (t == 0) m_run = max_halves(sacc[0][0] * c_t);
      exponentiate(WithCopies{});
      if (__builtin_amdgcn_ballot_w64(!(rs <= kOverflowSum)) != 0) {
        // the two conditions again, from opaque copies of their bounds, rather
        // than kept as masks through the exponentials above (this path is rare)
        int t_last = sp.t_last, t_mask = sp.t_mask;
        asm volatile("" : "+s"(t_last), "+s"(t_mask));
        next_q = t == t_last;
        masked = t >= t_mask;
        if (next_q) load_q(it);
        const char* Kl = kbuf0 + __builtin_amdgcn_readfirstlane(kslot(T) * G::kTileBytes);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Kl + 32 * kb * G::kRowBytes + k_off[ds]);
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], ds == 0 ? (f32x16_t){} : sacc[kb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);  // one operand read at a time: this path is rare
          }
        if (next_q) load_q(nx);
        if (masked) apply_mask();
        take_exact_max();
        exponentiate(std::integral_constant<int, 0>{});
      }
      l_run += rs;
    };

    // ---- prologue: group 0 copies K_0 and K_1 and waits for K_0; group 1
    // zero-fills the V slot that the first matrix phase reads with zero
    // probabilities (V_0 is copied in phase 0)
    if (grp == 0) {
      const Copy k0 = next_copy(), k1 = next_copy();
#pragma unroll
      for (int j = 0; j < NL / 2; ++j) copy_pair(j, k0, g_off);
#pragma unroll
      for (int j = 0; j < NL / 2; ++j) copy_pair(j, k1, g_off);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm<NL>());  // K_0 has landed
    } else {
      char* v_prev = vbuf0 + vslot(-1) * G::kTileBytes;
      for (int off = gtid * 16; off < G::kTileBytes; off += kGroupThreads * 16)
        *reinterpret_cast<u32x4_t*>(v_prev + off) = (u32x4_t){0u, 0u, 0u, 0u};
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the zeros are in LDS
    }
    phase_barrier();

    // ---- 2 (N + 1) phases, one barrier each.  The two groups run the same
    // phases with their roles swapped.  Group 0 copies K_{T+2} during phase
    // 2T+1 into the slot last read in phase 2T-1 and, before the barrier
    // closing phase 2T+1, waits for K_{T+1} (its copy from phase 2T-1).  Group 1
    // copies V_T during phase 2T into the slot last read in phase 2T-1 and waits
    // for it before the barrier closing phase 2T+1.  So K_{T+1} and V_T are in
    // LDS before their first reader, phase 2T+2.  In the softmax phase of an
    // item's first tile the previous item is written out first; in that of its
    // last tile the next item's Q operand is loaded first.
    Item prev = cur;
    int T = 0;
    // the softmax phase of tile t of the current item (flattened index T)
    auto softmax_step = [&](int t, const Item& nx, const Span& sp) {
      const Copy cp = next_copy();
      if (t == 0 && T > 0) finish_item(prev);
      const bool next_q = t == sp.t_last;
      if (next_q) load_q(nx);
      softmax_phase(cur, t, T, cp, next_q, nx, sp);
    };
    if (grp == 0) {
      matrix_phase(0);  // phase 0
      phase_barrier();
      for (;;) {
        const Item nx = item_at(cur.k + 1);
        const Span sp = span_of(cur, nx);
        for (int t = 0; t < cur.n_tiles; ++t, ++T) {
          softmax_step(t, nx, sp);  // phase 2T + 1
          __builtin_amdgcn_s_waitcnt(waitcnt_vm<NL>());
          phase_barrier();
          matrix_phase(T + 1);  // phase 2T + 2
          phase_barrier();
        }
        prev = cur;
        if (!nx.valid) break;
        cur = nx;
      }
      finish_item(prev);  // phase 2N + 1
      phase_barrier();
    } else {
      {  // phase 0: no scores yet, only the copy of V_0
        const Copy cp = next_copy();
#pragma unroll
        for (int j = 0; j < NL / 2; ++j) copy_pair(j, cp, g_off);
      }
      phase_barrier();
      matrix_phase(0);  // phase 1
      __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
      phase_barrier();
      for (;;) {
        const Item nx = item_at(cur.k + 1);
        const Span sp = span_of(cur, nx);
        for (int t = 0; t < cur.n_tiles; ++t, ++T) {
          softmax_step(t, nx, sp);  // phase 2T + 2
          phase_barrier();
          matrix_phase(T + 1);  // phase 2T + 3
          __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
          phase_barrier();
        }
        prev = cur;
        if (!nx.valid) break;
        cur = nx;
      }
      finish_item(prev);
    }
    // no global->LDS copy may still be writing when the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(waitcnt_vm<0>());
  };
  const Item first = static_item(0);
  if (first.valid) run_segment(first, F_{});
  if constexpr (BALANCED) {
    for (;;) {
      const Item it = claim();
      if (!it.valid) break;
      run_segment(it, T_{});
    }
    // This workgroup has made its last claim, and once every wave has read it
    // the slot is cleared.  The last workgroup to get here (all claims are
    // over) zeroes the counters: the workspace is left as it was found.
    phase_barrier();
    if (wave == 0 && lane_id() == 0) {
      unsigned* const slot = sched + kSchedSlots + 2 * blockIdx.x;
      __hip_atomic_store(slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(slot + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned done = __hip_atomic_fetch_add(&sched[kSchedDone], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (done == gridDim.x - 1) {
        for (int y = 0; y < 8; ++y)
          __hip_atomic_store(reinterpret_cast<unsigned long long*>(&sched[32 * y]), 0ull, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&sched[kSchedDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace pp
}  // namespace fa
