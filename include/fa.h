/*
 * fa.h -- C ABI of the MI355X (gfx950) causal attention forward library
 * (libfa_mi355x.so).
 *
 * The operation is the forward pass described on the aiml.sh page "Speed up
 * long contexts with FlashAttention" (lab.py, tiled_flash_attention; its
 * dense reference is standard_attention): for every batch b, head h and query
 * row i,
 *
 *     s_ij  = scale * (q_i . k_j)            for visible keys j
 *     o_i   = sum_j softmax_j(s_ij) * v_j
 *     lse_i = log(sum_j exp(s_ij))           (natural log, scale included)
 *
 * where key j is visible to row i when j <= i (causal) or always (non-causal).
 * The result is computed tile by tile with an online softmax (running maximum,
 * running sum, rescaled accumulator), so no S x S matrix ever reaches memory.
 * The log-sum-exp output is not on the pages; it is what a caller needs to
 * merge partial results over key shards or to run a backward pass.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major [B, H, S, D] (D fastest) for q, k, v, o and
 *    [B, H, S] for lse.  Element type of q, k, v, o is `dtype`; lse is fp32.
 *  - All pointers are DEVICE pointers owned by the caller.  The library
 *    allocates, frees and synchronises nothing; it enqueues work on `stream`
 *    (a hipStream_t; NULL = the null stream) and returns after the enqueue.
 *  - q, k, v, o must be 16-byte aligned, lse 4-byte aligned.  o must not
 *    overlap q, k or v (not checked).  lse may be NULL (then not written).
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call enqueues nothing and returns a status, it never aborts.
 *  - Non-finite inputs give undefined (but memory-safe) results.
 *  - Calls on one stream are ordered; calls on different streams that write
 *    the same o / lse race (the caller's responsibility).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
  FA_DTYPE_FP32 = 0, /* IEEE binary32 */
  FA_DTYPE_BF16 = 1  /* bfloat16 (1-8-7) */
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* NULL / misaligned pointer, B, H, S or D < 1, non-finite scale */
  FA_ERR_UNSUPPORTED = 2,      /* dtype, head dim, variant or size outside what is compiled */
  FA_ERR_HIP = 3               /* the HIP runtime rejected the launch; see fa_last_hip_error() */
} fa_status;

/* Kernel variants.  FA_VARIANT_AUTO picks one from the shape; the others
 * exist so tests can show that results do not depend on the tiling.
 *   MFMA_B256: bf16, D in {64, 128}, S >= 64; 256-row query blocks, 8 waves of
 *              32 rows in two groups that alternate matrix-core and softmax
 *              phases; 64-key tiles, always copied whole (a last tile cut short
 *              by S is copied as the sequence's last 64 rows, hence S >= 64).
 *   MFMA_B128: bf16, D in {64, 128}; 128-row query blocks, 4 waves of 32 rows,
 *              two workgroups per CU (used when 256-row blocks leave CUs idle).
 *   VALU:      fp32 or bf16, D in {16, 32, 64, 128}; one lane per query,
 *              fp32 vector arithmetic (the fp32 path, and small head dims).
 *   MFMA_B256_K128: as MFMA_B256 with 128-key tiles, S >= 128: twice the work
 *              per phase, half the barriers, 2-slot rings.
 *   SPLIT:     bf16, D in {64, 128}; short sequences: a workgroup of 8 waves
 *              runs a pair of 64-row query blocks (qb and n-1-qb, equal work
 *              under the causal rule), as two 32-row halves times four key
 *              streams whose partial results are merged on chip.  AUTO picks
 *              MFMA_B256_K128 from 256 blocks of 256 rows on (more than 256
 *              at D = 64; and S >= 128), except MFMA_B128 for S < 384 with
 *              B * H <= 384;
 *              below that SPLIT while the pairs of 64-row blocks number at
 *              most 256; beyond them SPLIT at D = 64 or from S = 2048 on,
 *              MFMA_B256_K128 for D = 128 and 128 <= S < 2048, and MFMA_B128
 *              for S < 128.
 *   MFMA_B128_K128: as MFMA_B128 with 128-key tiles; their 128 KB of LDS
 *              leave one workgroup per CU (a point of the tiling sweep, never
 *              chosen by AUTO). */
typedef enum fa_variant {
  FA_VARIANT_AUTO = 0,
  FA_VARIANT_MFMA_B256 = 1,
  FA_VARIANT_MFMA_B128 = 2,
  FA_VARIANT_VALU = 3,
  FA_VARIANT_MFMA_B256_K128 = 4,
  FA_VARIANT_SPLIT = 5,
  FA_VARIANT_MFMA_B128_K128 = 6
} fa_variant;

/*
 * fa_fwd -- tiled online-softmax attention forward.
 *
 *   q, k, v   in : [B, H, S, D] dtype, device memory
 *   o         out: [B, H, S, D] dtype, device memory
 *   lse       out: [B, H, S] fp32, device memory, or NULL
 *   B, H, S   batch, heads, sequence length (>= 1); any S (tails are masked)
 *   D         head dim: 16, 32, 64 or 128 (bf16 64/128 run on the matrix cores)
 *   causal    nonzero: key j visible to row i iff j <= i (the diagonal included)
 *   scale     multiplies q.k; used as given (callers normally pass 1/sqrt(D))
 *   dtype     FA_DTYPE_BF16 or FA_DTYPE_FP32; softmax state and accumulation
 *             are fp32 either way; on the matrix-core variants the
 *             probabilities are rounded to bf16 before the P.V product
 *   stream    hipStream_t or NULL
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED (also when
 * S*D >= 2^31 or the grid would exceed 2^31-1 blocks) or FA_ERR_HIP.
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                 int64_t H, int64_t S, int64_t D, int causal, float scale, fa_dtype dtype,
                 void *stream);

/* fa_fwd with an explicit kernel variant (fa_variant); FA_ERR_UNSUPPORTED if
 * that variant does not cover dtype/D/S (see fa_variant).  Same arguments and
 * semantics. */
fa_status fa_fwd_variant(const void *q, const void *k, const void *v, void *o, float *lse,
                         int64_t B, int64_t H, int64_t S, int64_t D, int causal, float scale,
                         fa_dtype dtype, int variant, void *stream);

/*
 * fa_fwd_ws -- fa_fwd with a scheduling workspace: the same operation, the
 * same arguments and results, bit for bit.  What the workspace buys: when the
 * 256-row matrix-core kernel runs resident (more work items than compute
 * units, B*H a multiple of 8), the last rounds of each XCD's work items
 * (about an eighth of the work) are not assigned in advance but claimed at
 * run time through counters in the workspace, and workgroups of an XCD that
 * runs ahead take items of the others.  Under load each XCD holds its own
 * clock, so a static split ends with the slowest XCD.  In every other case
 * the call runs exactly as fa_fwd and the workspace is not touched.
 *
 *   workspace  device memory owned by the caller, 8-byte aligned, at least
 *              fa_fwd_workspace_bytes() bytes, ZERO-FILLED before its first
 *              use (e.g. one hipMemset).  Every call leaves it zero-filled
 *              again: its last workgroup resets the counters.  A workspace
 *              that is not zero when a call starts gives wrong results (work
 *              items skipped).  Calls that share a workspace must be ordered
 *              on one stream.
 *
 * Returns what fa_fwd returns, and FA_ERR_INVALID_ARGUMENT for a NULL,
 * misaligned or too small workspace.
 */
fa_status fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
                    int64_t S, int64_t D, int causal, float scale, fa_dtype dtype, void *workspace,
                    int64_t workspace_bytes, void *stream);

/* Workspace bytes fa_fwd_ws needs (a constant, 8192).  Host-only. */
int64_t fa_fwd_workspace_bytes(void);

/*
 * fa_fwd_noalloc -- fa_fwd_ws for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments as fa_fwd; the same
 * results as fa_fwd_ws (and fa_fwd), bit for bit.
 *
 * The scheduling workspace is the library's own: one file-scope array of
 * 8192 bytes per device (the fa_fwd_ws workspace, up to 880 workgroups of
 * balanced schedule; a device with more compute units runs the static
 * schedule instead), held until the process ends.  It serves every problem
 * size, so no size is rejected for it.  The call allocates nothing and calls
 * no allocating routine.  At the first call on a device, with that device
 * current, it looks up the array's address and clears it with a fill kernel
 * on `stream` (stream-ordered, and capturable, unlike a memset); every call
 * leaves the counters zero again.
 *
 * All calls on one device share that array: calls that may overlap on one
 * device (different streams, or graphs replayed concurrently) race and give
 * wrong results.  Order them on one stream.
 *
 * Returns what fa_fwd returns; FA_ERR_HIP also if the array's address cannot
 * be obtained (fa_last_hip_error() has the code).  A call rejected for its
 * arguments enqueues nothing.
 */
fa_status fa_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                         int64_t H, int64_t S, int64_t D, int causal, float scale, fa_dtype dtype,
                         void *stream);

/* The variant fa_fwd would run for this shape (an fa_variant value), or -1
 * if the arguments are unsupported.  Host-only; touches no device. */
int fa_fwd_select_variant(int64_t B, int64_t H, int64_t S, int64_t D, fa_dtype dtype);

/* Number of key/value tiles the causal tile scheduler of `variant` visits for
 * one (batch, head) of length S (0 for an unsupported variant).  Host-only. */
int64_t fa_fwd_tiles_per_head(int64_t S, int causal, int variant);

/*
 * fa_dense_fwd -- the dense, materialising forward pass on the GPU: the
 * standard attention of the aiml.sh page "Speed up long contexts with
 * FlashAttention" (lab.py, standard_attention), whose N x N score and
 * probability matrices the page's traffic model (run-output.txt,
 * hbm_traffic_sweep) charges to HBM.  It computes the same O and lse as
 * fa_fwd, in three kernels: S = scale * Q K^T (fp32, to the workspace),
 * P = softmax(S) per row (normalised, bf16, to the workspace; lse from the
 * row's maximum and sum), O = P V.  Under the causal rule only the 128 x 128
 * tiles at or below the diagonal are computed, written and read.  It is the
 * baseline against which the tiled path's traffic and time are measured.
 *
 *   q, k, v, o, lse, B, H, S, causal, scale, stream: as for fa_fwd
 *   D          64 or 128
 *   dtype      FA_DTYPE_BF16 only
 *   workspace  device memory owned by the caller, 16-byte aligned, at least
 *              fa_dense_workspace_bytes(S) bytes (one head).  The (batch,
 *              head) pairs are processed in chunks of as many heads as fit:
 *              workspace_bytes / fa_dense_workspace_bytes(S).  Its contents
 *              on return are unspecified; calls that share a workspace must
 *              be ordered on one stream.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT (also for a NULL, misaligned or
 * too small workspace), FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_dense_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                       int64_t B, int64_t H, int64_t S, int64_t D, int causal, float scale,
                       fa_dtype dtype, void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes fa_dense_fwd needs per (batch, head): S rows of the fp32
 * score matrix and S rows of the bf16 probability matrix, each row padded to
 * a multiple of 8 elements; 0 for S < 1.  Host-only. */
int64_t fa_dense_workspace_bytes(int64_t S);

/*
 * fa_bwd -- gradients of the fa_fwd forward: dQ, dK, dV for an upstream
 * gradient dO of O.  The pages stop at the forward of the aiml.sh page "Speed
 * up long contexts with FlashAttention" (lab.py, tiled_flash_attention); this
 * is that forward differentiated, computed the same tiled way.  Per (batch,
 * head), with P = softmax(scale * Q K^T) under the causal rule:
 *
 *     delta_i = dO_i . O_i,  dP = dO V^T,  dS = P * (dP - delta)
 *     dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO
 *
 * P is recomputed tile by tile from Q, K and lse, so no S x S matrix reaches
 * memory.  Two kernels run on `stream`: one per block of 128 query rows (dQ,
 * and delta into the workspace), then one per block of 128 keys (dK, dV).
 *
 *   q, k, v    in : [B, H, S, D] bf16, the forward's inputs
 *   o, lse     in : the forward's outputs for the same causal and scale (o
 *                   [B, H, S, D] bf16, lse [B, H, S] fp32, natural log)
 *   dout       in : [B, H, S, D] bf16, the gradient of o
 *   dq, dk, dv out: [B, H, S, D] bf16; must not overlap any input (not checked)
 *   B, H, S, causal, scale, stream: as for fa_fwd
 *   D          64 or 128
 *   dtype      FA_DTYPE_BF16 only.  P and dS are rounded to bf16 as MFMA
 *              operands; sums are fp32
 *   workspace  device memory owned by the caller, 4-byte aligned, at least
 *              fa_bwd_workspace_bytes(B, H, S) bytes; its contents on return
 *              are the row dot products delta (fp32 [B, H, S]).  Calls that
 *              share a workspace must be ordered on one stream.
 *
 * All pointers are device pointers, 16-byte aligned (lse and workspace: 4).
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT (NULL or misaligned pointer, B, H, S
 * or D < 1, non-finite scale, workspace too small), FA_ERR_UNSUPPORTED (dtype,
 * D, or S * D >= 2^31) or FA_ERR_HIP.
 */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t S,
                 int64_t D, int causal, float scale, fa_dtype dtype, void *workspace,
                 int64_t workspace_bytes, void *stream);

/* Workspace bytes fa_bwd needs: B * H * S fp32 values; 0 if B, H or S < 1.
 * Host-only. */
int64_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S);

/* Static, never-NULL description of a status code. */
const char *fa_status_str(fa_status status);

/* hipError_t of the last FA_ERR_HIP returned on the calling thread (0 if none). */
int fa_last_hip_error(void);

/* Library version string, e.g. "fa_mi355x 0.1.0 gfx950". */
const char *fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
