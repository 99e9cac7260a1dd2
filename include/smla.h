/*
 * libsmla -- sparse top-k MLA attention (DeepSeek sparse attention) for AMD
 * MI355X (gfx950).  C ABI.
 *
 * What the library computes.  For each query token t, H query heads share one
 * latent KV row set (MQA): K = kv[:, :d_qk], V = kv[:, :d_v].  Token t attends
 * only to the KV rows named by its valid top-k slots, plus an optional
 * per-head sink logit that joins the softmax denominator and has no value row.
 * Sources (page title, section):
 *   [cuDNN-FE #785] "DSA backward SM90: fix three top-k and attention-sink
 *                    boundary failures" -- Summary 1-3, Why 1-3, Not addressed
 *   [cuDNN-FE #298] "DSA bwd SM100 fix dropped dKV gradients when topk width >
 *                    total_S_kv"
 *   [flash-attn #2882] "[CuTe, SM100] Support 1..128 Q heads in sparse MLA via
 *                    in-kernel TMA padding" -- Agent Notes, Mechanism
 *   [Automodel #3467] "Fix DeepSeek-V4 TileLang sparse-MLA backward
 *                    compilation on Blackwell" -- review (validity mask)
 *
 * Slot validity.  Slot j of token t is valid iff
 *   j < L_t   where L_t = clamp(topk_length[t], 0, W) if topk_length != NULL
 *             (compact layout) and L_t = W otherwise (non-compact layout, -1
 *             entries are padding) [cuDNN-FE #785 Why 2], and
 *   0 <= topk_idxs[t][j] < S_kv   [Automodel #3467 review].
 * The slot position is never compared with S_kv: in a non-compact row wider
 * than S_kv, valid indices may sit at any column [cuDNN-FE #298].
 *
 * Conventions shared by every call.
 *   - All tensors are dense, row-major, device memory, 16-byte aligned base
 *     pointers.  bf16 tensors are passed as void* holding IEEE bfloat16.
 *   - B > 1 batches are expressed by concatenating tokens and KV rows with
 *     global row indices.
 *   - Supported: d_qk in {512, 576}, d_v = 512, 1 <= H <= 128,
 *     1 <= W <= SMLA_MAX_W, S_kv >= 1 with S_kv * d_qk * 2 < 2^31 (KV rows
 *     are addressed with 32-bit byte offsets: S_kv <= 1864135 at d_qk = 576,
 *     2097151 at 512), T >= 0 (T = 0 is a no-op), scale finite.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     memory and never synchronises: work is enqueued on `stream` (a
 *     hipStream_t; NULL means the null stream) and the call returns.
 *   - Errors are reported by the return value before anything is enqueued;
 *     SMLA_ERR_LAUNCH reports a failed kernel launch.  No global state is kept
 *     (except the fixed scratch of smla_bwd_noalloc).
 *   - Outputs are fully overwritten (a NaN-prefilled output comes back fully
 *     written), including the rows of empty tokens.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

/* Entry points are the library's only exported symbols (it is built with
 * hidden visibility for everything else). */
#if defined(__GNUC__) || defined(__clang__)
#define SMLA_API __attribute__((visibility("default")))
#else
#define SMLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Largest supported top-k width W (slots per token). */
#define SMLA_MAX_W (1 << 24)

/* Workspace that smla_bwd_workspace_size asks for at most, unless one token's
 * chunk alone needs more (8 GiB). */
#define SMLA_BWD_DEFAULT_WORKSPACE ((size_t)8 << 30)

typedef enum {
    SMLA_OK = 0,
    SMLA_ERR_NULL = 1,        /* a required pointer is NULL                  */
    SMLA_ERR_SHAPE = 2,       /* a size is negative or inconsistent          */
    SMLA_ERR_UNSUPPORTED = 3, /* a size outside the supported range          */
    SMLA_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned       */
    SMLA_ERR_WORKSPACE = 5,   /* workspace NULL or too small for one token   */
    SMLA_ERR_LAUNCH = 6,      /* the HIP runtime refused a kernel launch     */
    SMLA_ERR_SCRATCH = 7      /* smla_bwd_noalloc: problem too large for its
                                 fixed scratch                               */
} smla_status;

/* Problem sizes.  T query tokens, S_kv KV rows, H heads, head widths d_qk and
 * d_v (d_v <= d_qk; V is the first d_v columns of each kv row), W top-k slots
 * per token, softmax scale (scores are scale * <q, k>). */
typedef struct {
    int32_t T, S_kv, H, d_qk, d_v, W;
    float scale;
} smla_dims;

/* Forward [flash-attn #2882 Agent Notes; cuDNN-FE #785 Summary 2-3].
 *   q          bf16 [T, H, d_qk]
 *   kv         bf16 [S_kv, d_qk]
 *   topk_idxs  int32 [T, W]
 *   topk_length int32 [T] or NULL (NULL = non-compact layout)
 *   attn_sink  fp32 [H] or NULL (NULL = no sink); +-inf and values beyond
 *              the fp32 log2(e) rescale limit are handled (saturating sink)
 *   o          bf16 [T, H, d_v]  out: softmax(valid scores + sink) @ V, the
 *              sink column dropped; 0 for a token with no valid slot
 *   lse        fp32 [T, H]       out: natural-log LSE of the valid scores,
 *              WITHOUT the sink; -inf for a token with no valid slot
 */
SMLA_API smla_status smla_fwd(const smla_dims* dims, const void* q, const void* kv,
                     const int32_t* topk_idxs, const int32_t* topk_length,
                     const float* attn_sink, void* o, float* lse, void* stream);

/* Bytes of device workspace with which smla_fwd_splitkv splits each token's
 * slot blocks over several workgroups: non-zero when the tokens alone (one
 * workgroup per token and group of 64 or 128 heads) give fewer than 128
 * workgroups, i.e. decode and short chunks against long top-k rows; 0 when
 * no split is made (then smla_fwd_splitkv is smla_fwd). */
SMLA_API size_t smla_fwd_splitkv_workspace_size(const smla_dims* dims);

/* The forward with split KV [cuDNN-FE #785 review thread: the SM90 tile
 * scheduler's grid of (blocks, heads x splits, batch)]: the 64-slot blocks
 * of a token are cut into up to ceil(W / 64) contiguous ranges, each run by
 * its own workgroup, which keeps the unnormalised O and its softmax sums in
 * workspace; a second kernel merges the ranges, folds the sink and writes O
 * and LSE exactly as smla_fwd defines them (the bits may differ from
 * smla_fwd's in the last places).  With a workspace smaller than
 * smla_fwd_splitkv_workspace_size the split count is reduced to fit (none
 * when it holds no split).  workspace: workspace_bytes of device memory,
 * 16-byte aligned, or NULL; used by this call only.  Arguments, outputs and
 * errors otherwise as smla_fwd. */
SMLA_API smla_status smla_fwd_splitkv(const smla_dims* dims, const void* q, const void* kv,
                             const int32_t* topk_idxs, const int32_t* topk_length,
                             const float* attn_sink, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Backward preprocess [cuDNN-FE #785 Not addressed: Delta = O . dO, fp32
 * reduction of the bf16-stored O].
 *   o, dO      bf16 [T, H, d_v]
 *   delta      fp32 [T, H]  out: sum_c o[t,h,c] * dO[t,h,c]
 */
SMLA_API smla_status smla_bwd_preprocess(const smla_dims* dims, const void* o, const void* dO,
                                float* delta, void* stream);

/* Exact Delta, the high-accuracy alternative to smla_bwd_preprocess
 * [cuDNN-FE #785 Not addressed: the table of delta sources, second row].
 * Recomputes, per token, the probabilities P_j (from lse and the sink as in
 * smla_bwd) and dP_j = dO . V_j over the valid slots and returns
 *   delta      fp32 [T, H] out: sum_j P_j dP_j, accumulated in fp32 (P_j in
 *              fp32, not rounded to bf16); 0 for a token with no valid slot
 * This equals O . dO for the exact O (the FlashAttention identity), without
 * the bf16 rounding of the stored O that limits smla_bwd_preprocess; fed to
 * smla_bwd it makes d_sink and the Delta term of dS exact to fp32 rounding.
 * It costs one more pass of the S and dP products over the gathered rows.
 * Inputs: q, kv, topk_idxs, topk_length, attn_sink as in smla_fwd; dO bf16
 * [T, H, d_v]; lse fp32 [T, H] from smla_fwd.  No workspace.
 */
SMLA_API smla_status smla_bwd_delta_exact(const smla_dims* dims, const void* q, const void* kv,
                                 const void* dO, const float* lse, const int32_t* topk_idxs,
                                 const int32_t* topk_length, const float* attn_sink,
                                 float* delta, void* stream);

/* Bytes of device workspace to give smla_bwd for these sizes (0 if T == 0):
 * the workspace of all T tokens at once when that is at most
 * SMLA_BWD_DEFAULT_WORKSPACE, else that of equal token chunks that fit in it
 * (never less than what one token needs).  Returns 0 for unsupported sizes
 * as well; smla_bwd reports the error.  smla_bwd accepts any larger or
 * smaller workspace down to one token's need and sizes its chunks to it. */
SMLA_API size_t smla_bwd_workspace_size(const smla_dims* dims);

/* Tokens per chunk that smla_bwd uses with a workspace of workspace_bytes
 * (the largest chunk whose workspace fits, evened out over the chunks when
 * that fits too); 0 if not even one token's chunk fits (smla_bwd then
 * returns SMLA_ERR_WORKSPACE) or the sizes are unsupported. */
SMLA_API int smla_bwd_chunk_tokens(const smla_dims* dims, size_t workspace_bytes);

/* Backward of L = sum(dO * O) [cuDNN-FE #785 Summary 1-3, Why 1-3;
 * cuDNN-FE #298].  Recomputes the probabilities from the forward's LSE and
 * the sink, dP = dO V^T, dS = P (dP - Delta), and returns
 *   dq         bf16 [T, H, d_qk] out: scale * dS K; 0 for a token with no
 *              valid slot (that token's q, dO, lse and delta are not read)
 *   dkv        fp32 [S_kv, d_qk] out: row r is the sum, over the valid slots
 *              that name r taken in token order, of scale * dS^T q (all d_qk
 *              columns) plus P^T dO (first d_v columns); each slot's
 *              contribution is accumulated in fp32 and kept until the row
 *              sum in blocks of 4 columns sharing an exponent, with error at
 *              most 2^-13 of the block's largest magnitude.
 *              The order is fixed, so dkv is the same bits run to run.  Rows
 *              never named by a valid slot (e.g. row 0 for -1 sentinels) are
 *              exactly 0.
 *   d_sink     fp32 [H] out: -sum_t p_sink[t,h] * delta[t,h] with
 *              p_sink = sigmoid(sink - lse); required iff attn_sink != NULL
 * Inputs: q, kv, topk_idxs, topk_length, attn_sink as in smla_fwd; dO bf16
 * [T, H, d_v]; lse fp32 [T, H] from smla_fwd; delta fp32 [T, H] from
 * smla_bwd_preprocess or smla_bwd_delta_exact.  workspace: workspace_bytes
 * of device memory (16-byte aligned), used by this call only.  The tokens
 * are processed in chunks of equal size, as many tokens per chunk as the
 * workspace holds (all T with smla_bwd_workspace_size bytes unless that is
 * capped); dkv sums a row's contributions chunk by chunk in token order, so
 * its bits depend on the chunk size but not on scheduling.  A chunk of fewer
 * than 128 tokens also splits each row's 64-slot blocks into ranges run by
 * separate workgroups (so that the GPU is filled); dq is then summed range by
 * range in fp32, and its bits follow the number of ranges.
 * SMLA_ERR_WORKSPACE if workspace is NULL or holds less than one token's
 * chunk.
 */
SMLA_API smla_status smla_bwd(const smla_dims* dims, const void* q, const void* kv, const void* dO,
                     const float* lse, const float* delta, const int32_t* topk_idxs,
                     const int32_t* topk_length, const float* attn_sink, void* dq,
                     float* dkv, float* d_sink, void* workspace, size_t workspace_bytes,
                     void* stream);

/* smla_bwd_preprocess followed by smla_bwd in one call [cuDNN-FE #785 Not
 * addressed: Delta = O . dO; Summary 1-3 for the backward]: the kernel that
 * recomputes P and dP also forms Delta = sum_c o . dO in fp32 from the rows
 * it loads anyway, so the separate pass over O and dO is saved.
 *   o          bf16 [T, H, d_v] in: the forward's output (from smla_fwd)
 *   delta      fp32 [T, H] out: sum_c o[t,h,c] * dO[t,h,c] (what
 *              smla_bwd_preprocess writes; the summation order differs, so
 *              the bits may differ in the last places)
 * Every other argument, output, the workspace and the errors are those of
 * smla_bwd; o must be non-NULL and 16-byte aligned when T > 0.
 */
SMLA_API smla_status smla_bwd_from_o(const smla_dims* dims, const void* q, const void* kv,
                            const void* dO, const void* o, const float* lse, float* delta,
                            const int32_t* topk_idxs, const int32_t* topk_length,
                            const float* attn_sink, void* dq, float* dkv, float* d_sink,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Number of stages smla_bwd runs, in order: index inversion, S/P/dP/dS with
 * dQ (one pass), the merge of dQ shares when a token's blocks are split over
 * several workgroups (empty otherwise), per-slot dKV contributions, dKV row
 * reduce, d_sink. */
#define SMLA_BWD_STAGES 6

/* smla_bwd with stage timing, for benchmarks and profilers.  Computes exactly
 * what smla_bwd computes (same passages, same kernels) and in addition records
 * stage_events[0] on `stream` before the first stage and stage_events[i] after
 * stage i (i = 1..SMLA_BWD_STAGES).  When the workspace splits the tokens into
 * several chunks, events 1..5 bracket the stages of the first chunk and the
 * last event follows the whole call.  stage_events: n_events >= 
 * SMLA_BWD_STAGES + 1 hipEvent_t handles created by the caller (recorded, not
 * created or destroyed, by the library).  Errors: SMLA_ERR_NULL for a NULL
 * array or handle, SMLA_ERR_SHAPE if n_events is too small, then as smla_bwd.
 */
SMLA_API smla_status smla_bwd_profiled(const smla_dims* dims, const void* q, const void* kv,
                              const void* dO, const float* lse, const float* delta,
                              const int32_t* topk_idxs, const int32_t* topk_length,
                              const float* attn_sink, void* dq, float* dkv, float* d_sink,
                              void* workspace, size_t workspace_bytes, void* stream,
                              void* const* stage_events, int n_events);

/* Bytes of the fixed per-GPU scratch of smla_bwd_noalloc (256 MiB). */
#define SMLA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* smla_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The library keeps
 * a fixed scratch of SMLA_NOALLOC_SCRATCH_BYTES in device memory on every GPU
 * it runs on (held until the process ends) and uses the current device's
 * copy as smla_bwd's workspace: the tokens are processed in chunks that fit
 * in it (for the T = 4096, H = 128, 640-slot headline about 150 tokens per
 * chunk).  No call allocates or frees anything.
 *
 * Arguments, outputs and errors are those of smla_bwd (no workspace), plus
 * SMLA_ERR_SCRATCH when even one token's chunk needs more than the scratch
 * (very wide rows or very many KV rows).  stream must belong to the current
 * device.  Nothing in the scratch needs to start at zero: every value read
 * in a call is written earlier in that call.  All calls on one GPU share its
 * scratch, so calls that overlap on one GPU (other streams, other threads)
 * race; serialise them.  dkv's bits follow the chunk size, so they can differ
 * from smla_bwd's with a larger workspace by the summation grouping.
 */
SMLA_API smla_status smla_bwd_noalloc(const smla_dims* dims, const void* q, const void* kv,
                             const void* dO, const float* lse, const float* delta,
                             const int32_t* topk_idxs, const int32_t* topk_length,
                             const float* attn_sink, void* dq, float* dkv, float* d_sink,
                             void* stream);

/* Static description of a status code. */
SMLA_API const char* smla_status_string(smla_status status);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
