/*
 * streamkl.h - C ABI of the StreamKL engine for AMD Instinct MI355X (gfx950).
 *
 * StreamKL computes, for every query row i of every (batch, head) slice, the KL divergence
 * KL(P1 || P2)[i] between two attention distributions P_t = softmax(scale * Q_t K_t^T) over the
 * keys, without ever forming an N_Q x N_K matrix, and the gradients of sum_i g_i * KL[i] in
 * two settings. Sources: "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting
 * Attention Distillation" as summarised on gist.science/pt/paper/2606.20005 ("Definicao do
 * Problema"; "Metodologia" sections 1-3) and gist.science/hi/paper/2606.20005 (technical
 * summary, same sections).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors q1, q2 are [batch, heads, n_q, head_dim] and k1, k2 are [batch, heads, n_k,
 *    head_dim], bfloat16, in device memory, addressed through the element strides of
 *    streamkl_problem_t (the head_dim axis is contiguous). All pointers must be 16-byte aligned
 *    and every stride a multiple of 8 elements. Row strides of 16 MiB or more are not supported
 *    (STREAMKL_ERROR_NOT_SUPPORTED): tiles are addressed with 32-bit offsets from a tile base.
 *  - Size limits (STREAMKL_ERROR_INVALID_VALUE beyond them): batch, heads, n_q, n_k and
 *    batch * heads below 2^30; batch * heads * (max(n_q, n_k) / 128 + 1) below 2^31 (grid
 *    size); each tensor's extent (from its first element to one past its last, through the
 *    strides) below 2^62 bytes and not wrapping past the top of the address space. The size
 *    queries return 0 for problems outside these limits.
 *  - Causal masking is top-left: key j is visible to query i iff j <= i. Every row then has at
 *    least one visible key.
 *  - Logits are S_t = scale * Q_t K_t^T; LSE values use the natural logarithm.
 *  - The caller owns every buffer. The library never allocates, frees or synchronises device
 *    memory; every call enqueues kernels on `stream` and returns without waiting. Buffers must
 *    stay valid until the stream has executed the work, and live on the device of `stream`
 *    (the current device for the null stream). There is no global mutable state apart
 *    from a thread-local error message, so calls from several host threads are safe.
 *  - Validation happens before anything is enqueued: an invalid call returns an error status
 *    and touches no buffer. A launch failure returns STREAMKL_ERROR_HIP; outputs are then
 *    undefined.
 *  - Non-finite inputs (NaN, infinity) are not checked. Every output that depends on one has an
 *    unspecified value (the kernels are built without NaN semantics, so a NaN is not
 *    guaranteed to reach the output); outputs that do not depend on it are unaffected. Per
 *    query row: kl, lse1, lse2 and the dQ row of query i depend only on row i of q1 / q2 and on
 *    every key; each dK row depends on every query row.
 *  - Inputs may alias each other (k2 == k1 and/or q2 == q1 are allowed and k2 == k1 is
 *    detected and loads the shared tensor once). Outputs must not overlap any input or each
 *    other (STREAMKL_ERROR_INVALID_VALUE).
 */
#ifndef STREAMKL_H
#define STREAMKL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STREAMKL_SUCCESS = 0,
  STREAMKL_ERROR_INVALID_VALUE = 1, /* bad pointer, size, stride, alignment or overlap */
  STREAMKL_ERROR_NOT_SUPPORTED = 2, /* valid but unsupported (head_dim, row stride, n_q) */
  STREAMKL_ERROR_HIP = 3            /* the HIP runtime reported an error (no device, launch) */
} streamkl_status_t;

typedef struct {
  int64_t batch;        /* >= 1 */
  int64_t heads;        /* >= 1 */
  int64_t n_q;          /* query rows per slice, >= 1 */
  int64_t n_k;          /* key rows per slice, >= 1 */
  int64_t head_dim;     /* 64 or 128 */
  int64_t q_stride[3];  /* element strides of (batch, head, row) for q1 and q2; row < 16 MiB */
  int64_t k_stride[3];  /* element strides of (batch, head, row) for k1 and k2; row < 16 MiB */
  float scale;          /* logit scale, finite and > 0 (1/sqrt(head_dim) is usual) */
  int32_t causal;       /* 0: every key visible; 1: top-left causal mask */
} streamkl_problem_t;

/*
 * Forward pass (gist.science/pt "Metodologia" section 1, "Formulacao Online"; saved state per
 * section 2, "Estado Salvo"; the split-K variant for small N_Q per section 3 and its gain under
 * "Resultados Experimentais", ablation).
 *
 * Streams key tiles through on-chip memory and keeps per query row the running maxima m1, m2,
 * the running sums of exponentials l1, l2 and the P1-weighted logit-difference accumulator acc,
 * all relative to the running maxima; then writes
 *     lse_t[i] = m_t + log l_t,      kl[i] = acc / l1 + lse2[i] - lse1[i].
 * The running maxima are raised on a row's first key tile and on tiles that need the causal or
 * ragged-end mask; other tiles are summed against the current maxima (the same sums up to
 * rounding). A row whose sums would leave the float32 range that way (a logit exceeding every
 * logit of its first tile by more than about 88 / (scale * log2(e)) in unscaled units, i.e.
 * 2^7 in exp2 units) is recomputed with the maxima raised on every tile.
 * Outputs (device, float32, contiguous [batch, heads, n_q], overwritten): kl, lse1, lse2.
 *
 * Adaptive: the kernels are chosen from the sizes alone. When few query blocks leave the chip
 * idle (streamkl_fwd_splitk_default_splits(problem) > 1: at most 256 work items unsplit) the
 * keys of every slice are cut into ranges, each range's partial online state goes to the
 * workspace and a second kernel merges them (as streamkl_fwd_splitk with n_splits = 0);
 * otherwise one pass (streamkl_fwd_one_pass) with no workspace. Either way the result is
 * bitwise deterministic for given sizes, and kl is exactly 0 where (Q1, K1) and (Q2, K2) hold
 * identical values.
 * workspace: device memory of at least streamkl_fwd_workspace_size(problem) bytes, 16-byte
 *   aligned, owned by the caller, overlapping no input or output; may be NULL when that size is
 *   0 (always the case at the large shapes, e.g. 32 heads x 64K rows). Contents on entry are
 *   ignored and on return unspecified.
 * Errors: STREAMKL_ERROR_INVALID_VALUE / _NOT_SUPPORTED for invalid or unsupported problems,
 *   pointers or overlaps and for a too small, NULL or misaligned workspace when one is needed.
 */
/* Workspace bytes streamkl_fwd needs for this problem (0 when it runs one pass, and for a NULL
 * problem or sizes < 1). */
size_t streamkl_fwd_workspace_size(const streamkl_problem_t* problem);
streamkl_status_t streamkl_fwd(const streamkl_problem_t* problem,
                               const void* q1, const void* k1, const void* q2, const void* k2,
                               float* kl, float* lse1, float* lse2, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * The one-pass forward kernel alone, whatever the sizes (no workspace): one block per 256 query
 * rows of a slice streams every visible key tile. Same outputs as streamkl_fwd; for callers that
 * want this kernel (or time it) at shapes where streamkl_fwd would split the keys.
 */
streamkl_status_t streamkl_fwd_one_pass(const streamkl_problem_t* problem, const void* q1,
                                        const void* k1, const void* q2, const void* k2,
                                        float* kl, float* lse1, float* lse2, hipStream_t stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same computation,
 * kernel choice and outputs as streamkl_fwd, but when the split-K path needs a workspace it
 * uses a scratch array that the library holds in device memory (one copy per GPU, kept until
 * the process ends) instead of a caller buffer. The call allocates nothing and frees nothing.
 * Limit: the split-K partial states must fit in streamkl_fwd_noalloc_max_workspace() bytes
 * (4 MiB). The default plan never needs more than 3.75 MiB (at most 256 work items unsplit, cut
 * into about 512 block items of 256 query rows or 1024 wavefront items of 32 rows, 5 floats per
 * row and key range), so every size runs; a plan beyond the scratch would return
 * STREAMKL_ERROR_NOT_SUPPORTED and enqueue nothing. The one-pass path needs no scratch.
 * Every call on a GPU shares that GPU's scratch: calls that may overlap on one GPU (several
 * streams, several host threads) race on it and must be ordered by the caller. The scratch is
 * fully written before it is read within a call, so no clearing is needed between calls. The
 * scratch copy used is the one on the device of `stream` (the current device for the null
 * stream); its address is looked up on the first call for that device.
 */
size_t streamkl_fwd_noalloc_max_workspace(void);
streamkl_status_t streamkl_fwd_noalloc(const streamkl_problem_t* problem, const void* q1,
                                       const void* k1, const void* q2, const void* k2,
                                       float* kl, float* lse1, float* lse2, hipStream_t stream);

/*
 * Forward pass with OCP fp8 e4m3 inputs (mixed precision for the two Q K^T contractions,
 * float32 state; mixed precision is named as future work in the agents-report article's
 * conclusion). Same outputs and semantics as streamkl_fwd, with
 * side t's logits S_t = scale * descale_t * Q_t K_t^T, where q_t, k_t hold e4m3 codes (1 byte,
 * bias 7, no infinities) and descale_t is the product of the two tensors' dequantisation
 * factors. Contractions run on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) with float32
 * accumulation; the online update is the bf16 forward's.
 *
 * Strides must be multiples of 16 elements (16 bytes); pointers 16-byte aligned.
 * descale1, descale2: finite and > 0 (STREAMKL_ERROR_INVALID_VALUE otherwise).
 */
streamkl_status_t streamkl_fwd_fp8(const streamkl_problem_t* problem, float descale1,
                                   float descale2, const void* q1, const void* k1,
                                   const void* q2, const void* k2, float* kl, float* lse1,
                                   float* lse2, hipStream_t stream);

/*
 * Split-K forward for few query rows (gist.science/pt "Resumo Tecnico", section "3. Otimizacoes
 * de Kernel de GPU", Split-K variant; its gain for small N_Q under "Resultados Experimentais",
 * ablation). Same outputs and semantics as streamkl_fwd, for any sizes.
 *
 * The keys of every slice are cut into n_splits contiguous ranges of whole key granules. With
 * n_q <= 32 a granule is a 32-key tile and each (slice, 32-row query block, range) is one
 * independent work item of one wavefront that reads its keys straight from memory; with
 * n_q > 32 a granule is one stage of the LDS-staged kernel (64 keys causal, 128 keys without
 * the mask) and each (slice, 256-row query block, range) is one block of that kernel, so that
 * the query rows of a block share every key read. Either way the work item writes the partial online state (m1, l1, m2, l2, acc) of its
 * rows to the workspace; a second kernel merges the ranges of each row (the online state of a
 * union of key sets follows from the states of its parts: the larger maximum wins and the other
 * sums are rescaled) and writes kl, lse1, lse2. Results agree with streamkl_fwd to float32
 * rounding (summation order differs) and are bitwise deterministic for a given n_splits.
 *
 * n_splits: requested number of ranges; <= 0 chooses streamkl_fwd_splitk_default_splits().
 *   The number used is min(n_splits, number of key granules, 4096), then reduced so that no
 *   range is empty.
 * workspace: device memory of at least streamkl_fwd_splitk_workspace_size(problem, n_splits)
 *   bytes, 16-byte aligned, owned by the caller, not overlapping any input or output; its
 *   contents on entry are ignored and on return are unspecified. It holds float32
 *   [batch * heads][ranges used][5][n_q].
 * Errors: as streamkl_fwd, plus STREAMKL_ERROR_INVALID_VALUE for a NULL, misaligned,
 *   overlapping or too small workspace.
 */
/* Number of key ranges chosen for n_splits <= 0: about 1024 wavefront work items (n_q <= 32)
 * or 512 block work items (n_q > 32), with at least 8 key granules per range (only keys some
 * row can see count when causal); 1 when there are more than 256 work items without splitting,
 * where streamkl_fwd is the faster path. 0 for a NULL problem or sizes < 1. */
int32_t streamkl_fwd_splitk_default_splits(const streamkl_problem_t* problem);
/* Workspace bytes streamkl_fwd_splitk needs for this n_splits; 0 for a NULL problem or sizes
 * < 1. */
size_t streamkl_fwd_splitk_workspace_size(const streamkl_problem_t* problem, int32_t n_splits);
streamkl_status_t streamkl_fwd_splitk(const streamkl_problem_t* problem,
                                      const void* q1, const void* k1, const void* q2,
                                      const void* k2, float* kl, float* lse1, float* lse2,
                                      int32_t n_splits, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * Workspace of the backward entry points streamkl_bwd_fixP1 / _fixP2 (gist.science/pt
 * "Metodologia" section 2, kernel fusion: the dQ buffer of the fused variant; "Resultados
 * Experimentais", ablation: the choice between fused and separate kernels adapts to N_Q).
 * Both settings choose their kernels from the sizes alone, the same way:
 *   - n_q <= 64: the fused single visit (as streamkl_bwd_fused): dS formed once per key group
 *     for both gradients, per-key-block partial dQ in the workspace, summed in a fixed order;
 *   - else, while the one-kernel dQ pass has fewer than 256 blocks: dQ with the keys split into
 *     ranges (as streamkl_bwd_dq_splitk with n_splits = 0, partials in the workspace) and the
 *     one-kernel dK pass;
 *   - else: the one-kernel dQ and dK passes (streamkl_bwd_dq + streamkl_bwd_dk), no workspace.
 * Returns the bytes that choice needs (0 for the last case, e.g. 32 heads x 64K rows; 0 for a
 * NULL problem, sizes < 1 or an unsupported head_dim).
 */
size_t streamkl_bwd_workspace_size(const streamkl_problem_t* problem);

/*
 * Backward, setting 1: P1 fixed (stop-gradient), P2 free - standard distillation
 * (gist.science/pt "Metodologia" section 2, "Configuracao 1").
 *
 * Regenerates P_t = exp(S_t - lse_t) tile by tile from the saved lse1, lse2 and the inputs,
 * forms dS2 = g_i * (P2 - P1) and writes the gradients of sum_i g_i * KL[i] w.r.t. Q2 and K2:
 *     dq2 = scale * dS2 K2,   dk2 = scale * dS2^T Q2.
 * lse1, lse2, grad_kl: device float32 contiguous [batch, heads, n_q]; lse_t as written by
 * streamkl_fwd for the same inputs. grad_kl holds g_i (any real values).
 * Outputs dq2 [batch, heads, n_q, head_dim] and dk2 [batch, heads, n_k, head_dim]: device
 * bfloat16, contiguous, overwritten; accumulation is float32. With k2 == k1, dk2 is the
 * gradient through the student side only. The kernels are chosen as described at
 * streamkl_bwd_workspace_size; no path uses atomics and every sum has a fixed order, so the
 * result is bitwise deterministic for given sizes.
 * workspace: at least streamkl_bwd_workspace_size(problem) bytes of device memory, 16-byte
 *   aligned, owned by the caller, overlapping no input or output; may be NULL when that size
 *   is 0. Contents on entry ignored, on return unspecified.
 * Errors: STREAMKL_ERROR_INVALID_VALUE / _NOT_SUPPORTED for invalid or unsupported problems,
 *   pointers or overlaps and for a too small, NULL or misaligned workspace when one is needed.
 */
streamkl_status_t streamkl_bwd_fixP1(const streamkl_problem_t* problem,
                                     const void* q1, const void* k1, const void* q2,
                                     const void* k2, const float* lse1, const float* lse2,
                                     const float* grad_kl, void* dq2, void* dk2,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * Backward, setting 2: P2 fixed (stop-gradient), P1 free (gist.science/pt "Metodologia"
 * section 2, "Configuracao 2"; the log-ratio follows section 3, "Estabilidade Numerica").
 *
 * Forms dS1 = g_i * P1 * (log P1 - log P2 - KL[i]) with the log-ratio taken from logit
 * differences and saved LSEs, (S1 - lse1) - (S2 - lse2), never from the log of a probability,
 * and writes  dq1 = scale * dS1 K1,  dk1 = scale * dS1^T Q1.
 * kl: the forward's saved KL, device float32 contiguous [batch, heads, n_q]; other arguments,
 * the kernel choice, the workspace and the errors as in streamkl_bwd_fixP1. Outputs dq1, dk1:
 * device bfloat16, contiguous, overwritten.
 */
streamkl_status_t streamkl_bwd_fixP2(const streamkl_problem_t* problem,
                                     const void* q1, const void* k1, const void* q2,
                                     const void* k2, const float* lse1, const float* lse2,
                                     const float* kl, const float* grad_kl, void* dq1, void* dk1,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * The two halves of a backward call, one kernel each, for callers that need only one gradient
 * (for example when K is frozen and only dQ is wanted) or that time the kernels separately.
 * streamkl_bwd_dq + streamkl_bwd_dk with setting = 1 is what streamkl_bwd_fixP1 runs at large
 * sizes, and setting = 2 likewise for streamkl_bwd_fixP2 (gist.science/pt "Metodologia" section 2:
 * dQ accumulates along K, dK along Q; here each runs in its own kernel and neither needs
 * atomics).
 * setting: 1 (P1 fixed; writes dq2 / dk2) or 2 (P2 fixed; writes dq1 / dk1). kl is read only for
 * setting 2 and may be NULL for setting 1. Other arguments as in streamkl_bwd_fixP1 / _fixP2;
 * dq (or dk) is the one output, contiguous bfloat16 [batch, heads, n_q (or n_k), head_dim].
 */
streamkl_status_t streamkl_bwd_dq(const streamkl_problem_t* problem, int32_t setting,
                                  const void* q1, const void* k1, const void* q2, const void* k2,
                                  const float* lse1, const float* lse2, const float* kl,
                                  const float* grad_kl, void* dq, hipStream_t stream);
streamkl_status_t streamkl_bwd_dk(const streamkl_problem_t* problem, int32_t setting,
                                  const void* q1, const void* k1, const void* q2, const void* k2,
                                  const float* lse1, const float* lse2, const float* kl,
                                  const float* grad_kl, void* dk, hipStream_t stream);

/*
 * dQ with the keys split into ranges, for few query rows: the adaptive side of the backward
 * (gist.science/pt "Resumo Tecnico": "Metodologia" section 2, kernel fusion and the conflict
 * between accumulating dQ along K and dK along Q; "Resultados Experimentais", ablation: the
 * kernel choice adapts to small N_Q). With few query rows the dQ kernel has one block per
 * 256-row query block and slice, too few for the chip; here block (query block, slice, range)
 * handles one contiguous range of 32-key tiles, writes its float32 partial dQ to the workspace,
 * and a second kernel sums the ranges and rounds once to bfloat16. No atomics: the result is
 * deterministic for a given n_splits and agrees with streamkl_bwd_dq to float32 summation
 * order before the rounding.
 *
 * n_splits: requested ranges; <= 0 chooses streamkl_bwd_dq_splitk_default_splits(). The number
 *   used is min(n_splits, visible key tiles, 1024), reduced so that no range is empty. With one
 *   range this is streamkl_bwd_dq and the workspace is not touched.
 * workspace: at least streamkl_bwd_dq_splitk_workspace_size(problem, n_splits) bytes of device
 *   memory (0 for one range), 16-byte aligned, owned by the caller, overlapping no input or
 *   output; contents on entry ignored, on return unspecified. It holds float32
 *   [ranges used][batch * heads][n_q][head_dim].
 * Other arguments and errors as streamkl_bwd_dq, plus STREAMKL_ERROR_INVALID_VALUE for a too
 * small, misaligned or overlapping workspace.
 */
/* Ranges chosen for n_splits <= 0: about one block per CU with at least 16 key tiles per range;
 * 1 when the dQ kernel already has 256 blocks or more. 0 for a NULL problem or sizes < 1. */
int32_t streamkl_bwd_dq_splitk_default_splits(const streamkl_problem_t* problem);
/* Workspace bytes streamkl_bwd_dq_splitk needs for this n_splits (0 with one range, and for a
 * NULL problem or sizes < 1). */
size_t streamkl_bwd_dq_splitk_workspace_size(const streamkl_problem_t* problem,
                                             int32_t n_splits);
streamkl_status_t streamkl_bwd_dq_splitk(const streamkl_problem_t* problem, int32_t setting,
                                         const void* q1, const void* k1, const void* q2,
                                         const void* k2, const float* lse1, const float* lse2,
                                         const float* kl, const float* grad_kl, void* dq,
                                         int32_t n_splits, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * Fused backward for few query rows (n_q <= 64): the pages' fused single visit of the key
 * tiles for small N_Q (gist.science/pt "Resumo Tecnico": "Metodologia" section 2, kernel fusion;
 * "Resultados Experimentais", ablation: fused against separate backward kernels for small N_Q).
 * One key-major pass recomputes S1 and S2 per (query tile, 32-key group), forms dS of the
 * setting's free side once, and uses it for both products: dK of the group's keys is written
 * directly, and the block's partial dQ (its 128 * G keys) goes to the workspace; a second kernel sums
 * the key blocks' partials in a fixed order and rounds once to bfloat16. The keys are read once
 * instead of once per gradient. No atomics: the four waves of a block add their partial dQ in
 * LDS in wave order, so the result is bitwise deterministic, and agrees with streamkl_bwd_dq /
 * streamkl_bwd_dk to float32 summation order before the rounding.
 *
 * setting: 1 (P1 fixed; outputs dQ2, dK2, kl unused and may be NULL) or 2 (P2 fixed; outputs
 *   dQ1, dK1, kl required).
 * dq, dk: contiguous bfloat16 [batch, heads, n_q, head_dim] and [batch, heads, n_k, head_dim].
 * workspace: at least streamkl_bwd_fused_workspace_size(problem) bytes of device memory,
 *   16-byte aligned, owned by the caller, overlapping no input or output; contents on entry
 *   ignored, on return unspecified. It holds float32 [ceil(n_k / (128 G))][batch * heads][n_q]
 *   [head_dim], where G, the 32-key groups per wave, is floor(S * batch * heads / 256) clamped to
 *   [1, min(64, S)] with S = ceil(n_k / 128) (about one block per CU).
 * Errors: as streamkl_bwd_fixP1 / _fixP2; STREAMKL_ERROR_NOT_SUPPORTED for n_q > 64;
 * STREAMKL_ERROR_INVALID_VALUE for a bad setting or a too small, misaligned or overlapping
 * workspace.
 */
/* Workspace bytes streamkl_bwd_fused needs (0 for a NULL problem, sizes < 1, n_q > 64 or an
 * unsupported head_dim). */
size_t streamkl_bwd_fused_workspace_size(const streamkl_problem_t* problem);
streamkl_status_t streamkl_bwd_fused(const streamkl_problem_t* problem, int32_t setting,
                                     const void* q1, const void* k1, const void* q2,
                                     const void* k2, const float* lse1, const float* lse2,
                                     const float* kl, const float* grad_kl, void* dq, void* dk,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* streamkl_status_string(streamkl_status_t status);

/* Detail of the last failed call on the calling host thread ("" if none). Valid until the
 * next call on that thread. */
const char* streamkl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_H */
