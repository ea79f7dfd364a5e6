/*
 * siggate.h -- C ABI of the MI355X (gfx950) sigmoid group-limited MoE gate
 * and its expert-major dispatch.
 *
 * What the calls compute (sources are page titles and the part of the page):
 *
 *   siggate_forward  -- the router of DeepSeek-V3 / Kimi-K2
 *     (DeepSeek-V3.2-Exp · Normalize weights, "Code": Gate forward;
 *      Kimi K2 · Normalize weights, "Code": gate forward, and the equation
 *      for G_i; AI Engineer Exhaustive · DeepSeek-V3 MoE Router,
 *      "How it works"):
 *        L = x . W^T in float32 (x upcast from bfloat16, no linear bias),
 *        s = sigmoid(L), v = s + bias (bias steers the choice only),
 *        group score = sum of the two largest v of each of n_group groups,
 *        keep the topk_group best groups, mask the rest to -inf,
 *        take the top_k experts by v, gather the unbiased s at them,
 *        w = route_scale * s / sum(s over the top_k).
 *   siggate_dispatch -- the first lines of moe_infer
 *     (Kimi K2 · Add shared output, "Code": moe_infer; Kimi K3 · MoE
 *      update, moe_infer):
 *        tokens_per_expert = per-expert count of the (token, slot) pairs,
 *        perm = expert-major order of the flat pair ids p = t*top_k + k,
 *        permuted_x[pos] = x[perm[pos] / top_k].
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller; no call
 *     allocates device memory.  Every call except siggate_forward_noalloc
 *     keeps no state between calls and is reentrant (that one shares a
 *     static device scratch, see its declaration).  Every pointer must be
 *     16-byte aligned.
 *   - All arrays are dense row-major.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously; there is no host synchronisation.
 *     Argument errors are detected on the host before anything is enqueued
 *     and leave every output untouched.
 *   - A selection tie (equal choice scores, or equal group scores) goes to
 *     the LOWER expert / group index.  The pages leave the tie order open.
 *   - The dispatch permutation is stable: the pairs of one expert keep
 *     ascending p, i.e. ascending token id.  The pages use an unstable
 *     argsort, of which this is one valid result.
 *   - NaN or Inf in x, W or bias give undefined selections.
 *
 * Supported shapes (others return SIGGATE_EUNSUPPORTED):
 *   E a multiple of 64 up to 512; n_group a power of two with 1 <= n_group <= 64;
 *   1 <= top_k <= 8; d a positive multiple of 8; 0 <= T <= 2^31 / top_k.
 * Invalid configurations return SIGGATE_EINVAL: topk_group outside
 * [1, n_group], top_k > topk_group * E / n_group, order not 0 or 1,
 * score_func, renorm, mask_zero or logits_path out of range, denom_eps
 * negative or NaN.
 */
#ifndef SIGGATE_H
#define SIGGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Router hyper-parameters and problem size. */
typedef struct siggate_cfg {
    int32_t T;           /* tokens in the batch                               */
    int32_t d;           /* hidden size (7168 for DeepSeek-V3 and Kimi K2)    */
    int32_t E;           /* routed experts N_r (256 DeepSeek-V3, 384 Kimi K2) */
    int32_t n_group;     /* expert groups (8 DeepSeek-V3, 1 Kimi K2)          */
    int32_t topk_group;  /* groups kept per token (4 DeepSeek-V3, 1 Kimi K2)  */
    int32_t top_k;       /* experts per token K_r (8 for both)                */
    float route_scale;   /* 2.5 DeepSeek-V3, 2.827 Kimi K2                    */
    int32_t order;       /* output order of a token's top_k entries:
                            0 = ascending expert id,
                            1 = choice score descending (index ascending on ties) */
    /* Variants of the gate (all zero = the DeepSeek-V3 / Kimi-K2 gate above).
     * Sources: DeepSeek-V3.2-Exp · Normalize weights, "Code" (softmax branch;
     * group maximum without a bias; renormalise only for sigmoid) and Kimi K2
     * · Normalize weights, "Code" (0.0 fill of dropped groups, 1e-20 added to
     * the denominator, renormalisation behind a config flag). */
    int32_t score_func;  /* 0 = sigmoid, 1 = softmax over the E logits        */
    int32_t renorm;      /* 0 = renormalise iff sigmoid, 1 = always, 2 = never */
    int32_t mask_zero;   /* 0 = dropped groups -> -inf, 1 = -> 0.0             */
    float denom_eps;     /* added to the renormalisation denominator (>= 0)   */
    /* How the float32 logits are computed (both give float32 logits of the
     * same sum; the selection and everything after it are shared):
     *   0 = on the float32 matrix cores (v_mfma_f32_32x32x2_f32);
     *   1 = each float32 weight split exactly into three bfloat16 parts
     *       (W = hi + mid + lo), x * each part (exact products) added into
     *       float32 accumulators on the bfloat16 matrix cores
     *       (v_mfma_f32_16x16x32_bf16).  Every part is a normal number
     *       for |W| >= 2^-103 (smaller W may give subnormal parts);
     *       the logits differ from route 0 by float32 summation order only.
     * Accuracy on N(0,1)-sized logits at d = 7168: route 0 adds its
     * accumulators into float32 totals every 512 columns (blocked
     * summation), so its choice scores sigmoid(L) + b stay within about
     * 6e-7 of exact arithmetic; route 1 keeps one chain per half of d
     * (about 1.3e-6). */
    int32_t logits_path;
} siggate_cfg_t;

typedef enum siggate_status {
    SIGGATE_OK = 0,
    SIGGATE_EINVAL = -1,        /* invalid configuration or null/misaligned pointer */
    SIGGATE_EUNSUPPORTED = -2,  /* valid configuration this library does not build  */
    SIGGATE_EWORKSPACE = -3,    /* workspace smaller than siggate_workspace_bytes   */
    SIGGATE_EHIP = -4,          /* the HIP runtime reported a launch error          */
    SIGGATE_ESCRATCH = -5       /* siggate_forward_noalloc: the configuration needs
                                   more than SIGGATE_SCRATCH_BYTES of workspace     */
} siggate_status_t;

/* Size of the static device scratch of siggate_forward_noalloc: 128 MiB. */
#define SIGGATE_SCRATCH_BYTES ((size_t)128 << 20)

/* Bytes of device workspace that siggate_forward and siggate_dispatch need
 * for this configuration: the larger of the two needs, counting only a call
 * that accepts the configuration (0 if neither does; 0 is also possible for
 * an accepted configuration).  It depends on logits_path: route 1 always
 * needs float32 partial logits (n_split x T x E), and from T = 1024 on also
 * the three bfloat16 planes of W (3 x E x d rounded up to 32 columns, x 2
 * bytes), about 42 MB at T = 16384, E = 384, d = 7168. */
size_t siggate_workspace_bytes(const siggate_cfg_t *cfg);

/* Gate.
 *   x        bfloat16 [T, d]  (raw bfloat16 bits)
 *   W        float32  [E, d]  (router weight, one row per expert)
 *   bias     float32  [E]     (selection-only bias), or NULL: then the choice
 *                             score is the affinity itself and a group scores
 *                             by its largest member (DeepSeek-V3.2-Exp · Normalize
 *                             weights, "Code": the branch without a bias)
 *   weights  float32  [T, top_k]  out: route_scale * renormalised s
 *   indices  int32    [T, top_k]  out: selected expert ids
 *   ws       device workspace of ws_bytes >= siggate_workspace_bytes(cfg)
 *            (may be NULL when that is 0); its contents on entry do not
 *            matter and are garbage on return.
 * Calls that share a workspace must not overlap in time. */
siggate_status_t siggate_forward(const void *x, const float *W, const float *bias,
                                 const siggate_cfg_t *cfg, float *weights,
                                 int32_t *indices, void *ws, size_t ws_bytes,
                                 void *stream);

/* Gate that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same computation, kernels and
 * results as siggate_forward; the workspace is the library's static device
 * array of SIGGATE_SCRATCH_BYTES, one copy per device, allocated when the
 * library's code is loaded on that device and held until the process ends.
 *   - The stream must belong to the current device.
 *   - Every call on one device shares that device's scratch, so calls that
 *     overlap in time on one device (several streams, several host threads)
 *     race and give undefined results; calls on one stream are ordered.
 *   - Configurations whose gate workspace exceeds SIGGATE_SCRATCH_BYTES
 *     return SIGGATE_ESCRATCH before anything is enqueued.  At d = 7168
 *     every T fits on logits_path 0; on logits_path 1 every T <= 38314
 *     (E = 384) or <= 65536 (E = 256) fits, and larger batches fit or not
 *     by the plan's slice count (siggate_workspace_bytes tells).
 *   - The first call on a device looks up the scratch's device address
 *     (hipGetSymbolAddress); it calls no hipMalloc or hipFree, then or ever.
 * Other arguments and errors as siggate_forward. */
siggate_status_t siggate_forward_noalloc(const void *x, const float *W, const float *bias,
                                         const siggate_cfg_t *cfg, float *weights,
                                         int32_t *indices, void *stream);

/* Dispatch.
 *   x                  bfloat16 [T, d]
 *   indices            int32 [T, top_k], every entry in [0, E) and the
 *                      top_k entries of a token distinct (as the gate makes
 *                      them); entries out of range are undefined behaviour
 *   tokens_per_expert  int32 [E]        out
 *   offsets            int32 [E + 1]    out, exclusive prefix sum of
 *                      tokens_per_expert (may be NULL)
 *   perm               int32 [T*top_k]  out, perm[pos] = p
 *   dest               int32 [T*top_k]  out, dest[p] = pos, the inverse of
 *                      perm (may be NULL)
 *   permuted_x         bfloat16 [T*top_k, d] out, row pos = x[perm[pos] / top_k]
 *   ws                 device workspace (see siggate_forward)
 * Only T, d, E and top_k of cfg are used: 1 <= top_k <= 8, top_k <= E <= 512,
 * d a positive multiple of 8 (others return SIGGATE_EUNSUPPORTED or
 * SIGGATE_EINVAL). */
siggate_status_t siggate_dispatch(const void *x, const int32_t *indices,
                                  const siggate_cfg_t *cfg,
                                  int32_t *tokens_per_expert, int32_t *offsets,
                                  int32_t *perm, int32_t *dest, void *permuted_x,
                                  void *ws, size_t ws_bytes, void *stream);

/* Combine (Kimi K2 · Add shared output, "Code": moe_infer, last lines):
 * un-permute the expert outputs and add each token's top_k rows weighted by
 * its gate weights, in float32, then round to bfloat16 (nearest even):
 *   y[t, :] = bf16( sum_k weights[t, k] * expert_out[dest[t*top_k + k], :] )
 * with the sum taken in ascending k.
 *   expert_out  bfloat16 [n_pos, d] in dispatch (expert-major) order,
 *               n_pos = T * top_k
 *   weights     float32 [T, top_k]  (siggate_forward's weights)
 *   dest        int32 [T*top_k]     (siggate_dispatch's dest); entries
 *               outside [0, n_pos) are skipped (contribute nothing)
 *   y           bfloat16 [T, d]     out
 * Only T, d and top_k of cfg are used; needs no workspace. */
siggate_status_t siggate_combine(const void *expert_out, const float *weights,
                                 const int32_t *dest, const siggate_cfg_t *cfg,
                                 void *y, void *stream);

/* Expert-parallel metadata on one GPU (Kimi K2 · Add shared output, "Code":
 * moe_infer, the ep_size > 1 branch).  Experts are split into ep_size ranks
 * of per = E / ep_size consecutive experts (E % ep_size must be 0).
 *
 * Send splits: send_counts[r] = sum of tokens_per_expert over rank r's
 * experts (rows of the dispatch buffer that go to rank r, which are
 * contiguous because expert-major order is rank-major), send_offsets [ep_size
 * + 1] their exclusive prefix.  1 <= ep_size <= E <= 4096. */
siggate_status_t siggate_ep_send_splits(const int32_t *tokens_per_expert, int32_t E,
                                        int32_t ep_size, int32_t *send_counts,
                                        int32_t *send_offsets, void *stream);

/* Receive-side regroup.  counts [ep_size, per] (int32): rows received from
 * source rank r for local expert j, in arrival order rank by rank and, in a
 * rank, local expert by local expert.  Writes local_counts[j] = sum_r
 * counts[r, j] and regroup[q] = arrival index of the row that goes to
 * position q when the rows are put in local-expert order, stably (rows of one
 * expert keep arrival order).  Positions q >= capacity are not written: size
 * regroup by the received row count.  ep_size * per <= 4096. */
siggate_status_t siggate_ep_regroup(const int32_t *counts, int32_t ep_size, int32_t per,
                                    int32_t capacity, int32_t *local_counts,
                                    int32_t *regroup, void *stream);

/* De-duplicated send list: each token is sent once to every rank that holds
 * at least one of its top_k experts.
 *   indices       int32 [T, top_k] (the gate's indices; cfg gives T, E, top_k)
 *   rank_counts   int32 [ep_size]      out, distinct tokens per rank
 *   rank_offsets  int32 [ep_size + 1]  out, exclusive prefix
 *   send_tokens   int32 [T * top_k]    out, first rank_offsets[ep_size]
 *                 entries: token ids, rank-major, ascending in a rank
 *   pair_slot     int32 [T * top_k]    out, position in send_tokens of
 *                 (t, rank of the k-th expert of t)
 *   ws            siggate_ep_workspace_bytes(cfg, ep_size) bytes
 * ep_size <= 512. */
size_t siggate_ep_workspace_bytes(const siggate_cfg_t *cfg, int32_t ep_size);
siggate_status_t siggate_ep_dedup(const int32_t *indices, const siggate_cfg_t *cfg,
                                  int32_t ep_size, int32_t *rank_counts,
                                  int32_t *rank_offsets, int32_t *send_tokens,
                                  int32_t *pair_slot, void *ws, size_t ws_bytes,
                                  void *stream);

/* Test hook: the float32 logits L = x . W^T [T, E] that siggate_forward
 * selects from, computed by the same kernels in the same summation order
 * (for the same T). */
siggate_status_t siggate_logits(const void *x, const float *W,
                                const siggate_cfg_t *cfg, float *logits,
                                void *ws, size_t ws_bytes, void *stream);

/* Static, human-readable name of a status code. */
const char *siggate_status_str(siggate_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SIGGATE_H */
