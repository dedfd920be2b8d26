/*
 * moelora.h -- C ABI of libmoelora, the MoE expert-MLP layer with Split LoRA on one MI355X
 * (gfx950). Forward and backward of
 *
 *     y_t = sum_{i in TopK(score(x_t W_r))} s_{t,i} * Expert_i(x_t),
 *     Expert_e(x) = (silu(x Wg_e + c (x Ag_e) Bg_e) * (x Wu_e + c (x Au_e) Bu_e)) Wd_e
 *                   + c ((...) Ad_e) Bd_e,                          c = alpha / r,
 *
 * the routing equation of the ailinkdeeptech.com cookbook page "Accelerating Mixture-of-Experts
 * Fine-Tuning: Unsloth Faster MoE, Split LoRA, and Grouped GEMM" (section "The Dynamic Dispatch
 * Bottleneck in Mixture-of-Experts Architectures") with every expert projection evaluated as
 * Split LoRA, Y = XW + (alpha/r)(XA)B (same page, section "2. Split LoRA Associative
 * Transformation"), never forming the m x n product of the LoRA factors. The expert weights are
 * one fused tensor per projection, gate and up concatenated along the output axis, gate first
 * (unsloth.ai "Faster MoE" documentation page, section on torch._grouped_mm).
 *
 * Conventions (all calls):
 *  - Tensors are caller-owned DEVICE pointers, dense row-major, 16-byte aligned. The library never
 *    allocates device memory, keeps no state between calls (apart from the opt-in stage timing
 *    below), never prints and never aborts.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream). Buffers must
 *    stay valid until the work on `stream` has finished.
 *  - All argument checks run on the host before anything is enqueued; on any error nothing is
 *    enqueued and a status other than MOE_OK is returned. MOE_ERR_HIP reports a failed launch.
 *  - Outputs are overwritten, never accumulated into.
 *  - Element type of X, W_r, weights, LoRA factors, Y, dY, dX: `shape->dtype` (fp32 or bf16).
 *    Routing weights, logits and LoRA-factor gradients are fp32; indices are int32.
 *  - Weights use the x.W orientation: W_r [m, E]; W_gu [E, m, 2n] (columns [0,n) gate, [n,2n) up);
 *    W_d [E, n, m]; A_g, A_u [E, m, r]; B_g, B_u [E, r, n]; A_d [E, n, r]; B_d [E, r, m].
 *    With MOE_FLAG_WEIGHTS_OUT_IN the two base expert tensors are stored output-major instead:
 *    W_gu [E, 2n, m] (rows [0,n) gate, [n,2n) up) and W_d [E, m, n].
 *  - Pair id p = t*k + j (token t, slot j of its selection order); P = s*k pairs.
 *
 * Supported shapes: s >= 0; m and n multiples of 64; 1 <= k <= E <= 1024; 1 <= r <= 64, and for
 * bf16 r a multiple of 8; s*k < 2^31 (pair and row indices are int32; element
 * offsets are 64-bit, so activations and intermediates may exceed 2^31 elements). Anything else
 * returns MOE_ERR_UNSUPPORTED (there is no fallback path).
 */
#ifndef MOELORA_H
#define MOELORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1 /* null or misaligned pointer, bad enum, inconsistent sizes */
#define MOE_ERR_UNSUPPORTED 2 /* a shape or mode the kernels do not implement */
#define MOE_ERR_WORKSPACE 3   /* a state/saved/workspace buffer smaller than its size query */
#define MOE_ERR_HIP 4         /* a kernel launch failed */

#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

#define MOE_SCORE_SOFTMAX 0 /* softmax over all E logits */
#define MOE_SCORE_SIGMOID 1 /* 1 / (1 + exp(-z)) per logit */

/* flags */
#define MOE_FLAG_REFERENCE_GEMM 1 /* run every GEMM with the plain one-thread-per-output kernels */
/* rank-stabilised LoRA scale c = alpha / sqrt(r) instead of alpha / r (bluecore.net/archives/629,
 * LoRA section, rsLoRA item) */
#define MOE_FLAG_RSLORA 2
/* base expert weights output-major, W_gu [E, 2n, m] and W_d [E, m, n]: the one-tensor-per-projection
 * layout that the unsloth.ai "Faster MoE" page shows for Transformers v5 (section "What is
 * torch._grouped_mm?"); the LoRA factors keep their shapes */
#define MOE_FLAG_WEIGHTS_OUT_IN 4
/* moe_lora_forward only: W_gu and W_d hold merged weights from moe_peft_merge; the LoRA factors
 * are not read (may be NULL) and no Split-LoRA work runs. moe_lora_backward rejects it
 * (MOE_ERR_UNSUPPORTED). */
#define MOE_FLAG_MERGED 8
/* moe_lora_backward may be called with saved == NULL: it then recomputes the forward's expert
 * intermediates (gu, h, the low-rank products, o) into its workspace first, trading one more
 * forward's GEMMs for the saved buffer (bluecore.net/archives/629, section 4 on Unsloth's gradient
 * checkpointing: activations are not kept and the forward is recomputed in the backward). With
 * this flag moe_bwd_ws_bytes includes that room; the forward may then run with saved == NULL. */
#define MOE_FLAG_RECOMPUTE 16
/* one LoRA pair on the fused gate/up projection instead of one per projection: the adapter targets
 * the single gate_up_proj tensor (unsloth.ai "Faster MoE" page, section "Faster LoRA MoE
 * training", the target_modules list of its get_peft_model example), so Delta W_gu = c A B with
 * A [E, m, r] passed as A_g and B [E, r, 2n] (gate columns [0, n), then up columns [n, 2n), as in
 * W_gu) passed as B_g. A_u and B_u are not read (may be NULL). moe_lora_backward writes dA [E, m, r]
 * to dA_g and dB [E, r, 2n] to dB_g and leaves dA_u and dB_u untouched (may be NULL); moe_peft_merge
 * merges the pair into both halves of W_gu. */
#define MOE_FLAG_FUSED_GU_LORA 32

typedef struct moe_shape {
  int32_t s;           /* tokens */
  int32_t m;           /* hidden size */
  int32_t n;           /* expert intermediate size */
  int32_t E;           /* experts */
  int32_t k;           /* experts per token */
  int32_t r;           /* LoRA rank */
  float alpha;         /* LoRA alpha; the LoRA scale is c = alpha / r (alpha / sqrt(r) with RSLORA) */
  int32_t dtype;       /* MOE_DTYPE_* */
  int32_t score;       /* MOE_SCORE_* */
  int32_t renormalize; /* 1: s_{t,j} = p_j / sum of the token's k selected p; 0: s_{t,j} = p_j */
  int32_t router_grad; /* 1: dX includes the path through the routing weights (top-k set fixed) */
  int32_t flags;       /* MOE_FLAG_* */
} moe_shape;

/* Name of a status code (static string). */
const char* moe_status_str(moe_status st);
/* ABI version of this header (incremented on any incompatible change). */
int32_t moe_abi_version(void);
/* Checks a shape without enqueuing anything: MOE_OK or the status any call would return. */
moe_status moe_check_shape(const moe_shape* shape);

/* Size queries (bytes). Return 0 for an invalid or unsupported shape. */
size_t moe_route_state_bytes(const moe_shape* shape);
size_t moe_fwd_saved_bytes(const moe_shape* shape);
/* Forward scratch; with_saved = 0 (inference, saved == NULL) also covers the intermediates that
 * would otherwise live in `saved`. */
size_t moe_fwd_ws_bytes(const moe_shape* shape, int32_t with_saved);
size_t moe_bwd_ws_bytes(const moe_shape* shape);

/*
 * moe_route -- router logits, top-k selection, routing weights and grouping of the P pairs into
 * contiguous per-expert runs.
 *   logits z = X W_r (+ router_bias), fp32 accumulate. Per token the k largest logits are selected
 *   (equal logits: lower expert id first; a NaN logit counts as -inf, so it is never selected
 *   before a number, scores 0, and every id written lies in [0, E)); slot j is the j-th selection. Scores: softmax over all E
 *   (MOE_SCORE_SOFTMAX) or sigmoid; weights s_{t,j} renormalised over the k selected when
 *   shape->renormalize. Grouping: expert_off[e] = number of pairs routed to experts < e
 *   (expert_off[E] = P); perm[row] = pair id, ordered by expert then token; inv_perm[pair] = row.
 * In:  X [s, m], W_r [m, E], router_bias [E] fp32 or NULL (a fixed per-expert logit bias).
 * Out: logits [s, E] fp32 (may be NULL), topk_idx [s, k] int32, topk_w [s, k] fp32,
 *      expert_off [E + 1] int32, perm [P] int32, inv_perm [P] int32.
 * route_state: >= moe_route_state_bytes(shape) bytes; keeps per-pair scores and the row tables the
 *      forward and backward calls read; must stay untouched until the backward has run.
 */
moe_status moe_route(const moe_shape* shape, const void* X, const void* W_r,
                     const float* router_bias, float* logits, int32_t* topk_idx, float* topk_w,
                     int32_t* expert_off, int32_t* perm, int32_t* inv_perm, void* route_state,
                     size_t route_state_bytes, void* stream);

/*
 * moe_lora_forward -- Y [s, m] = sum_j topk_w[t, j] * Expert_{topk_idx[t, j]}(X[t]).
 * The pairs are gathered into per-expert runs (Xp[row] = X[perm[row] / k]); per expert, one
 * grouped GEMM computes [g | u] = Xp W_gu + c [(Xp A_g) B_g | (Xp A_u) B_u] and h = silu(g) * u,
 * a second computes o = h W_d + c (h A_d) B_d; the combine sums the k rows of each token weighted
 * by topk_w in slot order (fp32 accumulate).
 * Routing arguments and route_state come from moe_route on the same X and shape.
 * saved: >= moe_fwd_saved_bytes bytes, receives what moe_lora_backward needs; NULL for inference.
 * ws: >= moe_fwd_ws_bytes(shape, saved != NULL) bytes of scratch (may be NULL if that is 0).
 */
moe_status moe_lora_forward(const moe_shape* shape, const void* X, const int32_t* topk_idx,
                            const float* topk_w, const int32_t* expert_off, const int32_t* perm,
                            const int32_t* inv_perm, const void* route_state, const void* W_gu,
                            const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                            const void* B_u, const void* A_d, const void* B_d, void* Y, void* saved,
                            size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_lora_backward -- gradients of the layer for upstream gradient dY [s, m]. The base weights
 * and the router are frozen; only the LoRA factors train (unsloth.ai "Faster MoE" page, section
 * "Implementation details").
 * Out: dX [s, m] (dtype): through the experts, plus through the routing weights when
 *      shape->router_grad (softmax without renormalisation is then MOE_ERR_UNSUPPORTED);
 *      dA_g, dA_u [E, m, r], dB_g, dB_u [E, r, n], dA_d [E, n, r], dB_d [E, r, m], all fp32.
 *      Experts that received no pair get exact zeros.
 * In: the routing outputs and route_state of moe_route, the same weights as the forward, and the
 *     `saved` buffer that moe_lora_forward filled (or NULL with MOE_FLAG_RECOMPUTE).
 *     ws >= moe_bwd_ws_bytes bytes of scratch.
 */
moe_status moe_lora_backward(const moe_shape* shape, const void* dY, const void* X,
                             const void* W_r, const int32_t* topk_idx, const float* topk_w,
                             const int32_t* expert_off, const int32_t* perm,
                             const int32_t* inv_perm, const void* route_state, const void* W_gu,
                             const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                             const void* B_u, const void* A_d, const void* B_d, const void* saved,
                             size_t saved_bytes, void* dX, float* dA_g, float* dB_g, float* dA_u,
                             float* dB_u, float* dA_d, float* dB_d, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * moe_lora_forward_noalloc -- moe_lora_forward for inference (saved == NULL) that allocates
 * nothing and takes no workspace argument: for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation). Same arguments,
 * semantics and results as moe_lora_forward(shape, ..., Y, NULL, 0, ws, ws_bytes, stream); its
 * scratch is a fixed array of MOE_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 * every GPU it runs on until the process ends.
 * Limit: moe_fwd_ws_bytes(shape, 0) <= MOE_NOALLOC_SCRATCH_BYTES (about 1 900 tokens of the
 * Qwen3-30B-A3B layer, 128 experts, top-8); larger shapes return MOE_ERR_WORKSPACE and enqueue
 * nothing.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (on different streams,
 * or from several host threads without ordering) race and must not be made. Nothing needs clearing
 * between calls; the array keeps the last call's intermediates.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_lora_forward_noalloc(const moe_shape* shape, const void* X, const int32_t* topk_idx,
                                    const float* topk_w, const int32_t* expert_off, const int32_t* perm,
                                    const int32_t* inv_perm, const void* route_state, const void* W_gu,
                                    const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                                    const void* B_u, const void* A_d, const void* B_d, void* Y,
                                    void* stream);

/*
 * moe_peft_merge -- the materialised form of the LoRA update that Split LoRA avoids
 * (ailinkdeeptech.com cookbook page, section "1. Standard PEFT Materialization Overhead"):
 *     W_gu' = W_gu + c [A_g B_g | A_u B_u],   W_d' = W_d + c A_d B_d      (per expert)
 * fp32 products rounded to dtype, in the base weights' orientation (x.W, or output-major with
 * MOE_FLAG_WEIGHTS_OUT_IN). Out: W_gu_merged and W_d_merged, shaped like W_gu and W_d (distinct
 * buffers). Feeds moe_lora_forward with MOE_FLAG_MERGED, to set the two evaluation orders side by
 * side; no training call needs it.
 */
moe_status moe_peft_merge(const moe_shape* shape, const void* W_gu, const void* W_d, const void* A_g,
                          const void* B_g, const void* A_u, const void* B_u, const void* A_d,
                          const void* B_d, void* W_gu_merged, void* W_d_merged, void* stream);

/*
 * Shared expert -- a dense SwiGLU expert that every token passes through, beside the routed ones,
 * with its output added to theirs (the DeepSeek-MoE-style layer of GLM 4.7 Flash: 64 routed experts
 * and 1 shared expert; unsloth.ai "Faster MoE" page, section "GLM 4.7 Benchmarks"). Its three
 * projections carry their own Split-LoRA pairs:
 *     [g | u] = X W_gu + c [(X A_g) B_g | (X A_u) B_u],  h = silu(g) * u,
 *     Y += h W_d + c (h A_d) B_d
 * shape: s, m, n (the shared expert's intermediate size), r, alpha, dtype and the flags RSLORA,
 * WEIGHTS_OUT_IN, FUSED_GU_LORA, RECOMPUTE, REFERENCE_GEMM apply; E, k, score, renormalize and
 * router_grad are not read. MERGED is MOE_ERR_UNSUPPORTED. Weights are those of one expert:
 * W_gu [m, 2n], W_d [n, m] (or output-major), A_g, A_u [m, r], B_g, B_u [r, n], A_d [n, r],
 * B_d [r, m] (fused gate/up pair: A [m, r] in A_g, B [r, 2n] in B_g).
 *
 * moe_shared_forward: Y [s, m] += the expert's output (call it on the Y of moe_lora_forward).
 *     saved (>= moe_shared_saved_bytes, 256-byte aligned) keeps gu, h and the low-rank products for
 *     the backward; NULL for inference. ws >= moe_shared_fwd_ws_bytes(shape, saved != NULL).
 * moe_shared_backward: dX [s, m] += the expert's input gradient (call it on the dX of
 *     moe_lora_backward); dA_*, dB_* (fp32, shaped like the factors) are overwritten. dO = dY.
 *     saved from moe_shared_forward, or NULL with MOE_FLAG_RECOMPUTE.
 *     ws >= moe_shared_bwd_ws_bytes. With s == 0 the gradients are zeroed and dX is untouched.
 * Both are asynchronous on `stream`; errors as for the routed calls (nothing is enqueued).
 */
size_t moe_shared_saved_bytes(const moe_shape* shape);
size_t moe_shared_fwd_ws_bytes(const moe_shape* shape, int32_t with_saved);
size_t moe_shared_bwd_ws_bytes(const moe_shape* shape);
moe_status moe_shared_forward(const moe_shape* shape, const void* X, const void* W_gu, const void* W_d,
                              const void* A_g, const void* B_g, const void* A_u, const void* B_u,
                              const void* A_d, const void* B_d, void* Y, void* saved, size_t saved_bytes,
                              void* ws, size_t ws_bytes, void* stream);
moe_status moe_shared_backward(const moe_shape* shape, const void* dY, const void* X, const void* W_gu,
                               const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                               const void* B_u, const void* A_d, const void* B_d, const void* saved,
                               size_t saved_bytes, void* dX, float* dA_g, float* dB_g, float* dA_u,
                               float* dB_u, float* dA_d, float* dB_d, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * Stage timing (diagnostics, off by default). While enabled, every call records a hipEvent pair on
 * its stream around each kernel stage (host-side state in the library; no device memory).
 * moe_timing_read waits for the recorded events, writes per-stage summed milliseconds and counts
 * into arrays of nstages >= moe_timing_stage_count() entries, and resets the sums.
 */
moe_status moe_timing_enable(int32_t on);
int32_t moe_timing_stage_count(void);
const char* moe_timing_stage_name(int32_t stage); /* NULL for an out-of-range index */
moe_status moe_timing_read(double* total_ms, int64_t* counts, int32_t nstages);

#ifdef __cplusplus
}
#endif
#endif /* MOELORA_H */
