/*
 * moe_lora.h -- C ABI of the MI355X (gfx950) MoE expert layer with split LoRA.
 *
 * The layer, as the two source pages describe it:
 *
 *  - Routing: the one-pass grouping from the article on Unsloth x NVIDIA
 *    training optimisations (m.yhxrc.cn), section "Optimisation 3: MoE routing
 *    grouped once": flatten every token's top-k expert assignments, sort them
 *    stably by expert id, take all per-expert counts with one bincount, derive
 *    offsets from the counts and slice the sorted list at those offsets.  The
 *    per-expert search loop it replaces needs one data-dependent query per
 *    expert; here nothing is ever read back to the host.
 *
 *  - Expert MLP: the Unsloth documentation page "Fine-tune MoE models 12x
 *    faster with Unsloth".  Experts are stored as single stacked parameters
 *    ("What is torch._grouped_mm?": gate_up [E, 2n, d], split into gate and up
 *    halves after the projection); LoRA is kept split, i.e. X W^T + s (X A) B,
 *    never merging B A^T into W ("Faster LoRA MoE training"; identical outputs
 *    and gradients in exact arithmetic); an adapter on a weight of shape
 *    (m, n) is A (m, r), B (r, n) ("Implementation details"); only A and B are
 *    trained and the router stays frozen.
 *
 * Readings where the pages are silent: top-k ties go to the lower expert id;
 * routing weights are the softmax of the k selected logits; offsets are
 * exclusive with offsets[E] = T*k; gate is the first half of gate_up's rows;
 * the activation is SwiGLU, h = silu(gate) * up; one optional shared expert is
 * stacked as expert index E with weight 1 for every token.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors), contiguous, row-major, 16-byte aligned.  16-bit tensors are
 *    passed as raw 16-bit patterns (moe_bf16; fp16 bits when dims->dtype is
 *    MOE_F16).
 *  - The caller owns every buffer.  The library allocates no device memory,
 *    frees nothing and keeps no pointer after returning; its only mutable
 *    global state is the opt-in kernel-timing recorder and the per-shape
 *    engine table, both declared at the end of this file.  Calls on
 *    different streams are independent.
 *  - Inputs are never written.  Outputs must not alias inputs or each other.
 *  - Outputs are overwritten, never accumulated into (an expert that receives
 *    no rows gets exactly zero LoRA gradients).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  No call synchronises the host or copies to the host,
 *    except moe_autotune and moe_timing_report, which wait for their own
 *    work.  The other calls allocate nothing, enqueue no memset and never
 *    wait, so they can be captured into a HIP graph; a replay reuses the
 *    pointers and sizes given at capture.
 *  - The return code covers host-side validation and launch errors only; on
 *    any error nothing has been enqueued except in the MOE_ERROR_LAUNCH case.
 *  - Device-side data errors (an expert id outside [0, E) in a routing
 *    struct that did not come from moe_route) are not detected; results are
 *    then undefined.
 *  - Non-finite logits never produce an invalid id: NaN ranks below every
 *    other value (-inf included) and equal NaNs go to the lower id, like any
 *    other tie.  The routing weights of a token are defined only when its k
 *    selected logits are finite (otherwise they may be NaN).
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16; /* raw bf16 bits */

typedef enum {
  MOE_SUCCESS = 0,
  MOE_ERROR_INVALID_VALUE = 1, /* null/misaligned pointer, T < 1, k not in [1,E], r < 1,
                                  n_shared not in {0,1}, d or n < 1, non-finite lora_scale */
  MOE_ERROR_UNSUPPORTED = 2,   /* outside the kernel envelope: d or n not a multiple of 64,
                                  E > 256, r > 128, P_tot = T*k + n_shared*T >= 2^31,
                                  or any buffer the kernels address with 32-bit byte
                                  offsets reaching 2^31 bytes: [T, d] and [P_tot, d],
                                  [P_tot, 2n], [P_tot, n] 16-bit activations, one expert's
                                  [2n, d] weight, the [P_tot, r] rank-r rows and their
                                  fp32 partial sums, the [P_tot, n/64] router partials */
  MOE_ERROR_WORKSPACE = 3,     /* a workspace / saved buffer smaller than its size query */
  MOE_ERROR_LAUNCH = 4         /* the HIP runtime reported an error when enqueueing */
} moe_status;

/* Layer shape.  T tokens, hidden size d, expert intermediate size n, E routed
 * experts, top-k, LoRA rank r, n_shared shared experts (0 or 1, stacked after
 * the routed ones), LoRA scale s applied to the low-rank term, and the element
 * type of every 16-bit tensor below (x, y, dy, dx, the weights and LoRA
 * factors, and the saved activations): MOE_BF16 (0) or MOE_F16 (1, the
 * faster-MoE page's fp16 variant of the grouped GEMM for GPUs without bf16).
 * Logits, routing weights, accumulation and the LoRA gradients stay fp32.
 * Derived: P = T*k routed pairs; P_tot = P + n_shared*T rows of every grouped
 * GEMM; E_tot = E + n_shared stacked experts. */
#define MOE_BF16 0
#define MOE_F16 1
typedef struct {
  int64_t T;
  int32_t d, n, E, k, r, n_shared;
  float lora_scale;
  int32_t dtype;
} moe_dims;

/* Routing tensors, written by moe_route and read by forward/backward.
 *   topk_ids    int32 [T, k]  expert ids per token, largest logit first
 *   topk_w      fp32  [T, k]  softmax of the selected logits
 *   counts      int32 [E]     rows per expert (one bincount)
 *   offsets     int32 [E+1]   exclusive prefix sum of counts, offsets[E] = P
 *   sorted_pair int32 [P]     flat pair index t*k + j at sorted position p;
 *                             expert e owns positions [offsets[e], offsets[e+1]),
 *                             ascending in t (stable)
 *   pair_pos    int32 [P]     inverse permutation: sorted position of pair i
 *   row_token   int32 [P_tot] gather table of the sorted rows: the token of
 *                             row p (sorted_pair[p] / k), and t for the shared
 *                             expert's row P + t
 *   row_weight  fp32  [P_tot] routing weight of row p (topk_w of sorted_pair[p]),
 *                             1 for the shared expert's rows */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int32_t* row_token;
  float* row_weight;
} moe_routing;

/* Frozen base weights and LoRA factors, bf16, stacked over E_tot experts:
 *   w_gate_up [E_tot, 2n, d]  rows [0,n) = gate, rows [n,2n) = up
 *   w_down    [E_tot, d, n]
 *   a_gate_up [E_tot, d, r]   b_gate_up [E_tot, r, 2n]
 *   a_down    [E_tot, n, r]   b_down    [E_tot, r, d]
 * The effective weights are W_gu + s (A_gu B_gu)^T and W_dn + s (A_dn B_dn)^T,
 * but the library only ever forms (X A) B. */
typedef struct {
  const moe_bf16* w_gate_up;
  const moe_bf16* w_down;
  const moe_bf16* a_gate_up;
  const moe_bf16* b_gate_up;
  const moe_bf16* a_down;
  const moe_bf16* b_down;
} moe_weights;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status s);

/* Size queries.  Each returns 0 if dims is NULL or invalid. */
size_t moe_route_workspace_bytes(const moe_dims* dims);
/* Buffer forward fills and backward reads: G [P_tot,2n], H [P_tot,n],
 * s X A_gu and s H A_dn [P_tot, r] (16-bit). */
size_t moe_forward_saved_bytes(const moe_dims* dims);
/* Scratch for one forward or backward call (contents are not preserved). */
size_t moe_workspace_bytes(const moe_dims* dims);

/* Top-k softmax routing and the one-pass grouping (article section
 * "Optimisation 3: MoE routing grouped once"), including the gather table of
 * the sorted rows (with the shared expert's rows when dims->n_shared is 1).
 *   logits  fp32 [T, E] router logits
 *   out     routing buffers to fill (all eight pointers required)
 *   ws      device scratch of at least moe_route_workspace_bytes(dims) */
moe_status moe_route(const moe_dims* dims, const float* logits, const moe_routing* out,
                     void* ws, size_t ws_bytes, void* stream);

/* moe_route for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace: its scratch is a MOE_ROUTE_NOALLOC_SCRATCH_BYTES (4 MiB)
 * array of device memory that the library holds on each GPU it runs on until
 * the process ends, looked up once per device on the first call.  The call
 * allocates nothing, on the device or on the host.
 *   Limit: moe_route_workspace_bytes(dims) <= 4 MiB (about T*k <= 983,040 at
 *   E = 256); a larger shape returns MOE_ERROR_UNSUPPORTED with nothing
 *   enqueued.  MOE_ERROR_LAUNCH if the device copy of the array cannot be
 *   found.  Otherwise arguments, outputs and errors are those of moe_route.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (on different streams, or from different threads) race and must be
 *   ordered by the caller. */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_route_noalloc(const moe_dims* dims, const float* logits, const moe_routing* out,
                             void* stream);

/* Forward of the expert layer with split LoRA (faster-MoE page, "What is
 * torch._grouped_mm?" and "Faster LoRA MoE training"):
 *   for each routed pair (t, j) with expert e = topk_ids[t,j]:
 *     G = x_t W_gu[e]^T + s (x_t A_gu[e]) B_gu[e];  gate, up = G[:n], G[n:]
 *     H = silu(gate) * up
 *     O = H W_dn[e]^T + s (H A_dn[e]) B_dn[e]
 *   y_t = sum_j topk_w[t,j] O(t,j)  (+ O of the shared expert, weight 1)
 *   x     bf16 [T, d] hidden states
 *   y     bf16 [T, d] output
 *   saved buffer of moe_forward_saved_bytes(dims), kept unchanged for backward
 *   ws    scratch of moe_workspace_bytes(dims) */
moe_status moe_lora_forward(const moe_dims* dims, const moe_bf16* x, const moe_routing* routing,
                            const moe_weights* weights, moe_bf16* y, void* saved,
                            size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);

/* Backward for dX and the LoRA factors (the pages freeze the router and the
 * base weights; no gradient is produced for the base weights):
 *   dy   bf16 [T, d] upstream gradient;  x as given to forward
 *   saved  the buffer forward filled, with the same dims/routing/weights
 *   dx   bf16 [T, d]
 *   da_gate_up fp32 [E_tot, d, r]   db_gate_up fp32 [E_tot, r, 2n]
 *   da_down    fp32 [E_tot, n, r]   db_down    fp32 [E_tot, r, d]
 *   d_topk_w   fp32 [T, k] or NULL: gradient w.r.t. the routing weights,
 *              d w[t,j] = <dY[t], O(t,j)> (Y is linear in w; O is the pair's
 *              down output before the weight)
 *   d_logits   fp32 [T, E] or NULL: gradient w.r.t. the router logits through
 *              the softmax over the k selected logits,
 *              d logit[t, id_j] = w_j (d w_j - sum_i w_i d w_i), 0 for the
 *              experts not selected (the selection is locally constant); the
 *              shared expert's weight is the constant 1 and takes none.
 *              For models that train the router (the pages freeze it).
 *              They come from the streamed dh kernel, which this call then
 *              uses whatever engine is set for the shape.
 *   ws   scratch of moe_workspace_bytes(dims) */
moe_status moe_lora_backward(const moe_dims* dims, const moe_bf16* dy, const moe_bf16* x,
                             const moe_routing* routing, const moe_weights* weights,
                             const void* saved, size_t saved_bytes, moe_bf16* dx,
                             float* da_gate_up, float* db_gate_up, float* da_down,
                             float* db_down, float* d_topk_w, float* d_logits, void* ws,
                             size_t ws_bytes, void* stream);

/* The merged-weight path the pages compare split LoRA against (faster-MoE
 * page, "Faster LoRA MoE training": PEFT merges the adapter into the base
 * weight; "MoE LoRA changes things": split LoRA wins until the token count s
 * passes a crossover, E m n / (k (m + n)) (1 + 1/(2r)) by the page's FLOP
 * count).  Provided to measure that crossover on this GPU; the layer itself
 * never merges.
 * moe_merge_lora forms, for every one of the E_tot experts,
 *   w_gate_up_merged[e] = W_gu[e] + s (A_gu[e] B_gu[e])^T    [E_tot, 2n, d]
 *   w_down_merged[e]    = W_dn[e] + s (A_dn[e] B_dn[e])^T    [E_tot, d, n]
 * with fp32 accumulation, rounded once to the element type.  The outputs are
 * caller-owned device buffers of the weights' shapes; no workspace.
 * moe_forward_merged is moe_lora_forward on such merged weights with the
 * low-rank pass off (no X A / H A products): Y = combine(silu(gate) * up of
 * X W'_gu^T, then H W'_dn^T).  saved and ws as for moe_lora_forward (the
 * rank-r parts of saved are left unwritten, so it does not feed
 * moe_lora_backward).  Its Y equals moe_lora_forward's to the layer's
 * tolerance. */
moe_status moe_merge_lora(const moe_dims* dims, const moe_weights* weights,
                          moe_bf16* w_gate_up_merged, moe_bf16* w_down_merged, void* stream);
moe_status moe_forward_merged(const moe_dims* dims, const moe_bf16* x, const moe_routing* routing,
                              const moe_bf16* w_gate_up_merged, const moe_bf16* w_down_merged,
                              moe_bf16* y, void* saved, size_t saved_bytes, void* ws,
                              size_t ws_bytes, void* stream);

/* Engines and tile configurations.  Every grouped product has two
 * implementations: register-path kernels (global -> registers -> LDS) and
 * streamed ones (global -> LDS by buffer_load ... lds through a ring, one
 * persistent workgroup per CU), the streamed ones in four tile
 * configurations.  What runs is chosen per layer shape (d, n, E, k, r,
 * n_shared; not T), process-wide (and per element type), by these bits:
 *   MOE_ENGINE_GATE_UP, _DOWN, _DH, _DX (bits 0-3)  set = streamed grouped
 *     GEMM for that product;
 *   MOE_ENGINE_RANK (bit 4)  set = streamed rank-r pre-passes and LoRA
 *     gradients (r <= 64; above that both settings use the register path);
 *   MOE_TILE256(p) (bits 5-8)  set = 256-row tiles for product p (0 gate_up,
 *     1 down, 2 dh, 3 dx), else 320 rows;
 *   MOE_STAGE32(p) (bits 9-12)  set = ring stages of 32 k for product p, else
 *     64 k (tile bits matter only when the product is streamed);
 *   MOE_SPLITK_1024, MOE_SPLITK_4096 (bits 13-14, one value)  rows per split-K
 *     chunk of the LoRA gradients, else 2048.
 * Without a recorded choice a shape uses MOE_ENGINE_DEFAULT (everything
 * streamed, 320-row tiles, 64-k stages, 2048-row chunks).
 * moe_set_engines records a choice (MOE_ERROR_INVALID_VALUE for unknown bits
 * or split-K field 3); moe_get_engines returns the choice in force.  Results
 * agree between settings to the layer's tolerance, not bitwise.
 * moe_autotune is the one-time start-up autotune of the faster-MoE page's
 * kernels ("Unsloth MoE Triton kernels"), cached per shape: it runs route +
 * forward + backward on the given inputs under seven settings (streamed with
 * each of the four tile configurations, register path, streamed with
 * 1024- and 4096-row split-K chunks), twice in alternation (one warm-up and
 * three timed steps each time, every kernel timed with events), and picks per
 * product the setting with the lowest time -- another setting than the
 * default only when it is more than 1 % faster -- then records and returns
 * the combined choice.  Unlike every other entry point it waits for the GPU;
 * it uses (and leaves switched off) the calling thread's kernel-timing
 * recorder, so autotunes on different threads do not interfere.  scratch:
 * device memory of at least moe_autotune_scratch_bytes(dims), 256-byte
 * aligned, for all the routing, saved, workspace and output buffers of those
 * steps; its contents are undefined afterwards.  logits, x, dy, weights as
 * for the other calls. */
#define MOE_ENGINE_GATE_UP 1u
#define MOE_ENGINE_DOWN 2u
#define MOE_ENGINE_DH 4u
#define MOE_ENGINE_DX 8u
#define MOE_ENGINE_RANK 16u
#define MOE_ENGINE_DEFAULT 31u
#define MOE_TILE256(p) (1u << (5 + (p)))
#define MOE_STAGE32(p) (1u << (9 + (p)))
#define MOE_SPLITK_1024 (1u << 13)
#define MOE_SPLITK_4096 (2u << 13)
moe_status moe_set_engines(const moe_dims* dims, unsigned engines);
unsigned moe_get_engines(const moe_dims* dims);
size_t moe_autotune_scratch_bytes(const moe_dims* dims);
moe_status moe_autotune(const moe_dims* dims, const float* logits, const moe_bf16* x,
                        const moe_bf16* dy, const moe_weights* weights, void* scratch,
                        size_t scratch_bytes, void* stream, unsigned* engines_out);

/* Kernel timing, for measurement tools (not part of the layer's math).
 * moe_timing_enable(1) starts recording: every kernel the library enqueues
 * afterwards from the calling host thread is bracketed by two HIP events on
 * its stream (a few microseconds of extra gaps per kernel).
 * moe_timing_enable(0) stops recording.  Both clear previous records.  Each
 * host thread has its own recorder; a thread's first enable creates its
 * event pool (host call, no device memory).  Returns MOE_ERROR_LAUNCH if events cannot be created.
 * moe_timing_report waits for the recorded events, then writes up to
 * max_entries distinct kernel names (each NUL-terminated in a name_len-byte
 * slot of `names`), the summed milliseconds and the launch count per name,
 * clears the records and returns the number of entries (-1 on a HIP error).
 * All buffers are host memory owned by the caller. */
moe_status moe_timing_enable(int on);
int moe_timing_report(char* names, int name_len, float* total_ms, int* launches, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LORA_H */
