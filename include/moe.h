/*
 * moe.h -- C ABI of libmoe, an MI355X (gfx950) implementation of the
 * Flash-MoE expert layer for decode.
 *
 * The layer (per token, per layer), as the pages describe it:
 *   h   = RMSNorm(x)                        two passes: sum of squares, then scaling
 *         ("48GB内存运行397B模型：Flash-Moe的极端量化与SSD流式加载实践", section
 *          "Metal GPU管线：手写Kernel与FMA优化", RMS归一化)
 *   z   = W_router h  over the experts; softmax; the top-K experts
 *         (juejin post, "3. 流水线设计——严格串行反而更快": GPU routing, then top-K;
 *          flash-moe README translation, "Pipeline mỗi lớp": softmax + topK routing)
 *   for each selected expert and the shared expert:
 *         a = silu(W_gate h) * (W_up h),  y = W_down a,
 *         every weight w = code * scale + bias, computed as fma(code, scale*x, bias*x)
 *         ("48GB内存运行397B模型", sections "量化策略" and "Metal GPU管线": 4-bit dequant
 *          mat-vec with the FMA rewrite; Fused SwiGLU)
 *   out = x + sum_k w_k y_k + sigmoid(g_s) y_shared,  g_s = w_sg . h
 *         (same page, "Metal GPU管线": fused MoE combine + residual + sigmoid gate)
 * 512 experts per layer, K = 4 active plus one shared expert, hidden 4096
 * (same page, section "MoE稀疏架构").  The K selected probabilities are
 * renormalised to sum to one.
 *
 * Conventions for every entry point:
 *  - Pointers named as device memory are HIP device pointers owned by the
 *    caller; the library never allocates or frees, and never synchronises
 *    except in moe_tier_layer_forward.  It keeps no state between calls apart
 *    from the workspace and the tier state the caller passes, and the one
 *    fixed device array per GPU that moe_layer_forward_noalloc works in.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work; faults surface at the caller's next synchronisation.
 *  - Arguments are checked on the host before anything is enqueued; a negative
 *    moe_status_t is returned and nothing is launched.  The library never
 *    aborts and never throws across this boundary.  A failed launch returns
 *    MOE_ERR_HIP.
 *  - Activations are fp32, [n_tokens][hidden] row-major.  bf16 tensors are
 *    passed as their 16-bit patterns (uint16_t).
 *  - Inputs are assumed finite; a NaN in x propagates to the outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* NULL pointer, out-of-range size, bad dims   */
    MOE_ERR_UNSUPPORTED = -2, /* valid in principle, not built (shape, bits) */
    MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes   */
    MOE_ERR_ALIGNMENT = -4,   /* pointer not aligned as documented            */
    MOE_ERR_HIP = -5          /* a HIP launch or copy failed                  */
} moe_status_t;

/*
 * Shape of one layer.
 *   hidden      H, the token width (4096 in the pages' model)
 *   ffn         F, the expert FFN width (1024)
 *   n_experts   E, routed experts per layer (512), 1 <= E <= 1024
 *   top_k       K, experts selected per token (4; the model's native 10), 1 <= K <= min(E, 16)
 *   bits        2 or 4: width of a quantisation code
 *   group_size  64: one bf16 scale and one bf16 bias per 64 consecutive
 *               entries along a row's reduction axis
 *   rms_eps     epsilon of the RMSNorm (1e-6)
 * Built shapes: H and F powers of two in [128, 4096].  Other shapes return
 * MOE_ERR_UNSUPPORTED.
 */
typedef struct moe_dims {
    int32_t hidden;
    int32_t ffn;
    int32_t n_experts;
    int32_t top_k;
    int32_t bits;
    int32_t group_size;
    float rms_eps;
} moe_dims_t;

/*
 * Weights of one layer (all device memory, 256-byte aligned).
 *   norm_weight    bf16 [H]          RMSNorm weight gamma
 *   router_weight  bf16 [E][H]       router matrix, row e gives logit e
 *   shared_gate    bf16 [H]          sigmoid gate vector of the shared expert
 *   experts        E packed experts, expert e at byte offset e * moe_expert_bytes()
 *   shared_expert  one packed expert (the always-active shared expert)
 * Packed experts are produced by moe_pack_expert or moe_generate_layer; their
 * byte layout is private to the library.
 */
typedef struct moe_layer {
    const uint16_t *norm_weight;
    const uint16_t *router_weight;
    const uint16_t *shared_gate;
    const void *experts;
    const void *shared_expert;
} moe_layer_t;

/* Returns MOE_OK if the library supports `dims`, else the status it would return. */
int moe_check_dims(const moe_dims_t *dims);

/*
 * Bytes of one packed expert: codes of gate [F][H], up [F][H] and down [H][F]
 * (bits/8 bytes per weight) plus a 4-byte bf16 scale+bias pair per group of 64:
 *   3*H*F*bits/8 + 3*(H*F/64)*4.
 * 7,077,888 B (6.75 MiB) at H=4096, F=1024, 4-bit -- the pages' "about 6.75MB per
 * expert, 27MB for K=4" ("48GB内存运行397B模型", section "MoE稀疏架构").
 * Returns 0 for unsupported dims.
 */
size_t moe_expert_bytes(const moe_dims_t *dims);

/*
 * Bytes of workspace a forward call with up to n_tokens tokens needs (the same
 * for moe_layer_forward and moe_stack_forward).  Returns 0 for unsupported dims
 * or n_tokens < 1.
 */
size_t moe_workspace_bytes(const moe_dims_t *dims, int32_t n_tokens);

/*
 * Zero the workspace's control block: its first 8 KiB (device memory, 256-B
 * aligned, workspace_bytes >= 8192), which hold the counters through which
 * the batched path's blocks claim their work.  Needed once, before the first
 * forward call on a new workspace; every forward call that completes leaves
 * the control block zero again.  Enqueued on `stream`.
 */
int moe_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * Pack one expert from canonical tensors (all device memory):
 *   codes[m]  uint8 [rows][cols], one code per byte, each < 2^bits
 *   scale[m]  bf16  [rows][cols/64]
 *   bias[m]   bf16  [rows][cols/64]
 * for m = 0 gate [F][H], 1 up [F][H], 2 down [H][F] (row = output index,
 * column = reduction index).  dst: moe_expert_bytes() bytes of device memory,
 * 256-byte aligned.  Codes >= 2^bits are masked to their low `bits` bits.
 */
int moe_pack_expert(const moe_dims_t *dims, const uint8_t *const codes[3],
                    const uint16_t *const scale[3], const uint16_t *const bias[3], void *dst,
                    void *stream);

/*
 * Generate the packed synthetic experts of one layer on the device from a
 * seed: codes uniform in [0, 2^bits), scales uniform in [0.005, 0.02), biases
 * uniform in [-0.1, 0), all drawn from counter-based SplitMix64 streams keyed by
 * (seed, layer, expert, matrix, kind).  The result equals moe_pack_expert of the
 * canonical tensors that the same streams define (the stream definition is
 * stated in the generator's source, moe_pack.hip).
 *   experts        E packed experts (NULL: skip), shared_expert: 1 (NULL: skip).
 */
int moe_generate_layer(const moe_dims_t *dims, uint64_t seed, uint32_t layer, void *experts,
                       void *shared_expert, void *stream);

/*
 * One MoE layer for n_tokens tokens.  Batches of fewer than 72 assignments
 * (n_tokens * top_k < 72) run three kernels per layer, one row of blocks per
 * token; batches of 72 to 4096 assignments are grouped by expert so that every
 * selected expert's weights are read once for all of its tokens (larger ones run
 * the per-token kernels).  Both give the same results up to fp32 rounding order.
 *   x          fp32 [n_tokens][H] device, 16-B aligned (may equal y: in place)
 *   y          fp32 [n_tokens][H] device, 16-B aligned: x + routed combine + gated shared
 *   route_idx  int32 [n_tokens][K] device or NULL: selected experts, ordered by
 *              (logit descending, expert index ascending)
 *   route_w    fp32 [n_tokens][K] device or NULL: renormalised weights (sum 1)
 *   workspace  device, 256-B aligned, >= moe_workspace_bytes(dims, n_tokens),
 *              control block zeroed once by moe_workspace_init.
 * Calls that share one workspace must be ordered (same stream); calls on
 * different streams need different workspaces.
 */
int moe_layer_forward(const moe_dims_t *dims, const moe_layer_t *layer, const float *x, float *y,
                      int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes of device memory inside the library, one
 * per GPU, held from the library's load until the process ends; its address on
 * the current device is looked up on the first call there.  The call
 * allocates nothing and calls no allocating routine.
 *  - `stream` must belong to the current device.
 *  - Every call on one GPU uses that GPU's one array: calls that may overlap
 *    on one GPU (different streams, or different threads without ordering)
 *    race and give wrong results.  Stream-ordered calls are safe; each call
 *    starts from what it needs to be zero (the grouped path's control block
 *    is cleared by a kernel first).
 *  - A batch whose workspace, moe_workspace_bytes(dims, n_tokens), exceeds
 *    MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE before anything is
 *    enqueued.  16 MiB holds every single-token call of the built shapes and
 *    up to 32 tokens with top-10 at hidden 4096, FFN 1024, 512 experts.
 * Other arguments, checks and results as for moe_layer_forward (bit for bit).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
int moe_layer_forward_noalloc(const moe_dims_t *dims, const moe_layer_t *layer, const float *x, float *y,
                              int32_t n_tokens, int32_t *route_idx, float *route_w, void *stream);

/*
 * Enqueue one stage of the layer, for profiling or for interleaving other work
 * between stages.  The stages are those of the path moe_layer_forward takes for
 * n_tokens (moe_forward_stage_count gives their number); enqueued in order
 * 0, 1, ... with identical arguments (same workspace, stream order) they
 * produce exactly what moe_layer_forward produces.
 * Per-token path (3 stages): 0 RMSNorm, router GEMV and
 * shared-gate logit; 1 softmax/top-K/renormalise and the fused gate+up dequant
 * GEMV with SwiGLU for the selected and the shared experts; 2 down projection
 * with the weighted combine, sigmoid-gated shared expert and residual.
 * Grouped path (7 stages): 0 RMSNorm of every token; 1 router GEMM and
 * shared-gate logits; 2 softmax/top-K/renormalise of every token and grouping
 * of the assignments by expert; 3 gate+up with SwiGLU per touched expert over
 * its tokens (and the shared expert over all tokens); 4 limb encoding of the
 * activations; 5 down projection per touched expert; 6 weighted combine,
 * sigmoid-gated shared expert and residual.
 * Arguments as for moe_layer_forward; a stage outside 0 .. count-1 is
 * MOE_ERR_INVALID_ARG.
 */
int moe_layer_forward_stage(const moe_dims_t *dims, const moe_layer_t *layer, const float *x, float *y,
                            int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                            size_t workspace_bytes, int32_t stage, void *stream);

/* Number of stages of moe_layer_forward_stage for this batch size (3 or 7), or
 * a negative status for invalid dims or n_tokens outside 1 .. 65535. */
int moe_forward_stage_count(const moe_dims_t *dims, int32_t n_tokens);

/*
 * n_layers layers chained: x_{l+1} = layer_l(x_l), x_0 = x, y = x_{n_layers}
 * (no final norm), the per-layer pipeline repeated over the model's 60 layers
 * ("48GB内存运行397B模型", section "MoE稀疏架构": 60 layers, each with 512 experts
 * and top-K routing; flash-moe README translation, "Pipeline mỗi lớp": a layer's
 * expert command buffer runs the experts, the combine and the norm, and the
 * next layer starts from its output).  `layers` is a HOST array of n_layers
 * layer descriptors.  route_idx / route_w (device or NULL):
 * [n_layers][n_tokens][K].
 * Every layer is enqueued back to back on `stream`; nothing waits on the host.
 * The result equals n_layers chained moe_layer_forward calls bit for bit: the
 * next layer's RMSNorm stays in its router kernel, which reads all of x_{l+1}
 * for the router product anyway.
 */
int moe_stack_forward(const moe_dims_t *dims, const moe_layer_t *layers, int32_t n_layers,
                      const float *x, float *y, int32_t n_tokens, int32_t *route_idx,
                      float *route_w, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Tiered expert residency.  The pages keep every expert on SSD and, once a
 * layer's routing is known, read the K selected experts in parallel, leaving
 * the operating system's LRU page cache to keep recently used experts in
 * memory ("48GB内存运行397B模型", section "SSD流式加载：绕过统一内存瓶颈": 2.41 ms
 * of a 4.28 ms layer is that read, about 71% of reads hit the cache; the
 * compute and the reads run one after the other, never overlapped).  Here the
 * backing store is host memory, HBM holds a cache of n_slots experts keyed by
 * (layer, expert) with least-recently-used replacement, and a miss is a copy
 * of the whole packed expert over the host link.  The dense weights
 * (norm, router, shared gate) and the shared expert stay in device memory.
 *
 * A call runs the per-token kernels only (n_tokens up to max_tokens):
 *   1. RMSNorm + router GEMV, then softmax/top-K/renormalise on the device,
 *      which also writes the selected indices into the state, each as one
 *      8-byte entry tagged with the call;
 *   2. the calling thread WAITS for them, spinning until every entry holds
 *      this call's tag (the one entry point that synchronises; an entry that
 *      does not land within ~1e8 polls, as after a failed launch, makes it
 *      synchronise `stream` and report the error);
 *   3. cache lookups in token order, then rank order; each miss takes the
 *      least recently used slot; one kernel then copies the missing experts
 *      into their slots, reading the host memory directly (a host store that
 *      is not pinned, mapped memory is copied by DMA instead);
 *   4. gate/up + SwiGLU and down + combine read the selected experts from
 *      their slots, whose numbers travel in the kernel arguments (hence at
 *      most 64 assignments, max_tokens * top_k <= 64, per call).
 * y, route_idx and route_w are bit for bit those of moe_layer_forward's
 * per-token kernels with every expert resident.
 *
 * State: the cache's bookkeeping lives in host memory the caller allocates
 * with hipHostMalloc (pinned and mapped: the routing kernel writes the
 * indices into it), moe_tier_state_bytes() bytes, 8-byte aligned; the slots
 * live in device memory of moe_tier_device_bytes() bytes, 256-byte aligned.  Both
 * belong to the state until the caller frees them; the library keeps no
 * pointer elsewhere.  Calls on one state must come from one host thread at a
 * time and use one stream.
 */
typedef struct moe_tier_stats {
    uint64_t calls;        /* moe_tier_layer_forward calls that completed */
    uint64_t lookups;      /* (token, rank) assignments looked up */
    uint64_t hits;         /* assignments whose expert was already in a slot */
    uint64_t misses;       /* assignments whose expert was copied in */
    uint64_t bytes_copied; /* host-to-device bytes of those copies */
} moe_tier_stats_t;

/* Host bytes of the state for n_layers layers, n_slots device slots and calls
 * of up to max_tokens tokens; 0 for invalid or unsupported arguments
 * (n_layers >= 1, max_tokens >= 1 with max_tokens * top_k <= 64,
 * n_slots >= max_tokens * top_k so that one call's experts always fit,
 * n_layers * n_experts < 2^31). */
size_t moe_tier_state_bytes(const moe_dims_t *dims, int32_t n_layers, int32_t n_slots, int32_t max_tokens);

/* Device bytes: n_slots packed experts, n_slots * moe_expert_bytes(); 0 for
 * invalid or unsupported arguments. */
size_t moe_tier_device_bytes(const moe_dims_t *dims, int32_t n_slots, int32_t max_tokens);

/*
 * Initialise a state: every slot empty, statistics zero.  `state` (pinned
 * host, state_bytes) and `device` (device, device_bytes) as sized above.
 * Enqueues nothing; makes no HIP call.  max_tokens * top_k > 64 is
 * MOE_ERR_UNSUPPORTED.
 */
int moe_tier_init(const moe_dims_t *dims, int32_t n_layers, int32_t n_slots, int32_t max_tokens,
                  void *state, size_t state_bytes, void *device, size_t device_bytes);

/*
 * One layer through the cache.  `layer` as for moe_layer_forward except that
 * layer->experts is HOST memory, 256-byte aligned, holding the layer's
 * n_experts packed experts, expert e at byte offset e * moe_expert_bytes().
 * Pinned memory (hipHostMalloc) is read directly by the copy kernel; other
 * host memory is copied by DMA, more slowly.  It must stay valid and unchanged
 * until the work this call enqueues on `stream` has completed;
 * layer_index (0 .. n_layers-1) names the layer in the cache's keys, so each
 * index must always come with the same experts.  Other arguments as for
 * moe_layer_forward, n_tokens <= max_tokens.  Returns after the copies and the
 * expert kernels are enqueued (the routing has completed).  A state whose
 * memory is not pinned host memory is MOE_ERR_INVALID_ARG.  On MOE_ERR_HIP
 * the state's slots may be stale: re-initialise it.
 */
int moe_tier_layer_forward(void *state, int32_t layer_index, const moe_layer_t *layer, const float *x,
                           float *y, int32_t n_tokens, int32_t *route_idx, float *route_w,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * n_layers layers through the cache, chained as in moe_stack_forward: layer l
 * uses layers[l] (a HOST array; experts in host memory as above) and cache
 * layer index l, for l = 0 .. n_layers-1 (n_layers at most the state's).
 * route_idx / route_w (device or NULL): [n_layers][n_tokens][K].  Waits once
 * per layer for its routing, as moe_tier_layer_forward does; stops at the
 * first error and returns it.
 */
int moe_tier_stack_forward(void *state, const moe_layer_t *layers, int32_t n_layers, const float *x, float *y,
                           int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Statistics since moe_tier_init. */
int moe_tier_get_stats(const void *state, moe_tier_stats_t *out);

/* *slot = the slot holding (layer_index, expert), or -1 when it is not cached. */
int moe_tier_lookup(const void *state, int32_t layer_index, int32_t expert, int32_t *slot);

/* Static text for a status code. */
const char *moe_status_string(int status);

/* Text of the HIP error behind the calling thread's last MOE_ERR_HIP (static storage). */
const char *moe_last_error(void);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
