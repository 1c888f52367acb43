/*
 * moe.h -- C ABI of libmoe: the per-token sparse MoE block of a
 * "streaming experts" decode engine, on AMD Instinct MI355X (gfx950).
 *
 * The calls follow the pages' statement of the per-layer problem (the
 * Flash-MoE engine as described on toolarium.ru and hakusoku.com):
 *   route    -- the router picks K of E experts per token and layer
 *               (toolarium.ru, "Mixture of Experts и почему SSD достаточно";
 *               softmax/topK step in hakusoku.com, "パイプライン概要");
 *   fetch    -- the K selected experts' weights are brought to the GPU
 *               (toolarium.ru, "Flash-MoE: чистый C, Metal и никакого
 *               Python": parallel reads of ~6.75 MB per expert);
 *   forward  -- dequantised expert FFNs (gate, up, SwiGLU, down) for the
 *               selected experts plus the shared expert, weighted combine,
 *               residual add and RMSNorm in one pass whose output feeds the
 *               next layer (hakusoku.com, "主要技術"; toolarium.ru,
 *               "Оптимизации, которые сработали").
 *
 * Conventions (all calls):
 *  - Status: MOE_OK (0) or a negative MOE_E* code.  On an error nothing has
 *    been enqueued.  moe_last_error() gives a message for the calling thread.
 *  - Memory: every buffer belongs to the caller.  The library allocates and
 *    frees nothing, except the pinned host memory that moe_host_alloc and
 *    moe_host_free exist for.  Pointers are device pointers unless marked
 *    "host".
 *  - Asynchrony: calls enqueue work on the given HIP stream (passed as
 *    void*, a hipStream_t; NULL = the legacy default stream) and return;
 *    results are valid once the stream has been synchronised.  No call
 *    synchronises the device, except where stated.
 *  - Dtypes: activations, router weights, gamma and routing weights are fp32;
 *    expert weights are packed unsigned codes with bf16 group scale/bias
 *    inside the canonical blob (below); indices are int32.
 *  - Validation happens on the host before anything is enqueued: non-NULL
 *    pointers, 16-byte aligned for activations, weights and blobs and 4-byte
 *    aligned for topk_idx / topk_w / logits, a 256-byte aligned workspace,
 *    bits in {2,4}, group == 64, hidden and
 *    inter multiples of 64 (hidden <= 8192, inter <= 4096), 1 <= top_k <=
 *    min(n_experts, 8), n_experts <= 4096, 1 <= n_tokens <= 64, and
 *    blob_bytes == moe_blob_bytes(...).
 *  - Device-side faults: an expert index outside [0, n_experts) met on the
 *    device sets bit MOE_DEVERR_EXPERT_RANGE in workspace word 0 and that
 *    expert's contribution is skipped; a wait of a fused layer step for
 *    data from other workgroups is bounded (2^16 polls with a short sleep
 *    between them, some tens of milliseconds): when it runs out,
 *    MOE_DEVERR_BARRIER_TIMEOUT is set and the kernel runs to its end (its
 *    results are then invalid).  Word 0 is only ever OR-ed into.
 *  - Thread safety: calls are reentrant.  Two calls that share a workspace
 *    must be ordered on one stream (they reuse its scratch and counters).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)        /* bad shape, pointer or alignment; nothing enqueued  */
#define MOE_EUNSUPPORTED (-2)  /* valid request that this build does not implement    */
#define MOE_EHIP (-3)          /* HIP runtime error; moe_last_error() has the text    */
#define MOE_ESTATE (-4)        /* streamer misuse: bad slot, layer or id, no arena    */

#define MOE_DEVERR_EXPERT_RANGE 1u   /* an expert index outside [0, n_experts) */
#define MOE_DEVERR_BARRIER_TIMEOUT 2u /* a grid-wide wait of a fused layer step timed out */
#define MOE_DEVERR_WORKSPACE 4u       /* a fused layer step met a workspace last used with another grid */

/*
 * Canonical expert blob (one contiguous byte range per expert; the unit the
 * pages stream, about 6.75 MB per expert at 4-bit, toolarium.ru "Flash-MoE:
 * чистый C, Metal и никакого Python"):
 *
 *   [gate.q | up.q | down.q | gate.sb | up.sb | down.sb]
 *
 * gate and up: [inter rows][hidden cols]; down: [hidden rows][inter cols];
 * all row-major.  q regions: element c of a row is held at bit offset c*bits
 * of that row, in little-endian 32-bit words, lowest bits first; codes are
 * unsigned in [0, 2^bits).  sb regions: one 32-bit word per group of 64
 * consecutive columns of a row: bf16 scale in bits 0..15, bf16 bias in bits
 * 16..31.  The dequantised weight is w = q*scale + bias (toolarium.ru,
 * "Оптимизации, которые сработали": nibble*scale + bias).
 *
 * Returns 3*hidden*inter*bits/8 + 3*hidden*inter/group*4, or 0 for invalid
 * arguments.  hidden=4096, inter=1024, bits=4, group=64 gives 7,077,888 B.
 */
size_t moe_blob_bytes(int32_t hidden, int32_t inter, int32_t bits, int32_t group);

/* One MoE layer.  Plain data, owned by the caller. */
typedef struct moe_layer_desc {
    int32_t hidden;        /* D */
    int32_t n_experts;     /* E routed experts */
    int32_t top_k;         /* K selected per token */
    int32_t inter;         /* I, expert intermediate size */
    int32_t n_shared;      /* 0 or 1 always-active shared expert (hakusoku.com, "モデルアーキテクチャ") */
    int32_t bits;          /* 4 or 2 */
    int32_t group;         /* 64 */
    float rms_eps;         /* RMSNorm epsilon, inside the square root */
    const float *router_w; /* [E][D] fp32 row-major */
    const float *gamma;    /* [D] fp32 RMSNorm weight */
    /* Resident mode: E canonical blobs, blob_bytes apart, expert e at
     * experts + e*blob_bytes, and the shared blob at `shared`.  Both may
     * also point into pinned host memory from moe_host_alloc (mapped into
     * the device's address space): the kernels then read the selected
     * experts over the host link themselves (zero-copy streaming, one
     * launch per token with moe_stack_step, no copies, no host wait).
     * Streamed mode: experts == NULL and slab != NULL: slab holds top_k+1
     * blobs, blob_bytes apart: slot k = the token's k-th selected expert,
     * slot top_k = the shared expert (streamed mode needs n_tokens == 1).
     * Address-table mode: experts == NULL, slab == NULL and expert_addr !=
     * NULL: expert_addr is a device array of n_experts blob addresses, each
     * 16-byte aligned, in HBM or in pinned host memory from moe_host_alloc
     * (per-expert residency: frequently routed experts in HBM, the rest
     * read over the host link, in one launch); the shared blob is at
     * `shared`.  Only the single-token fused stack takes it (moe_layer_step
     * with n_tokens == 1 and moe_stack_step on a shape moe_layer_plan reports
     * as fused); other uses return MOE_EUNSUPPORTED.  The table is read on
     * the device by the launch: change it only between launches. */
    const uint8_t *experts;
    const uint8_t *shared;
    const uint8_t *slab;
    uint64_t blob_bytes;   /* must equal moe_blob_bytes(hidden, inter, bits, group) */
    const uint64_t *expert_addr;
} moe_layer_desc;

/* Workspace bytes that moe_route / moe_expert_forward / moe_layer_step need
 * for this layer shape and token count (0 for an invalid descriptor).
 * The caller zero-fills a workspace once after allocating it; the library
 * keeps its counters consistent from call to call.  A workspace serves one
 * layer shape (hidden, n_experts, inter, bits, top_k + n_shared) on one
 * device, with any token count up to the one it was sized for: the
 * grid-barrier state of the fused layer step belongs to that shape's grid,
 * and a fused step on a workspace last used with another grid sets
 * MOE_DEVERR_WORKSPACE and does nothing. */
size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t n_tokens);

/* The leading bytes of a workspace that carry state from one call to the
 * next (error word, self-resetting arrival counters, the fused step's grid
 * size, per-workgroup epochs and its exchange words).  They sit at the same
 * offsets for every token count; every byte after them is scratch of one
 * call.  0 for an invalid descriptor. */
size_t moe_workspace_state_bytes(const moe_layer_desc *desc);

/* Human-readable text of a status code; static storage. */
const char *moe_strerror(int status);
/* Text of the calling thread's most recent error; thread-local storage. */
const char *moe_last_error(void);

/*
 * Routing (toolarium.ru, "Mixture of Experts и почему SSD достаточно";
 * hakusoku.com, "パイプライン概要": softmax over the router logits, top-K).
 * For each token t:
 *   logits[t][e] = sum_d router_w[e][d] * x[t][d]
 *   topk_idx[t][0..K) = the K largest logits in descending order, the lower
 *                       expert index first on an exact tie
 *   topk_w[t][k] = softmax over all E logits renormalised over the K
 *                  selected (= exp(l_k - l_max) / sum_j exp(l_j - l_max))
 * x: [T][D]; topk_idx: [T][K] int32; topk_w: [T][K]; logits: [T][E] or
 * NULL (then kept in the workspace).
 */
int moe_route(const moe_layer_desc *desc, const float *x, int32_t n_tokens, int32_t *topk_idx,
              float *topk_w, float *logits, void *workspace, size_t ws_bytes, void *stream);

/*
 * Expert forward and combine, no residual (hakusoku.com, "主要技術": 4/2-bit
 * dequant matvec, SwiGLU, MoE combine):
 *   E_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x)),  silu(z) = z / (1 + exp(-z))
 *   y[t] = sum_k topk_w[t][k] * E_{topk_idx[t][k]}(x[t]) + S(x[t])
 * where S is the shared expert (weight 1; absent when n_shared == 0).
 * x, y: [T][D]; topk_idx, topk_w: [T][K] as produced by moe_route (or any
 * caller-chosen routing).
 */
int moe_expert_forward(const moe_layer_desc *desc, const float *x, int32_t n_tokens,
                       const int32_t *topk_idx, const float *topk_w, float *y, void *workspace,
                       size_t ws_bytes, void *stream);

/*
 * One whole layer: route, expert forward and combine, then residual add and
 * RMSNorm fused (toolarium.ru, "Оптимизации, которые сработали": combine +
 * residual + normalisation in one GPU kernel; hakusoku.com, "主要技術": the
 * result goes straight to the next layer):
 *   c = moe_expert_forward(route(x))
 *   resid <- resid + c
 *   x <- resid / sqrt(mean_d(resid^2) + rms_eps) * gamma
 * resid, x: [T][D], in/out, must not overlap.  topk_idx/topk_w: [T][K]
 * outputs (the routing used), except in streamed mode (slab): there they are
 * inputs, the routing the slab was filled for (slot k holds the expert
 * topk_idx[k], typically moe_route's choice), and the step applies that
 * routing and its weights as given, without routing again.
 */
int moe_layer_step(const moe_layer_desc *desc, float *resid, float *x, int32_t n_tokens,
                   int32_t *topk_idx, float *topk_w, void *workspace, size_t ws_bytes, void *stream);

/*
 * A stack of n_layers layers for one token (batch 1): moe_layer_step applied
 * to layers[0], layers[1], ... in turn, each layer's (resid, x) output
 * feeding the next (the pages' engine hands the fused combine + norm result
 * straight to the next layer, hakusoku.com, "主要技術"; attention between
 * layers is absent here).  Results equal those of the n separate
 * moe_layer_step calls bit for bit; the stack runs as one persistent launch
 * per 64 layers, which removes the per-layer launch and lets each layer's
 * routing-independent weights (next router rows, shared expert) be fetched
 * while the previous layer finishes.
 * layers: host array of n_layers descriptors with the same hidden,
 * n_experts, top_k, inter, n_shared, bits and rms_eps (MOE_EINVAL
 * otherwise); each may be resident or streamed (its slab must then already
 * hold the experts its row of topk_idx names, in that order, and that row
 * and its topk_w row are inputs, as for moe_layer_step).  resid, x: [D]
 * device, in/out, must not overlap.  topk_idx/topk_w: [n_layers][K] device,
 * outputs for the resident layers.  record: NULL or device
 * [n_layers + 1][2][D], 16-byte aligned, receiving (resid, x) entering every
 * layer and the final output.  workspace: as moe_workspace_bytes(&layers[0],
 * 1).
 */
int moe_stack_step(const moe_layer_desc *layers, int32_t n_layers, float *resid, float *x, int32_t *topk_idx,
                   float *topk_w, float *record, void *workspace, size_t ws_bytes, void *stream);

/*
 * The dequantised expert GEMVs alone, for a range of a resident layer's
 * experts and one activation vector: the matrix-vector kernel the pages
 * measure against the memory bandwidth (hakusoku.com, 「Apple Siliconにおける
 * メモリ制約」), in the dequant form w = q*scale + bias.  For n < count and
 * expert e = first + n:
 *   h[n][i] = silu(sum_j Wg_e[i][j] x[j]) * sum_j Wu_e[i][j] x[j]
 *   y[n][o] = sum_i Wd_e[o][i] h[n][i]
 * No routing, no weighting, no residual.  One launch; a workgroup runs whole
 * experts (gate/up, then down from h kept on chip), so every byte of the
 * range's blobs is read once.
 * desc: resident (experts != NULL, no address table); 0 <= first, 1 <=
 * count, first + count <= n_experts (MOE_EINVAL otherwise).  x: [D]; h:
 * [count][I]; y: [count][D]; all 16-byte aligned device memory.
 */
int moe_expert_gemv(const moe_layer_desc *desc, const float *x, int32_t first, int32_t count, float *h, float *y,
                    void *stream);

/*
 * moe_stack_step without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  The library's own scratch serves as the
 * workspace: a 1 MiB device array per device, in the library's code object,
 * held until the process ends (every valid one-token shape fits; a shape
 * that does not returns MOE_EINVAL).  It is cleared before its first use on
 * a device and then keeps the state one call hands to the next, exactly as
 * a caller's workspace does.  Every call on a device shares that device's
 * array: calls that overlap on one device (on two streams, or from two
 * threads without ordering) race and their results are undefined; order
 * them on one stream.  The call allocates and frees nothing.
 * Arguments as moe_stack_step; flags: NULL or a device uint32 (4-byte
 * aligned, zeroed by the caller) into which the call's kernels OR their
 * MOE_DEVERR_* bits (with NULL they go to the scratch, unseen).
 */
int moe_stack_step_noalloc(const moe_layer_desc *layers, int32_t n_layers, float *resid, float *x, int32_t *topk_idx,
                           float *topk_w, float *record, uint32_t *flags, void *stream);

/*
 * How moe_layer_step / moe_stack_step will run this shape on the current
 * device (queries the device, enqueues nothing).  out[7] (host) receives:
 * fused (1 when a token's layers run as one persistent launch with
 * grid-wide barriers, 0 when each layer is three launches: route, gate/up,
 * down + norm), grid blocks, block threads, blocks per CU the device reports
 * for the persistent kernel, CU count, VGPRs per lane, scratch bytes per
 * lane.
 */
int moe_layer_plan(const moe_layer_desc *desc, int32_t n_tokens, int32_t *out);

/*
 * Token -> expert grouping of a batched call (n_tokens >= 2).  After
 * moe_route, moe_expert_forward or moe_layer_step on a batch, the workspace
 * holds, as int32 arrays at the byte offsets written to out[6] (host):
 *   out[0] count[E]        pairs routed to each expert
 *   out[1] offset[E+1]     exclusive prefix sum of count
 *   out[2] perm[T*K]       pair indices t*K + k grouped by expert (ascending
 *                          expert, ascending pair index inside an expert)
 *   out[3] pos[T*K]        inverse of perm (-1 for an out-of-range id)
 *   out[4] act[E]          the experts with count > 0, ascending
 *   out[5] n_act[1]        how many there are
 * Every routed expert's rows are read once per batched step and applied to
 * all of its tokens.  Queries the layout only; enqueues nothing.
 */
int moe_workspace_grouping(const moe_layer_desc *desc, int32_t n_tokens, size_t *out);

/*
 * Host-to-HBM expert streaming (toolarium.ru, "Flash-MoE: чистый C, Metal и
 * никакого Python": per layer, the selected experts' weights are read in
 * parallel and handed to the GPU; hakusoku.com, "パイプライン概要": the K=4
 * reads sit between routing and the expert forward).
 *
 * The expert weights live in pinned host memory; two device slab slots of
 * slab_blobs blobs each receive one layer's selections while the other slot
 * is being computed on.
 */
/*
 * HBM-side cache of expert blobs for the streamed layers, the analog
 * of the page cache that serves most expert reads on the pages' machine
 * (toolarium.ru, "Flash-MoE: чистый C, Metal и никакого Python": caching is
 * left to the OS page cache, which hits about 71% of reads).  n_slots blobs
 * in HBM hold recently streamed blobs (a layer's routed expert, or its
 * shared expert), replaced least recently used first.  moe_stream_token
 * then copies a cached blob into the slab device to device instead of over
 * the host link; a missed blob comes over the link into the slab and from
 * there into the least recently used slot.  All copies run on the copy
 * stream in issue order, so a slot is never refilled before earlier copies
 * out of it.
 *   slots:  device, n_slots * blob_bytes (caller-owned)
 *   meta:   host, moe_expert_cache_meta_bytes(n_slots, n_layers, n_experts)
 *           bytes, 8-byte aligned (caller-owned): the blob -> slot index and the
 *           LRU list, written by moe_expert_cache_reset and moe_stream_token
 *   hits, misses: blobs served from the cache / over the link
 *           (moe_expert_cache_reset clears them)
 *   speculate: when nonzero, right after a streamed layer's copies are
 *           queued, the routed experts the previous token selected in the
 *           next streamed layer (a temporal guess of the routing; the same
 *           article lists route prediction among the variants that were
 *           slower than the page cache there) that are not cached are
 *           copied host -> HBM into the cache, ahead of that layer's own
 *           routing
 *   spec_fills: blobs copied by that guess (moe_expert_cache_reset clears it)
 * moe_stream_prefetch itself never uses the cache.  A cache belongs to one
 * streamer (its n_layers and n_experts) and to one thread at a time.
 */
typedef struct moe_expert_cache {
    uint8_t *slots;
    int32_t n_slots;
    void *meta;
    uint64_t hits;
    uint64_t misses;
    int32_t speculate;
    uint64_t spec_fills;
} moe_expert_cache;

/* Bytes of host metadata for a cache of n_slots blobs over n_layers x
 * (n_experts routed + 1 shared) blobs (0 for a non-positive argument). */
size_t moe_expert_cache_meta_bytes(int32_t n_slots, int32_t n_layers, int32_t n_experts);

/* Empty the cache: every slot free, nothing indexed, counters zero.
 * MOE_EINVAL for a NULL cache, slots or meta, a meta block that is not
 * 8-byte aligned, or a non-positive size. */
int moe_expert_cache_reset(moe_expert_cache *c, int32_t n_layers, int32_t n_experts);

typedef struct moe_streamer {
    const uint8_t *host_arena;  /* host, pinned: routed blobs, blob_bytes apart */
    const uint8_t *host_shared; /* host, pinned: shared blobs, blob_bytes apart, or NULL */
    uint64_t blob_bytes;
    int32_t n_experts;          /* E */
    int32_t n_layers;
    /* Physical blobs in the arenas.  (layer, e) lives at arena blob
     * (layer*E + e) mod arena_blobs and layer's shared blob at shared blob
     * layer mod shared_blobs; arena_blobs = n_layers*E means no aliasing. */
    int64_t arena_blobs;
    int64_t shared_blobs;
    uint8_t *slab[2];           /* device: two slots of slab_blobs blobs */
    int32_t slab_blobs;         /* blobs per slot (top_k + 1) */
    moe_expert_cache *cache;    /* HBM expert cache used by moe_stream_token, or NULL */
} moe_streamer;

/*
 * Enqueue host->device copies of layer `layer`'s experts expert_ids[0..n_ids)
 * (host array, read before the call returns) into slab[slot] blobs 0..n_ids,
 * plus, when with_shared != 0, the layer's shared blob into blob
 * slab_blobs-1 of the slot, all on copy_stream; then record done_event
 * (a hipEvent_t, may be NULL) on copy_stream.  Ids out of range, n_ids >
 * slab_blobs - (with_shared != 0), a bad slot or layer, or a missing arena
 * return MOE_ESTATE before anything is enqueued.  The caller orders the
 * copy after the last kernel that read the slot (e.g. hipStreamWaitEvent).
 */
int moe_stream_prefetch(const moe_streamer *s, int32_t layer, const int32_t *expert_ids, int32_t n_ids,
                        int32_t slot, int32_t with_shared, void *copy_stream, void *done_event);

/*
 * Page-locked host memory for the streamer's arenas (hipHostMalloc): the
 * device's copy engines read it directly, so moe_stream_prefetch's copies
 * run asynchronously at link speed.  moe_host_alloc stores the address in
 * *out (NULL on failure) and returns MOE_EINVAL for bytes == 0 or out ==
 * NULL, MOE_EHIP when the runtime cannot pin that much.  The caller owns
 * the memory and releases it with moe_host_free (NULL is a no-op) after
 * every copy from it has completed.
 */
int moe_host_alloc(size_t bytes, void **out);
int moe_host_free(void *p);

/*
 * One decode token through n_layers layers, streamed or resident (the
 * per-layer pipeline of hakusoku.com, "パイプライン概要": routing, then the
 * selected experts' reads, then the expert forward with combine, residual
 * and norm; the expert work is queued without the host waiting for it, as
 * the pages' deferred command buffer).  A streamed layer l, the j-th
 * streamed one, uses slot s = j mod 2:
 *   1. moe_route on compute_stream; the K selections are copied to
 *      host_ids (pinned host, K int32) and the host waits for them;
 *   2. moe_stream_prefetch of those experts into slab slot s on
 *      copy_stream, after the streamed layer that last read the slot (j-2)
 *      (with st->cache set, cached experts are copied from HBM instead, see
 *      moe_expert_cache);
 *   3. compute_stream waits for the copies, then moe_layer_step reads the
 *      slot under the routing of step 1 (the slab's experts, in the order
 *      they were copied, with step 1's weights; the step does not route
 *      again);
 *   4. the shared expert of the next streamed layer (independent of
 *      routing) is queued on copy_stream right behind layer l's copies, so
 *      the link stays busy while the host waits for that layer's routing.
 * A resident layer (descriptor with experts != NULL: its experts in HBM, as
 * for moe_layer_step) runs moe_layer_step on compute_stream with no copy and
 * no host wait, so a caller chooses per layer which ones stream (hybrid
 * residency: the layers that fit in HBM stay there, the rest stream).
 * layers: host array of n_layers descriptors; streamed ones have experts ==
 * NULL and their slab field is replaced by st->slab[j mod 2]; all share
 * top_k and n_shared, and st->slab_blobs == top_k + n_shared.  resid, x:
 * [D] device, in/out.  topk_idx, topk_w: device [n_layers][K] outputs.
 * record: NULL or device [n_layers + 1][2][D], 16-byte aligned, receiving
 * (resid, x) entering every layer and the final output.
 * events: five hipEvent_t (route_done, copy_done[2], compute_done[2]).
 * Returns after the last layer has been enqueued; the caller synchronises
 * compute_stream for the result.
 */
int moe_stream_token(const moe_layer_desc *layers, int32_t n_layers, const moe_streamer *st, float *resid,
                     float *x, int32_t *topk_idx, float *topk_w, float *record, int32_t *host_ids, void *workspace,
                     size_t ws_bytes, void *compute_stream, void *copy_stream, void *const *events);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
