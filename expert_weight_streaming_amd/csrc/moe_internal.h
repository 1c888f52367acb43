// moe_internal.h -- shared between libmoe's host entry points and kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kGroup = 64;
constexpr int kMaxTopK = 8;
constexpr int kMaxSlots = kMaxTopK + 1;  // routed + shared
constexpr int kMaxLayerBlocks = 1024;    // grid cap of the persistent stack kernel
constexpr int kSlotWords = 16;           // one 64-byte barrier slot per block
// In a batch, experts with at least this many tokens take the matrix-core
// grouped kernels, the others the dot-product ones.
constexpr int kRouteSplit = 8;  // hidden-dimension slices of the batched router (partial logits)

// Router GEMV of one token (shared by the fused stack kernel and k_route, so
// that both produce the same fp32 logits bit for bit): RSL waves per router
// row, wave s owning float4 columns [s*Q, min(D/4, s*Q + Q)), Q = ceil(D/4 /
// RSL), fetched in rounds of 64*RN float4; the wave's partial sums are reduced
// across the wave and the RSL slice sums added in slice order.
constexpr int kRouterRN = 4;
constexpr int kRouterSlices = 4;

// Workspace layout (byte offsets), all 64-byte aligned.  The leading
// `state` bytes hold what a call hands to the next one on the same workspace
// (error flags, self-resetting arrival counters, the fused step's grid size,
// per-block epochs and tagged exchange words); their offsets depend on the
// layer shape only, never on the token count, so calls with different token
// counts can share one workspace.  Everything after `state` is per-call
// scratch.
struct WsLayout {
    size_t flags = 0;        // uint32 device error bits (OR-ed)
    size_t ctr_route = 64;   // uint32 arrival counter of the route kernel
    size_t hdr = 128;        // uint32 grid size of the persistent stack kernel last run on this workspace
    size_t ctr_down = 192;   // uint32 arrival counter of the down kernel (layer mode)
    size_t ctr_group = 224;  // uint32 arrival counter of the batched top-K kernel (its last block groups)
    size_t slots = 0;        // uint32 [kMaxLayerBlocks][kSlotWords] epochs reached by each block of the stack kernel
    // the stack kernel's exchanges: (value, epoch) pairs, uint64
    size_t tss = 0;          // [kMaxLayerBlocks] per-block sums of squares
    size_t tlog = 0;         // [E] logits
    size_t th = 0;           // [slots][I] h
    size_t tres = 0;         // [D] residual rows
    size_t state = 0;        // end of the state carried from call to call
    // per-call scratch
    size_t ss = 0;           // float [max(kMaxLayerBlocks, down blocks)] partial sums of squares (k_down)
    size_t logits = 0;       // float [T][E]
    size_t h = 0;            // float [T][slots][I]
    // batches (T > 1)
    size_t lpart = 0;        // float [kRouteSplit][T][E] partial logits
    size_t count = 0, offset = 0, perm = 0, pos_of_pair = 0, act = 0, n_act = 0;
    size_t mwork = 0, n_mwork = 0;  // expert-kernel work list: (item << 2 | 16-token tile), its length
    // digit words of x and h, with each (vector, scale group)'s sum and step
    size_t xdig = 0, xcsum = 0, xinv = 0, hdig = 0, hcsum = 0, hinv = 0, y = 0;
    size_t total = 0;
};

// Where the blobs of one layer live.
struct BlobSrc {
    const uint8_t *experts;  // resident arena (NULL when streamed)
    const uint8_t *shared;   // resident shared blob (or NULL)
    const uint8_t *slab;     // streamed slab (or NULL)
    uint64_t blob_bytes;
    int32_t n_experts;
    int32_t top_k;
    int32_t n_slots;         // top_k + n_shared
};

struct RouteArgs {
    const float *router;     // [E][D]
    const float *x;          // [D]
    float *logits;           // [E]
    int32_t *topk_idx;       // [K]
    float *topk_w;           // [K]
    uint32_t *counter;
    int32_t D, E, K;
};

struct GateUpArgs {
    BlobSrc src;
    const int32_t *topk_idx; // [K]
    const float *x;          // [D]
    float *h;                // [slots][I]
    uint32_t *flags;
    int32_t D, I;
    int32_t blocks_per_slot;
};

struct DownArgs {
    BlobSrc src;
    const int32_t *topk_idx; // [K]
    const float *topk_w;     // [K]
    const float *h;          // [slots][I]
    float *y;                // [D] combine output (mode 0)
    float *resid;            // [D] in/out (mode 1)
    float *x;                // [D] out (mode 1)
    const float *gamma;      // [D] (mode 1)
    float *ss;               // [blocks] (mode 1)
    uint32_t *counter;       // (mode 1)
    uint32_t *flags;
    int32_t D, I;
    float eps;
    int32_t mode;            // 0: y = combine; 1: resid += combine, x = RMSNorm(resid)
};


// A batch of T > 1 tokens (moe_batch.hip).  "Positions" number the
// (token, slot) pairs grouped by expert: routed pairs at offset[e] ..
// offset[e]+count[e]-1 in ascending pair index, then one shared-expert
// position per token at T*K + t.
struct BatchArgs {
    BlobSrc src;
    const float *router;     // [E][D]
    const float *gamma;      // [D]
    const float *x;          // [T][D] input activations
    float *resid;            // [T][D] in/out (mode 1)
    float *xout;             // [T][D] normalised output (mode 1)
    float *yout;             // [T][D] combine output (mode 0)
    int32_t *topk_idx;       // [T][K]
    float *topk_w;           // [T][K]
    float *logits;           // [T][E]
    float *lpart;            // [splits][T][E] partial logits over slices of the hidden dimension
    int32_t *count;          // [E]
    int32_t *offset;         // [E+1]
    int32_t *perm;           // [T*K] position -> pair index t*K + k
    int32_t *pos_of_pair;    // [T*K] pair index -> position (-1: invalid id)
    int32_t *act;            // [E] active experts, ascending
    int32_t *n_act;          // [1]
    int32_t *mwork;          // [(E+1)*4] expert-kernel work: item ii (act[ii], or the shared expert for
                             // ii == n_act) << 2 | tile of 16 of its tokens
    int32_t *n_mwork;        // [1]
    uint32_t *grp_arrive;    // arrival counter of k_topk_b's blocks (zero between calls)
    int *xdig;               // [T][D/64][48] digit words of x, per scale group
    float *xcsum;            // [T][D/64] group sums of x
    float *xinv;             // [T][D/64] group steps 2^-k
    int *hdig;               // [positions][I/64][48] digit words of h
    float *hcsum;            // [positions][I/64]
    float *hinv;             // [positions][I/64]
    float *y;                // [positions][D]
    uint32_t *flags;
    int32_t T, D, E, K, I;
    float eps;
    int32_t mode;            // 0: yout = combine; 1: residual + RMSNorm
};

// The expert GEMVs of a range of resident experts (moe_gemv.hip).
struct GemvArgs {
    const uint8_t *experts;  // resident arena, blob_bytes apart
    uint64_t blob_bytes;
    int32_t first, count;    // experts first .. first + count - 1
    const float *x;          // [D]
    float *h;                // [count][I]
    float *y;                // [count][D]
    int32_t D, I;
};

// Down-projection lane split: LPR lanes per row (a power of two <= 64),
// cpl 16-byte chunks per lane.
struct DownShape {
    int lpr, cpl;
};
DownShape down_shape(int I, int bits);

hipError_t launch_route(const RouteArgs &a, hipStream_t s);
hipError_t launch_batch_route(const BatchArgs &a, int do_topk, int bits, hipStream_t s);
hipError_t launch_batch_experts(const BatchArgs &a, int bits, hipStream_t s);
hipError_t launch_gate_up(const GateUpArgs &a, int bits, hipStream_t s);
hipError_t launch_down(const DownArgs &a, int bits, hipStream_t s);

struct LayerPlan;
// hipErrorNotSupported (nothing launched) for a shape without a plan; p
// (optional) receives the launch shape.
hipError_t launch_expert_gemv(const GemvArgs &a, int bits, hipStream_t s, LayerPlan *p);

// Launch plan of the persistent stack kernel for a shape (nothing
// launched): grid 0 when the shape takes the three-launch path.
struct LayerPlan {
    int grid = 0, block = 0, per_cu = 0, n_cu = 0, vgprs = 0, scratch = 0;
};

// One launch for a whole stack of layers (batch 1), moe_stack.hip.
constexpr int kMaxStackLayers = 64;
constexpr int kProbePoints = 16;  // stamps per layer and wave in timeline builds
constexpr int kStackThreads = 512;

struct StackLayer {
    const float *router;     // [E][D]
    const float *gamma;      // [D]
    const uint8_t *experts;  // resident arena of E blobs, or NULL
    const uint64_t *addr;    // or: [E] blob addresses (HBM or pinned host), or NULL
    const uint8_t *shared;   // shared blob (resident or address-table mode), or NULL
    const uint8_t *slab;     // streamed: slot k = selection k, slot K = shared
};

struct StackArgs {
    StackLayer layer[kMaxStackLayers];
    float *resid;            // [D] in/out
    float *x;                // [D] in/out
    int32_t *topk_idx;       // [n_layers][K] out
    float *topk_w;           // [n_layers][K] out
    float *record;           // [n_layers+1][2][D] (r, x) entering each layer and the output, or NULL
    uint64_t *tlog;          // workspace [E]: (logit, epoch)
    uint64_t *th;            // workspace [slots][I]: (h, epoch)
    uint64_t *tres;          // workspace [D]: (residual, epoch)
    uint64_t *tss;           // workspace [kMaxLayerBlocks]: (partial sum of squares, epoch)
    uint64_t *probe;         // timeline builds (MOE_STACK_PROBE): [n_layers][grid][8 waves][kProbePoints]
                             // s_memrealtime stamps, or NULL; unused otherwise
    uint32_t *hdr;           // workspace: grid of the last persistent launch (0: none yet)
    uint32_t *slots;         // workspace: per-block epoch reached by the last launch
    uint32_t *flags;
    uint64_t blob_bytes;
    int32_t n_layers, D, E, K, I, n_slots;
    float eps;
};

// Dynamic LDS of the stack kernel (byte offsets, 16-byte aligned).
struct StackLds {
    uint32_t xs, rs, dig, csum, xcinv, u, hdig, hcsum, hcinv, yh, misc, total;
};
constexpr int kStackMiscWords = 256;
// LDS of the stack kernel: x (fp32) and r of the layer, x's digit table
// with per-chunk sums and steps, a region shared by the router partials
// (phase A: one per wave and round of router rows) and the combined rows
// (phase C), h's digit tables with their per-chunk
// sums and steps, the slot partials that helper waves hand to their
// partners in the down phase, and small scalars (selection, weights, ready
// flags).
__host__ __device__ inline StackLds stack_lds(int D, int E, int I, int S, int bits)
{
    const uint32_t codes = 128 / bits, dw = 4 * (8 / bits) * 3;
    const uint32_t xc = (uint32_t)D / codes, hc = (uint32_t)S * ((uint32_t)I / codes);
    StackLds l;
    uint32_t o = 0;
    auto take = [&](uint32_t &f, uint32_t bytes) {
        f = o;
        o = (o + bytes + 15u) & ~15u;
    };
    take(l.xs, (uint32_t)D * 4);
    take(l.rs, (uint32_t)D * 4);
    take(l.dig, xc * dw * 4);
    take(l.csum, xc * 4);
    take(l.xcinv, xc * 4);
    const uint32_t un = (uint32_t)D > 4u * (uint32_t)E + 16u ? (uint32_t)D : 4u * (uint32_t)E + 16u;
    take(l.u, un * 4);
    take(l.hdig, hc * dw * 4);
    take(l.hcsum, hc * 4);
    take(l.hcinv, hc * 4);
    take(l.yh, 4u * 4u * 64u * 4u);  // helper waves' slot partials: [4 waves][4 slots][64 lanes]
    take(l.misc, kStackMiscWords * 4);
    l.total = o;
    return l;
}

// Persistent stack launch.  hipErrorNotSupported (nothing launched) when the
// shape has no resident-grid plan (scratch or LDS limits).
// a == NULL: only fill the plan (grid 0: no plan, the caller takes the
// three-launch path).
// tables: some layer of the launch is in address-table mode
hipError_t stack_bits4(const StackArgs *a, int D, int E, int I, int S, bool tables, hipStream_t s, LayerPlan *p);
hipError_t stack_bits2(const StackArgs *a, int D, int E, int I, int S, bool tables, hipStream_t s, LayerPlan *p);

int down_blocks(int D, int I, int bits);
int gate_up_blocks_per_slot(int I, int n_slots);

}  // namespace moe
