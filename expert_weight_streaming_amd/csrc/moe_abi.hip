// moe_abi.hip -- libmoe's C entry points: validation, workspace layout,
// launches, and the host->HBM expert streamer.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

// The workspace of moe_stack_step_noalloc: one array per device in the
// library's code object, held until the process ends.  Host code uses only
// the per-device addresses that hipGetSymbolAddress returns for it.
static __device__ __align__(256) uint8_t scratch[1u << 20];

namespace {

thread_local char g_err[512] = "";

// Timeline builds (-DMOE_STACK_PROBE): where the stack kernel stores its
// stamps (moe_probe_set); always NULL otherwise.
uint64_t *g_probe = nullptr;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

uint64_t blob_bytes_of(int32_t D, int32_t I, int32_t bits, int32_t group)
{
    if (D <= 0 || I <= 0 || (bits != 2 && bits != 4) || group != moe::kGroup) return 0;
    if (D % group || I % group) return 0;
    const uint64_t n = 3ull * (uint64_t)D * (uint64_t)I;
    return n * (uint64_t)bits / 8 + n / (uint64_t)group * 4;
}

int check_desc(const moe_layer_desc *d, int32_t T)
{
    if (!d) return fail(MOE_EINVAL, "desc is NULL");
    if (d->group != moe::kGroup) return fail(MOE_EINVAL, "group must be 64 (got %d)", d->group);
    if (d->bits != 2 && d->bits != 4) return fail(MOE_EINVAL, "bits must be 2 or 4 (got %d)", d->bits);
    if (d->hidden <= 0 || d->hidden % 64 || d->hidden > 8192)
        return fail(MOE_EINVAL, "hidden must be a positive multiple of 64, <= 8192 (got %d)", d->hidden);
    if (d->inter <= 0 || d->inter % 64 || d->inter > 4096)
        return fail(MOE_EINVAL, "inter must be a positive multiple of 64, <= 4096 (got %d)", d->inter);
    if (d->n_experts <= 0 || d->n_experts > 4096)
        return fail(MOE_EINVAL, "n_experts must be in [1, 4096] (got %d)", d->n_experts);
    if (d->top_k < 1 || d->top_k > moe::kMaxTopK || d->top_k > d->n_experts)
        return fail(MOE_EINVAL, "top_k must be in [1, min(n_experts, 8)] (got %d)", d->top_k);
    if (d->n_shared != 0 && d->n_shared != 1) return fail(MOE_EINVAL, "n_shared must be 0 or 1");
    if (!(d->rms_eps >= 0.f)) return fail(MOE_EINVAL, "rms_eps must be >= 0");
    if (T < 1 || T > 64) return fail(MOE_EINVAL, "n_tokens must be in [1, 64] (got %d)", T);
    if (d->blob_bytes != blob_bytes_of(d->hidden, d->inter, d->bits, d->group))
        return fail(MOE_EINVAL, "blob_bytes %llu does not match the shape (%llu)", (unsigned long long)d->blob_bytes,
                    (unsigned long long)blob_bytes_of(d->hidden, d->inter, d->bits, d->group));
    if (!d->router_w || !aligned16(d->router_w)) return fail(MOE_EINVAL, "router_w NULL or not 16-byte aligned");
    if (!d->gamma || !aligned16(d->gamma)) return fail(MOE_EINVAL, "gamma NULL or not 16-byte aligned");
    if (d->expert_addr) {
        if (d->experts || d->slab) return fail(MOE_EINVAL, "expert_addr excludes experts and slab");
        if (!aligned16(d->expert_addr)) return fail(MOE_EINVAL, "expert_addr not 16-byte aligned");
        if (d->n_shared && (!d->shared || !aligned16(d->shared)))
            return fail(MOE_EINVAL, "n_shared=1 needs a 16-byte aligned shared blob");
        if (T != 1) return fail(MOE_EUNSUPPORTED, "address-table mode takes one token per call");
        return MOE_OK;
    }
    const bool streamed = d->experts == nullptr;
    if (streamed) {
        if (!d->slab || !aligned16(d->slab)) return fail(MOE_EINVAL, "streamed mode needs a 16-byte aligned slab");
        if (T != 1) return fail(MOE_EUNSUPPORTED, "streamed mode takes one token per call");
    } else {
        if (!aligned16(d->experts)) return fail(MOE_EINVAL, "experts not 16-byte aligned");
        if (d->n_shared && (!d->shared || !aligned16(d->shared)))
            return fail(MOE_EINVAL, "n_shared=1 needs a 16-byte aligned shared blob");
    }
    return MOE_OK;
}

int check_ptr(const void *p, const char *name)
{
    if (!p || !aligned16(p)) return fail(MOE_EINVAL, "%s NULL or not 16-byte aligned", name);
    return MOE_OK;
}

int check_ptr4(const void *p, const char *name)
{
    if (!p || ((uintptr_t)p & 3u)) return fail(MOE_EINVAL, "%s NULL or not 4-byte aligned", name);
    return MOE_OK;
}

moe::WsLayout layout(const moe_layer_desc *d, int32_t T)
{
    moe::WsLayout L;
    size_t off = 256;
    auto take = [&](size_t &field, size_t bytes) {
        field = off;
        off = round_up(off + bytes, 256);
    };
    const size_t S = (size_t)d->top_k + d->n_shared;
    // state carried from call to call: offsets independent of T
    take(L.slots, (size_t)moe::kMaxLayerBlocks * moe::kSlotWords * 4);
    take(L.tss, (size_t)moe::kMaxLayerBlocks * 8);
    take(L.tlog, (size_t)d->n_experts * 8);
    take(L.th, S * d->inter * 8);
    take(L.tres, (size_t)d->hidden * 8);
    L.state = off;
    // per-call scratch
    const size_t nss = (size_t)moe::kMaxLayerBlocks > (size_t)moe::down_blocks(d->hidden, d->inter, d->bits)
                           ? (size_t)moe::kMaxLayerBlocks
                           : (size_t)moe::down_blocks(d->hidden, d->inter, d->bits);
    take(L.ss, nss * 4);
    take(L.logits, (size_t)T * d->n_experts * 4);
    take(L.h, (size_t)T * S * d->inter * 4);
    if (T > 1) {
        const size_t E = d->n_experts, K = d->top_k, D = d->hidden, I = d->inter;
        const size_t P = (size_t)T * (K + d->n_shared);
        const size_t G = moe::kGroup;  // activations per scale group
        take(L.lpart, (size_t)moe::kRouteSplit * T * E * 4);
        take(L.count, E * 4);
        take(L.offset, (E + 1) * 4);
        take(L.perm, T * K * 4);
        take(L.pos_of_pair, T * K * 4);
        take(L.act, E * 4);
        take(L.n_act, 4);
        take(L.mwork, (E + 1) * 4 * 4);
        take(L.n_mwork, 4);
        take(L.xdig, (size_t)T * (D * 3 / 4) * 4);
        take(L.xcsum, (size_t)T * (D / G) * 4);
        take(L.xinv, (size_t)T * (D / G) * 4);
        take(L.hdig, P * (I * 3 / 4) * 4);
        take(L.hcsum, P * (I / G) * 4);
        take(L.hinv, P * (I / G) * 4);
        take(L.y, P * D * 4);
    }
    L.total = off;
    return L;
}

moe::BlobSrc blob_src(const moe_layer_desc *d)
{
    moe::BlobSrc s;
    s.experts = d->experts;
    s.shared = d->experts ? d->shared : nullptr;
    s.slab = d->experts ? nullptr : d->slab;
    s.blob_bytes = d->blob_bytes;
    s.n_experts = d->n_experts;
    s.top_k = d->top_k;
    s.n_slots = d->top_k + d->n_shared;
    return s;
}

int check_ws(const moe_layer_desc *d, int32_t T, void *ws, size_t ws_bytes)
{
    if (!ws || ((uintptr_t)ws & 255u)) return fail(MOE_EINVAL, "workspace NULL or not 256-byte aligned");
    const size_t need = layout(d, T).total;
    if (ws_bytes < need) return fail(MOE_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
    return MOE_OK;
}

int enqueue_route(const moe_layer_desc *d, const float *x, int32_t *idx, float *w, float *logits, uint8_t *ws,
                  const moe::WsLayout &L, hipStream_t s)
{
    moe::RouteArgs a;
    a.router = d->router_w;
    a.x = x;
    a.logits = logits ? logits : reinterpret_cast<float *>(ws + L.logits);
    a.topk_idx = idx;
    a.topk_w = w;
    a.counter = reinterpret_cast<uint32_t *>(ws + L.ctr_route);
    a.D = d->hidden;
    a.E = d->n_experts;
    a.K = d->top_k;
    hipError_t e = moe::launch_route(a, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "route launch");
}

// Gate/up then down + combine.  y != NULL: y = combine (no residual).
// y == NULL: resid += combine, xout = RMSNorm(resid) * gamma.
int enqueue_forward(const moe_layer_desc *d, const float *x, const int32_t *idx, const float *w, float *y,
                    float *resid, float *xout, uint8_t *ws, const moe::WsLayout &L, hipStream_t s,
                    uint32_t *flags = nullptr)
{
    moe::GateUpArgs g;
    g.src = blob_src(d);
    g.topk_idx = idx;
    g.x = x;
    g.h = reinterpret_cast<float *>(ws + L.h);
    g.flags = flags ? flags : reinterpret_cast<uint32_t *>(ws + L.flags);
    g.D = d->hidden;
    g.I = d->inter;
    g.blocks_per_slot = moe::gate_up_blocks_per_slot(d->inter, d->top_k + d->n_shared);
    hipError_t e = moe::launch_gate_up(g, d->bits, s);
    if (e != hipSuccess) return hip_fail(e, "gate/up launch");

    moe::DownArgs a;
    a.src = g.src;
    a.topk_idx = idx;
    a.topk_w = w;
    a.h = g.h;
    a.y = y;
    a.resid = resid;
    a.x = xout;
    a.gamma = d->gamma;
    a.ss = reinterpret_cast<float *>(ws + L.ss);
    a.counter = reinterpret_cast<uint32_t *>(ws + L.ctr_down);
    a.flags = g.flags;
    a.D = d->hidden;
    a.I = d->inter;
    a.eps = d->rms_eps;
    a.mode = y ? 0 : 1;
    e = moe::launch_down(a, d->bits, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "down launch");
}

moe::StackLayer stack_layer(const moe_layer_desc *d)
{
    moe::StackLayer y;
    const bool on_device = d->experts || d->expert_addr;
    y.router = d->router_w;
    y.gamma = d->gamma;
    y.experts = d->experts;
    y.addr = d->expert_addr;
    y.shared = on_device ? d->shared : nullptr;
    y.slab = on_device ? nullptr : d->slab;
    return y;
}

// tables: some layer of the launch is in address-table mode
hipError_t stack_plan_or_launch(const moe::StackArgs *a, const moe_layer_desc *d, bool tables, hipStream_t s,
                                moe::LayerPlan *p)
{
    const int S = d->top_k + d->n_shared;
    return d->bits == 4 ? moe::stack_bits4(a, d->hidden, d->n_experts, d->inter, S, tables, s, p)
                        : moe::stack_bits2(a, d->hidden, d->n_experts, d->inter, S, tables, s, p);
}

// n layers of one token (batch 1).  Persistent launches of up to
// kMaxStackLayers layers each; shapes without a resident-grid plan take
// three launches per layer (route, gate/up, down with residual and norm).
// record (optional): [n+1][2][D] (r, x) entering every layer and the output.
int enqueue_stack(const moe_layer_desc *ds, int32_t n, float *resid, float *x, int32_t *idx, float *w, float *record,
                  uint8_t *ws, const moe::WsLayout &L, hipStream_t s, uint32_t *flags = nullptr)
{
    const moe_layer_desc *d = &ds[0];
    const int D = d->hidden, K = d->top_k;
    for (int32_t j = 0; j < n; ++j)
        if (ds[j].expert_addr) {
            // address tables are read by the fused kernel only
            moe::LayerPlan p;
            hipError_t e = stack_plan_or_launch(nullptr, d, true, s, &p);
            if (e != hipSuccess) return hip_fail(e, "stack plan");
            if (p.grid == 0) return fail(MOE_EUNSUPPORTED, "address-table mode needs the fused stack, which this shape has no plan for");
            break;
        }
    for (int32_t l0 = 0; l0 < n; l0 += moe::kMaxStackLayers) {
        const int cnt = n - l0 < moe::kMaxStackLayers ? n - l0 : moe::kMaxStackLayers;
        moe::StackArgs a;
        bool tables = false;
        for (int j = 0; j < cnt; ++j) {
            a.layer[j] = stack_layer(&ds[l0 + j]);
            tables = tables || ds[l0 + j].expert_addr;
        }
        a.resid = resid;
        a.x = x;
        a.topk_idx = idx + (size_t)l0 * K;
        a.topk_w = w + (size_t)l0 * K;
        a.record = record ? record + (size_t)l0 * 2 * D : nullptr;
        a.tlog = reinterpret_cast<uint64_t *>(ws + L.tlog);
        a.th = reinterpret_cast<uint64_t *>(ws + L.th);
        a.tres = reinterpret_cast<uint64_t *>(ws + L.tres);
        a.tss = reinterpret_cast<uint64_t *>(ws + L.tss);
        a.probe = g_probe;
        a.hdr = reinterpret_cast<uint32_t *>(ws + L.hdr);
        a.slots = reinterpret_cast<uint32_t *>(ws + L.slots);
        a.flags = flags ? flags : reinterpret_cast<uint32_t *>(ws + L.flags);
        a.blob_bytes = d->blob_bytes;
        a.n_layers = cnt;
        a.D = D;
        a.E = d->n_experts;
        a.K = K;
        a.I = d->inter;
        a.n_slots = K + d->n_shared;
        a.eps = d->rms_eps;
        moe::LayerPlan p;
        hipError_t e = stack_plan_or_launch(&a, d, tables, s, &p);
        if (e == hipSuccess) continue;
        if (e != hipErrorNotSupported) return hip_fail(e, "stack launch");
        // no resident-grid plan for this shape: three launches per layer
        for (int j = 0; j < cnt; ++j) {
            const moe_layer_desc *dj = &ds[l0 + j];
            int32_t *ij = idx + (size_t)(l0 + j) * K;
            float *wj = w + (size_t)(l0 + j) * K;
            if (record) {
                float *rj = record + (size_t)(l0 + j) * 2 * D;
                if ((e = hipMemcpyAsync(rj, resid, (size_t)D * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
                    (e = hipMemcpyAsync(rj + D, x, (size_t)D * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
                    return hip_fail(e, "record copy");
            }
            // a streamed layer's routing is the one its slab was filled for (given)
            const bool slab = !dj->experts && !dj->expert_addr;
            int rc = slab ? MOE_OK : enqueue_route(dj, x, ij, wj, nullptr, ws, L, s);
            if (rc) return rc;
            if ((rc = enqueue_forward(dj, x, ij, wj, nullptr, resid, x, ws, L, s, flags))) return rc;
        }
        if (record) {
            float *rn = record + (size_t)(l0 + cnt) * 2 * D;
            if ((e = hipMemcpyAsync(rn, resid, (size_t)D * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
                (e = hipMemcpyAsync(rn + D, x, (size_t)D * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
                return hip_fail(e, "record copy");
        }
    }
    return MOE_OK;
}

moe::BatchArgs batch_args(const moe_layer_desc *d, int32_t T, const float *x, int32_t *idx, float *w,
                          float *logits, uint8_t *ws, const moe::WsLayout &L)
{
    moe::BatchArgs b;
    b.src = blob_src(d);
    b.router = d->router_w;
    b.gamma = d->gamma;
    b.x = x;
    b.resid = nullptr;
    b.xout = nullptr;
    b.yout = nullptr;
    b.topk_idx = idx;
    b.topk_w = w;
    b.logits = logits ? logits : reinterpret_cast<float *>(ws + L.logits);
    b.lpart = reinterpret_cast<float *>(ws + L.lpart);
    b.count = reinterpret_cast<int32_t *>(ws + L.count);
    b.offset = reinterpret_cast<int32_t *>(ws + L.offset);
    b.perm = reinterpret_cast<int32_t *>(ws + L.perm);
    b.pos_of_pair = reinterpret_cast<int32_t *>(ws + L.pos_of_pair);
    b.act = reinterpret_cast<int32_t *>(ws + L.act);
    b.n_act = reinterpret_cast<int32_t *>(ws + L.n_act);
    b.mwork = reinterpret_cast<int32_t *>(ws + L.mwork);
    b.n_mwork = reinterpret_cast<int32_t *>(ws + L.n_mwork);
    b.grp_arrive = reinterpret_cast<uint32_t *>(ws + L.ctr_group);
    b.xdig = reinterpret_cast<int *>(ws + L.xdig);
    b.xcsum = reinterpret_cast<float *>(ws + L.xcsum);
    b.xinv = reinterpret_cast<float *>(ws + L.xinv);
    b.hdig = reinterpret_cast<int *>(ws + L.hdig);
    b.hcsum = reinterpret_cast<float *>(ws + L.hcsum);
    b.hinv = reinterpret_cast<float *>(ws + L.hinv);
    b.y = reinterpret_cast<float *>(ws + L.y);
    b.flags = reinterpret_cast<uint32_t *>(ws + L.flags);
    b.T = T;
    b.D = d->hidden;
    b.E = d->n_experts;
    b.K = d->top_k;
    b.I = d->inter;
    b.eps = d->rms_eps;
    b.mode = 0;
    return b;
}

}  // namespace

extern "C" {

size_t moe_blob_bytes(int32_t hidden, int32_t inter, int32_t bits, int32_t group)
{
    return (size_t)blob_bytes_of(hidden, inter, bits, group);
}

size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t n_tokens)
{
    if (check_desc(desc, n_tokens) != MOE_OK) return 0;
    return layout(desc, n_tokens).total;
}

size_t moe_workspace_state_bytes(const moe_layer_desc *desc)
{
    if (check_desc(desc, 1) != MOE_OK) return 0;
    return layout(desc, 1).state;
}

const char *moe_strerror(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported request";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_ESTATE: return "streamer state error";
    default: return "unknown status";
    }
}

const char *moe_last_error(void) { return g_err; }

int moe_route(const moe_layer_desc *desc, const float *x, int32_t n_tokens, int32_t *topk_idx, float *topk_w,
              float *logits, void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_desc(desc, n_tokens);
    if (rc) return rc;
    if ((rc = check_ptr(x, "x")) || (rc = check_ptr4(topk_idx, "topk_idx")) || (rc = check_ptr4(topk_w, "topk_w")))
        return rc;
    if (logits && ((uintptr_t)logits & 3u)) return fail(MOE_EINVAL, "logits not 4-byte aligned");
    if ((rc = check_ws(desc, n_tokens, workspace, ws_bytes))) return rc;
    const moe::WsLayout L = layout(desc, n_tokens);
    if (n_tokens > 1) {
        const moe::BatchArgs b = batch_args(desc, n_tokens, x, topk_idx, topk_w, logits, (uint8_t *)workspace, L);
        hipError_t e = moe::launch_batch_route(b, 1, desc->bits, (hipStream_t)stream);
        return e == hipSuccess ? MOE_OK : hip_fail(e, "batched route launch");
    }
    return enqueue_route(desc, x, topk_idx, topk_w, logits, (uint8_t *)workspace, L, (hipStream_t)stream);
}

int moe_expert_forward(const moe_layer_desc *desc, const float *x, int32_t n_tokens, const int32_t *topk_idx,
                       const float *topk_w, float *y, void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_desc(desc, n_tokens);
    if (rc) return rc;
    if ((rc = check_ptr(x, "x")) || (rc = check_ptr4(topk_idx, "topk_idx")) || (rc = check_ptr4(topk_w, "topk_w")) ||
        (rc = check_ptr(y, "y")))
        return rc;
    if ((rc = check_ws(desc, n_tokens, workspace, ws_bytes))) return rc;
    if (desc->expert_addr) return fail(MOE_EUNSUPPORTED, "moe_expert_forward does not take address-table mode");
    const moe::WsLayout L = layout(desc, n_tokens);
    if (n_tokens > 1) {
        moe::BatchArgs b = batch_args(desc, n_tokens, x, const_cast<int32_t *>(topk_idx), const_cast<float *>(topk_w),
                                      nullptr, (uint8_t *)workspace, L);
        b.yout = y;
        b.mode = 0;
        hipError_t e = moe::launch_batch_route(b, 0, desc->bits, (hipStream_t)stream);
        if (e == hipSuccess) e = moe::launch_batch_experts(b, desc->bits, (hipStream_t)stream);
        return e == hipSuccess ? MOE_OK : hip_fail(e, "batched expert launch");
    }
    return enqueue_forward(desc, x, topk_idx, topk_w, y, nullptr, nullptr, (uint8_t *)workspace, L,
                           (hipStream_t)stream);
}

int moe_layer_step(const moe_layer_desc *desc, float *resid, float *x, int32_t n_tokens, int32_t *topk_idx,
                   float *topk_w, void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_desc(desc, n_tokens);
    if (rc) return rc;
    if ((rc = check_ptr(resid, "resid")) || (rc = check_ptr(x, "x")) || (rc = check_ptr4(topk_idx, "topk_idx")) ||
        (rc = check_ptr4(topk_w, "topk_w")))
        return rc;
    const size_t span = (size_t)n_tokens * desc->hidden * 4;
    if ((const uint8_t *)resid < (const uint8_t *)x + span && (const uint8_t *)x < (const uint8_t *)resid + span)
        return fail(MOE_EINVAL, "resid and x overlap");
    if ((rc = check_ws(desc, n_tokens, workspace, ws_bytes))) return rc;
    const moe::WsLayout L = layout(desc, n_tokens);
    if (n_tokens > 1) {
        moe::BatchArgs b = batch_args(desc, n_tokens, x, topk_idx, topk_w, nullptr, (uint8_t *)workspace, L);
        b.resid = resid;
        b.xout = x;
        b.mode = 1;
        hipError_t e = moe::launch_batch_route(b, 1, desc->bits, (hipStream_t)stream);
        if (e == hipSuccess) e = moe::launch_batch_experts(b, desc->bits, (hipStream_t)stream);
        return e == hipSuccess ? MOE_OK : hip_fail(e, "batched layer launch");
    }
    return enqueue_stack(desc, 1, resid, x, topk_idx, topk_w, nullptr, (uint8_t *)workspace, L, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// moe_stack_step's checks of everything but the workspace.
int check_stack(const moe_layer_desc *layers, int32_t n_layers, float *resid, float *x, int32_t *topk_idx,
                float *topk_w, float *record)
{
    if (!layers || n_layers < 1) return fail(MOE_EINVAL, "no layers");
    int rc = check_desc(&layers[0], 1);
    if (rc) return rc;
    const moe_layer_desc *d = &layers[0];
    for (int32_t l = 1; l < n_layers; ++l) {
        const moe_layer_desc *e = &layers[l];
        if ((rc = check_desc(e, 1))) return rc;
        if (e->hidden != d->hidden || e->n_experts != d->n_experts || e->top_k != d->top_k || e->inter != d->inter ||
            e->n_shared != d->n_shared || e->bits != d->bits || e->rms_eps != d->rms_eps)
            return fail(MOE_EINVAL, "layer %d differs in shape or rms_eps from layer 0", l);
    }
    if ((rc = check_ptr(resid, "resid")) || (rc = check_ptr(x, "x")) || (rc = check_ptr4(topk_idx, "topk_idx")) ||
        (rc = check_ptr4(topk_w, "topk_w")))
        return rc;
    if (record && !aligned16(record)) return fail(MOE_EINVAL, "record not 16-byte aligned");
    const size_t span = (size_t)d->hidden * 4;
    if ((const uint8_t *)resid < (const uint8_t *)x + span && (const uint8_t *)x < (const uint8_t *)resid + span)
        return fail(MOE_EINVAL, "resid and x overlap");
    return MOE_OK;
}

// Per-device address of `scratch` (hipGetSymbolAddress with the device
// current) and whether it has been cleared by an eager launch.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[kMaxDevices];
bool g_scratch_clear[kMaxDevices];

__global__ void k_zero16(uint4 *p, uint32_t n16)
{
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" {

int moe_stack_step_noalloc(const moe_layer_desc *layers, int32_t n_layers, float *resid, float *x, int32_t *topk_idx,
                           float *topk_w, float *record, uint32_t *flags, void *stream)
{
    int rc = check_stack(layers, n_layers, resid, x, topk_idx, topk_w, record);
    if (rc) return rc;
    if (flags && ((uintptr_t)flags & 3u)) return fail(MOE_EINVAL, "flags not 4-byte aligned");
    const moe::WsLayout L = layout(&layers[0], 1);
    if (L.total > sizeof(scratch))
        return fail(MOE_EINVAL, "this shape needs %zu bytes of workspace, more than the %zu of the library's scratch",
                    L.total, sizeof(scratch));
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "current device");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device %d beyond the %d the library serves", dev, kMaxDevices);
    uint8_t *ws = nullptr;
    bool clear = false;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void *p = nullptr;
            if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return hip_fail(e, "scratch address");
            g_scratch_ptr[dev] = static_cast<uint8_t *>(p);
        }
        ws = g_scratch_ptr[dev];
        clear = !g_scratch_clear[dev];
    }
    hipStream_t s = (hipStream_t)stream;
    if (clear) {
        // the epochs and exchange words must start at zero: a fill kernel
        // ahead of the step (also when the stream is being captured, so that
        // a graph clears it on each replay); once an eager launch has
        // cleared it, the state carries over from call to call
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if ((e = hipStreamIsCapturing(s, &cap)) != hipSuccess) return hip_fail(e, "capture status");
        hipLaunchKernelGGL(k_zero16, dim3(256), dim3(256), 0, s, reinterpret_cast<uint4 *>(ws),
                           (uint32_t)(sizeof(scratch) / 16));
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "scratch clear");
        if (cap == hipStreamCaptureStatusNone) {
            std::lock_guard<std::mutex> lock(g_scratch_mu);
            g_scratch_clear[dev] = true;
        }
    }
    return enqueue_stack(layers, n_layers, resid, x, topk_idx, topk_w, record, ws, L, s, flags);
}

int moe_stack_step(const moe_layer_desc *layers, int32_t n_layers, float *resid, float *x, int32_t *topk_idx,
                   float *topk_w, float *record, void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_stack(layers, n_layers, resid, x, topk_idx, topk_w, record);
    if (rc) return rc;
    if ((rc = check_ws(&layers[0], 1, workspace, ws_bytes))) return rc;
    const moe::WsLayout L = layout(&layers[0], 1);
    return enqueue_stack(layers, n_layers, resid, x, topk_idx, topk_w, record, (uint8_t *)workspace, L,
                         (hipStream_t)stream);
}

int moe_expert_gemv(const moe_layer_desc *desc, const float *x, int32_t first, int32_t count, float *h, float *y,
                    void *stream)
{
    int rc = check_desc(desc, 1);
    if (rc) return rc;
    if (!desc->experts || desc->expert_addr)
        return fail(MOE_EINVAL, "moe_expert_gemv needs a resident layer (experts in device-visible memory)");
    if (first < 0 || count < 1 || (int64_t)first + count > desc->n_experts)
        return fail(MOE_EINVAL, "expert range [%d, %d + %d) outside [0, %d)", first, first, count, desc->n_experts);
    if ((rc = check_ptr(x, "x")) || (rc = check_ptr(h, "h")) || (rc = check_ptr(y, "y"))) return rc;
    moe::GemvArgs a;
    a.experts = desc->experts;
    a.blob_bytes = desc->blob_bytes;
    a.first = first;
    a.count = count;
    a.x = x;
    a.h = h;
    a.y = y;
    a.D = desc->hidden;
    a.I = desc->inter;
    hipError_t e = moe::launch_expert_gemv(a, desc->bits, (hipStream_t)stream, nullptr);
    if (e == hipErrorNotSupported) return fail(MOE_EUNSUPPORTED, "no expert GEMV plan for this shape");
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert GEMV launch");
}

int moe_layer_plan(const moe_layer_desc *desc, int32_t n_tokens, int32_t *out)
{
    int rc = check_desc(desc, n_tokens);
    if (rc) return rc;
    if (!out) return fail(MOE_EINVAL, "out is NULL");
    moe::LayerPlan p;
    hipError_t e = stack_plan_or_launch(nullptr, desc, desc->expert_addr != nullptr, nullptr, &p);
    if (e != hipSuccess) return hip_fail(e, "layer plan");
    out[0] = p.grid > 0 && n_tokens == 1 ? 1 : 0;
    out[1] = p.grid;
    out[2] = p.block;
    out[3] = p.per_cu;
    out[4] = p.n_cu;
    out[5] = p.vgprs;
    out[6] = p.scratch;
    return MOE_OK;
}

int moe_workspace_grouping(const moe_layer_desc *desc, int32_t n_tokens, size_t *out)
{
    int rc = check_desc(desc, n_tokens);
    if (rc) return rc;
    if (!out) return fail(MOE_EINVAL, "out is NULL");
    if (n_tokens < 2) return fail(MOE_EINVAL, "the grouping exists for n_tokens >= 2");
    const moe::WsLayout L = layout(desc, n_tokens);
    out[0] = L.count;
    out[1] = L.offset;
    out[2] = L.perm;
    out[3] = L.pos_of_pair;
    out[4] = L.act;
    out[5] = L.n_act;
    return MOE_OK;
}

// ---- HBM expert cache: host metadata laid out in the caller's meta block
//   CacheHead | tag[n_slots] (int64 key, -1 free) | where[L*E + L] (int32:
//   slot, -1 not cached) | prev[n_slots] | next[n_slots] (LRU list, most
//   recent first) | pred[L][kMaxTopK] (int32: the previous token's
//   selection per layer, -1 none).  Keys: layer*E + e for routed expert e of
//   a layer, L*E + layer for the layer's shared expert.
struct CacheHead {
    int32_t n_layers, n_experts, n_slots, head, tail, pad;
};
struct CacheView {
    CacheHead *h;
    int64_t *tag;
    int32_t *where, *prev, *next, *pred;
};
static CacheView cache_view(void *meta, int32_t n_slots, int32_t n_layers, int32_t n_experts)
{
    CacheView v;
    uint8_t *p = static_cast<uint8_t *>(meta);
    v.h = reinterpret_cast<CacheHead *>(p);
    v.tag = reinterpret_cast<int64_t *>(p + sizeof(CacheHead));
    v.where = reinterpret_cast<int32_t *>(v.tag + n_slots);
    v.prev = v.where + (size_t)n_layers * (n_experts + 1);
    v.next = v.prev + n_slots;
    v.pred = v.next + n_slots;
    return v;
}
static void lru_unlink(CacheView &v, int32_t s)
{
    const int32_t p = v.prev[s], n = v.next[s];
    if (p >= 0) v.next[p] = n; else v.h->head = n;
    if (n >= 0) v.prev[n] = p; else v.h->tail = p;
}
static void lru_push_front(CacheView &v, int32_t s)
{
    v.prev[s] = -1;
    v.next[s] = v.h->head;
    if (v.h->head >= 0) v.prev[v.h->head] = s;
    v.h->head = s;
    if (v.h->tail < 0) v.h->tail = s;
}

size_t moe_expert_cache_meta_bytes(int32_t n_slots, int32_t n_layers, int32_t n_experts)
{
    if (n_slots <= 0 || n_layers <= 0 || n_experts <= 0) return 0;
    return sizeof(CacheHead) + (size_t)n_slots * 8 + (size_t)n_layers * (n_experts + 1) * 4 + (size_t)n_slots * 8 +
           (size_t)n_layers * moe::kMaxTopK * 4;
}

int moe_expert_cache_reset(moe_expert_cache *c, int32_t n_layers, int32_t n_experts)
{
    if (!c || !c->slots || !c->meta) return fail(MOE_EINVAL, "cache, its slots or its meta block is NULL");
    if (reinterpret_cast<uintptr_t>(c->meta) & 7u) return fail(MOE_EINVAL, "cache meta block not 8-byte aligned");
    if (c->n_slots <= 0 || n_layers <= 0 || n_experts <= 0)
        return fail(MOE_EINVAL, "cache sizes must be positive (slots %d, layers %d, experts %d)", c->n_slots, n_layers, n_experts);
    CacheView v = cache_view(c->meta, c->n_slots, n_layers, n_experts);
    *v.h = CacheHead{n_layers, n_experts, c->n_slots, -1, -1, 0};
    for (int32_t s = 0; s < c->n_slots; ++s) {
        v.tag[s] = -1;
        lru_push_front(v, s);
    }
    for (size_t k = 0; k < (size_t)n_layers * (n_experts + 1); ++k) v.where[k] = -1;
    for (size_t k = 0; k < (size_t)n_layers * moe::kMaxTopK; ++k) v.pred[k] = -1;
    c->hits = c->misses = c->spec_fills = 0;
    return MOE_OK;
}

static int stream_copies(const moe_streamer *st, int32_t layer, const int32_t *expert_ids, int32_t n_ids, int32_t slot,
                         int32_t with_shared, hipStream_t cs, void *done_event, bool use_cache);

// moe_stream_prefetch's checks, then its copies (through st->cache when
// use_cache is set and the streamer has one)
static int prefetch_impl(const moe_streamer *st, int32_t layer, const int32_t *expert_ids, int32_t n_ids, int32_t slot,
                         int32_t with_shared, void *copy_stream, void *done_event, bool use_cache)
{
    if (!st) return fail(MOE_ESTATE, "streamer is NULL");
    if (!st->host_arena || st->arena_blobs <= 0) return fail(MOE_ESTATE, "no host arena registered");
    if (with_shared && (!st->host_shared || st->shared_blobs <= 0)) return fail(MOE_ESTATE, "no shared arena registered");
    if (slot != 0 && slot != 1) return fail(MOE_ESTATE, "slot must be 0 or 1 (got %d)", slot);
    if (!st->slab[slot]) return fail(MOE_ESTATE, "slab slot %d is NULL", slot);
    if (layer < 0 || layer >= st->n_layers) return fail(MOE_ESTATE, "layer %d out of range", layer);
    if (st->blob_bytes == 0 || st->n_experts <= 0) return fail(MOE_ESTATE, "streamer shape unset");
    if (n_ids < 0 || n_ids + (with_shared ? 1 : 0) > st->slab_blobs)
        return fail(MOE_ESTATE, "%d ids (+shared) do not fit %d slab blobs", n_ids, st->slab_blobs);
    if (n_ids > 0 && !expert_ids) return fail(MOE_ESTATE, "expert_ids is NULL");
    for (int32_t j = 0; j < n_ids; ++j)
        if (expert_ids[j] < 0 || expert_ids[j] >= st->n_experts)
            return fail(MOE_ESTATE, "expert id %d out of range", expert_ids[j]);
    return stream_copies(st, layer, expert_ids, n_ids, slot, with_shared, (hipStream_t)copy_stream, done_event,
                         use_cache && st->cache);
}

int moe_stream_prefetch(const moe_streamer *st, int32_t layer, const int32_t *expert_ids, int32_t n_ids,
                        int32_t slot, int32_t with_shared, void *copy_stream, void *done_event)
{
    return prefetch_impl(st, layer, expert_ids, n_ids, slot, with_shared, copy_stream, done_event, false);
}

// The copies of moe_stream_prefetch (checked already); with use_cache, the
// routed blobs go through st->cache.
static int stream_copies(const moe_streamer *st, int32_t layer, const int32_t *expert_ids, int32_t n_ids, int32_t slot,
                         int32_t with_shared, hipStream_t cs, void *done_event, bool use_cache)
{
    const uint64_t bb = st->blob_bytes;
    moe_expert_cache *c = use_cache ? st->cache : nullptr;
    CacheView v{};
    if (c) v = cache_view(c->meta, c->n_slots, st->n_layers, st->n_experts);
    // one blob into dst: from the cache on a hit, else from host memory
    // `src` (and then into the least recently used slot, after every earlier
    // copy out of that slot: all copies are on cs)
    auto one = [&](uint8_t *dst, const uint8_t *src, int64_t key) -> int {
        hipError_t e;
        if (c && v.where[key] >= 0) {
            const int32_t s = v.where[key];
            e = hipMemcpyAsync(dst, c->slots + (uint64_t)s * bb, bb, hipMemcpyDeviceToDevice, cs);
            if (e != hipSuccess) return hip_fail(e, "cached expert copy");
            lru_unlink(v, s);
            lru_push_front(v, s);
            ++c->hits;
            return MOE_OK;
        }
        e = hipMemcpyAsync(dst, src, bb, hipMemcpyHostToDevice, cs);
        if (e != hipSuccess) return hip_fail(e, "expert copy");
        if (c) {
            const int32_t s = v.h->tail;
            if (v.tag[s] >= 0) v.where[v.tag[s]] = -1;
            v.tag[s] = key;
            v.where[key] = s;
            lru_unlink(v, s);
            lru_push_front(v, s);
            e = hipMemcpyAsync(c->slots + (uint64_t)s * bb, dst, bb, hipMemcpyDeviceToDevice, cs);
            if (e != hipSuccess) return hip_fail(e, "cache fill copy");
            ++c->misses;
        }
        return MOE_OK;
    };
    const int64_t LE = (int64_t)st->n_layers * st->n_experts;
    for (int32_t j = 0; j < n_ids; ++j) {
        const int64_t key = (int64_t)layer * st->n_experts + expert_ids[j];
        if (int rc = one(st->slab[slot] + (uint64_t)j * bb, st->host_arena + (uint64_t)(key % st->arena_blobs) * bb, key))
            return rc;
    }
    if (with_shared) {
        const int64_t pb = (int64_t)layer % st->shared_blobs;
        if (int rc = one(st->slab[slot] + (uint64_t)(st->slab_blobs - 1) * bb, st->host_shared + (uint64_t)pb * bb,
                         LE + layer))
            return rc;
    }
    if (done_event) {
        hipError_t e = hipEventRecord((hipEvent_t)done_event, cs);
        if (e != hipSuccess) return hip_fail(e, "event record");
    }
    return MOE_OK;
}

int moe_stream_token(const moe_layer_desc *layers, int32_t n_layers, const moe_streamer *st, float *resid, float *x,
                     int32_t *topk_idx, float *topk_w, float *record, int32_t *host_ids, void *workspace,
                     size_t ws_bytes, void *compute_stream, void *copy_stream, void *const *events)
{
    if (!layers || n_layers < 1) return fail(MOE_EINVAL, "no layers");
    if (!st || !st->slab[0] || !st->slab[1]) return fail(MOE_ESTATE, "streamer has no slab");
    if (n_layers > st->n_layers) return fail(MOE_ESTATE, "%d layers but the streamer holds %d", n_layers, st->n_layers);
    if (!host_ids || !events || !topk_idx || !topk_w) return fail(MOE_EINVAL, "NULL host_ids, events or routing buffers");
    for (int i = 0; i < 5; ++i)
        if (!events[i]) return fail(MOE_EINVAL, "event %d is NULL", i);
    const int K = layers[0].top_k;
    const int with_shared = layers[0].n_shared;
    if (st->slab_blobs != K + with_shared) return fail(MOE_ESTATE, "slab holds %d blobs, the layers need %d", st->slab_blobs, K + with_shared);
    for (int32_t l = 0; l < n_layers; ++l) {
        if (layers[l].top_k != K || layers[l].n_shared != with_shared)
            return fail(MOE_EINVAL, "layer %d has another top_k / n_shared", l);
        if (layers[l].experts || layers[l].expert_addr) {
            // a resident layer: its experts (and shared expert) in HBM
            if (int rc = check_desc(&layers[l], 1)) return rc;
            continue;
        }
        moe_layer_desc d = layers[l];
        d.slab = st->slab[0];
        if (int rc = check_desc(&d, 1)) return rc;
        if (d.blob_bytes != st->blob_bytes || d.n_experts != st->n_experts)
            return fail(MOE_ESTATE, "layer %d does not match the streamer's blob size / expert count", l);
    }
    if (int rc = check_ws(&layers[0], 1, workspace, ws_bytes)) return rc;
    if (record && !aligned16(record)) return fail(MOE_EINVAL, "record not 16-byte aligned");
    const size_t D = (size_t)layers[0].hidden;
    for (int32_t l = 1; l < n_layers; ++l)
        if ((size_t)layers[l].hidden != D) return fail(MOE_EINVAL, "layer %d has another hidden size", l);
    if (const moe_expert_cache *c = st->cache) {
        if (!c->slots || !c->meta || c->n_slots <= 0) return fail(MOE_ESTATE, "expert cache without slots or meta block");
        const CacheHead *h = static_cast<const CacheHead *>(c->meta);
        if (h->n_layers != st->n_layers || h->n_experts != st->n_experts || h->n_slots != c->n_slots)
            return fail(MOE_ESTATE, "expert cache not reset for this streamer (moe_expert_cache_reset)");
    }
    hipStream_t cs = (hipStream_t)compute_stream, ps = (hipStream_t)copy_stream;
    hipEvent_t route_done = (hipEvent_t)events[0];
    hipEvent_t copy_done[2] = {(hipEvent_t)events[1], (hipEvent_t)events[2]};
    hipEvent_t compute_done[2] = {(hipEvent_t)events[3], (hipEvent_t)events[4]};
    hipError_t e;
    // (resid, x) entering layer l (l == n_layers: the output) into record
    auto rec = [&](int32_t l) -> int {
        if (!record) return MOE_OK;
        float *rl = record + (size_t)l * 2 * D;
        if ((e = hipMemcpyAsync(rl, resid, D * 4, hipMemcpyDeviceToDevice, cs)) != hipSuccess ||
            (e = hipMemcpyAsync(rl + D, x, D * 4, hipMemcpyDeviceToDevice, cs)) != hipSuccess)
            return hip_fail(e, "record copy");
        return MOE_OK;
    };
    int32_t j = 0;  // streamed layers so far: layer l, the j-th streamed one, uses slot j mod 2
    for (int32_t l = 0; l < n_layers; ++l) {
        int32_t *idx = topk_idx + (size_t)l * K;
        float *w = topk_w + (size_t)l * K;
        if (int rc = rec(l)) return rc;
        if (layers[l].experts || layers[l].expert_addr) {
            // resident: routing and experts stay on the device, no host wait
            int rc = moe_layer_step(&layers[l], resid, x, 1, idx, w, workspace, ws_bytes, compute_stream);
            if (rc) return rc;
            continue;
        }
        const int s = j & 1;
        moe_layer_desc d = layers[l];
        d.slab = st->slab[s];
        // 1. routing, and its selections to the host (the one device->host wait per layer)
        int rc = moe_route(&d, x, 1, idx, w, nullptr, workspace, ws_bytes, compute_stream);
        if (rc) return rc;
        if ((e = hipMemcpyAsync(host_ids, idx, (size_t)K * 4, hipMemcpyDeviceToHost, cs)) != hipSuccess)
            return hip_fail(e, "selection copy");
        if ((e = hipEventRecord(route_done, cs)) != hipSuccess) return hip_fail(e, "event record");
        if ((e = hipEventSynchronize(route_done)) != hipSuccess) return hip_fail(e, "selection wait");
        if (moe_expert_cache *c = st->cache) {
            // this token's selection: the next token's guess for layer l
            int32_t *pred = cache_view(c->meta, c->n_slots, st->n_layers, st->n_experts).pred + (size_t)l * moe::kMaxTopK;
            for (int k = 0; k < K; ++k) pred[k] = host_ids[k];
        }
        // 2. the selected experts into slot s, after the kernel that last read it (streamed layer j-2)
        if (j >= 2 && (e = hipStreamWaitEvent(ps, compute_done[s], 0)) != hipSuccess) return hip_fail(e, "wait");
        rc = prefetch_impl(st, l, host_ids, K, s, j == 0 ? with_shared : 0, copy_stream, copy_done[s], true);
        if (rc) return rc;
        // 3. the layer itself once its weights have landed, under the routing
        // the copies followed (idx, w: read by the streamed step, not recomputed)
        if ((e = hipStreamWaitEvent(cs, copy_done[s], 0)) != hipSuccess) return hip_fail(e, "wait");
        rc = moe_layer_step(&d, resid, x, 1, idx, w, workspace, ws_bytes, compute_stream);
        if (rc) return rc;
        if ((e = hipEventRecord(compute_done[s], cs)) != hipSuccess) return hip_fail(e, "event record");
        // 4. the next streamed layer's shared expert needs no routing: queue
        // it behind this layer's copies, into the slot that layer will use
        int32_t ln = l + 1;
        while (ln < n_layers && (layers[ln].experts || layers[ln].expert_addr)) ++ln;
        if (with_shared && ln < n_layers) {
            const int s1 = (j + 1) & 1;
            if (j >= 1 && (e = hipStreamWaitEvent(ps, compute_done[s1], 0)) != hipSuccess) return hip_fail(e, "wait");
            rc = prefetch_impl(st, ln, nullptr, 0, s1, 1, copy_stream, nullptr, true);
            if (rc) return rc;
        }
        // 5. the guess for the next streamed layer (the previous token's
        // selection there) into the cache, behind every copy above
        if (moe_expert_cache *c = st->cache; c && c->speculate && ln < n_layers) {
            CacheView v = cache_view(c->meta, c->n_slots, st->n_layers, st->n_experts);
            const uint64_t bb = st->blob_bytes;
            for (int k = 0; k < K; ++k) {
                const int32_t pe = v.pred[(size_t)ln * moe::kMaxTopK + k];
                if (pe < 0 || pe >= st->n_experts) continue;
                const int64_t key = (int64_t)ln * st->n_experts + pe;
                if (v.where[key] >= 0) continue;
                const int32_t slot_c = v.h->tail;
                if (v.tag[slot_c] >= 0) v.where[v.tag[slot_c]] = -1;
                v.tag[slot_c] = key;
                v.where[key] = slot_c;
                lru_unlink(v, slot_c);
                lru_push_front(v, slot_c);
                if ((e = hipMemcpyAsync(c->slots + (uint64_t)slot_c * bb, st->host_arena + (uint64_t)(key % st->arena_blobs) * bb,
                                        bb, hipMemcpyHostToDevice, ps)) != hipSuccess)
                    return hip_fail(e, "speculative copy");
                ++c->spec_fills;
            }
        }
        ++j;
    }
    return rec(n_layers);
}

#ifdef MOE_STACK_PROBE
// Timeline builds only (not part of the C ABI of moe.h): the device buffer
// of [n_layers][grid][8][kProbePoints] uint64 stamps that the next stack
// launches fill, or NULL.
int moe_probe_set(void *buf)
{
    g_probe = static_cast<uint64_t *>(buf);
    return MOE_OK;
}
#endif

int moe_host_alloc(size_t bytes, void **out)
{
    if (!out) return fail(MOE_EINVAL, "out is NULL");
    *out = nullptr;
    if (bytes == 0) return fail(MOE_EINVAL, "zero-byte host arena");
    void *p = nullptr;
    hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "pinned host allocation");
    *out = p;
    return MOE_OK;
}

int moe_host_free(void *p)
{
    if (!p) return MOE_OK;
    hipError_t e = hipHostFree(p);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "pinned host free");
}

}  // extern "C"
