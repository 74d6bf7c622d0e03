// Quantization of a list of layers (a transformer block's linears) with the phases of
// different layers overlapped.
//
// GPTQ summary page, the statement of the procedure: the model is quantized one layer
// at a time, each layer from its own calibration inputs, and layers that read the same
// inputs (a block's q, k and v; gate and up) need only one H = 2 X X^T and one
// factorization between them.  Every layer goes through the same kernels as the
// one-call-per-phase entry points (Hessian, factorization of the damped inverse,
// blocked sweep), so its codes, scales and zeros are bit-identical to theirs.
//
// Schedule.  Consecutive layers with the same inputs form a group.  Groups are started
// widest first (the factorization grows as d_col^3, so the longest chain starts first
// and the rest fits beside it; ties keep the caller's order); a layer's result does
// not depend on the order.  With a caller-owned context, the groups' Hessians run one
// after another on the context's Hessian stream; the k-th started group's
// factorization and its layers' sweeps run on slot stream k mod n_slots, each slot with
// its own H, U and workspaces and its own auxiliary stream for the factorization's
// inverse.  So the next group's Hessian (matrix-core bound) runs beside the current
// groups' factorizations (latency-bound chains of 64-column steps) and sweeps, and the
// factorizations of up to n_slots groups overlap one another.  A group's Hessian waits
// until its slot's previous group has finished with H and U.  Events order the whole
// call after the work already on the caller's stream, and the caller's stream after
// it.  Without a context every group runs on the caller's stream, one after another.

#include <algorithm>
#include <new>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace gptq {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__global__ void zero_f32_kernel(float* p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

void zero_f32(float* p, int64_t n, hipStream_t s) {
    const int64_t blocks = (n + 255) / 256;
    zero_f32_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, s>>>(p, n);
}

static bool same_inputs(const gptq_layer& a, const gptq_layer& b) {
    return a.X == b.X && a.x_dtype == b.x_dtype && a.n_tokens == b.n_tokens && a.ldx == b.ldx && a.d_col == b.d_col;
}

// Workspace: n_slots x (H, U, factorization workspace, sweep workspace), each sized for
// the largest layer, then one Hessian workspace (the Hessians run one at a time).
struct LayersPlan {
    size_t h_bytes = 0, p_bytes = 0, q_bytes = 0, hw_bytes = 0, slot_bytes = 0, total = 0;
};

static LayersPlan layers_plan(const gptq_layer* L, int n, int n_slots) {
    LayersPlan p;
    for (int i = 0; i < n; ++i) {
        const int64_t d = L[i].d_col;
        p.h_bytes = std::max(p.h_bytes, align256((size_t)d * d * sizeof(float)));
        p.p_bytes = std::max(p.p_bytes, align256(prep_ws_bytes(d)));
        p.q_bytes = std::max(p.q_bytes, align256(quant_ws_bytes(L[i].d_row, d)));
        p.hw_bytes = std::max(p.hw_bytes, align256(hessian_ws_bytes(L[i].n_tokens, d)));
    }
    p.slot_bytes = 2 * p.h_bytes + p.p_bytes + p.q_bytes;
    p.total = n > 0 ? (size_t)n_slots * p.slot_bytes + p.hw_bytes : 0;
    return p;
}

size_t layers_ws_bytes(const gptq_layer* L, int n, int n_slots) { return layers_plan(L, n, n_slots).total; }

gptq_status layers_launch(const gptq_layer* L, int n, float percdamp, const gptq_params& prm, int n_slots,
                          void* ws, size_t ws_bytes, int32_t* info, gptq_context* ctx, hipStream_t caller) {
    const LayersPlan plan = layers_plan(L, n, n_slots);
    if (ws == nullptr || ws_bytes < plan.total || (reinterpret_cast<uintptr_t>(ws) & 255)) return GPTQ_ERR_WORKSPACE;
    gptq_status st;
    char* base = reinterpret_cast<char*>(ws);
    void* hws = base + (size_t)n_slots * plan.slot_bytes;
    auto slot_ptr = [&](int s, size_t off) { return base + (size_t)s * plan.slot_bytes + off; };

    fill_i32(info, 2 * n, 0, caller);
    GPTQ_LAUNCH_CHECK();
    // Without a context everything runs on the caller's stream, group after group.
    const hipStream_t hs = ctx ? ctx->hs : caller;
    if (ctx) {
        if (hipEventRecord(ctx->start, caller) != hipSuccess || hipStreamWaitEvent(hs, ctx->start, 0) != hipSuccess)
            return GPTQ_ERR_HIP;
        for (int s = 0; s < n_slots; ++s)
            if (hipStreamWaitEvent(ctx->slot[s].s, ctx->start, 0) != hipSuccess) return GPTQ_ERR_HIP;
    }

    // groups [first, end) of consecutive layers with the same inputs, widest first
    std::vector<std::pair<int, int>> grp;
    for (int i = 0; i < n;) {
        int j = i + 1;
        while (j < n && same_inputs(L[i], L[j])) ++j;
        grp.push_back({i, j});
        i = j;
    }
    std::stable_sort(grp.begin(), grp.end(), [&](const std::pair<int, int>& a, const std::pair<int, int>& b) {
        return L[a.first].d_col > L[b.first].d_col;
    });
    int groups = 0;
    for (const auto& gr : grp) {
        const int i = gr.first, j = gr.second;
        const int s = groups % n_slots;
        gptq_context::Slot* sl = ctx ? &ctx->slot[s] : nullptr;
        const hipStream_t ss = sl ? sl->s : caller;
        const int64_t d = L[i].d_col;
        float* H = reinterpret_cast<float*>(slot_ptr(s, 0));
        float* U = reinterpret_cast<float*>(slot_ptr(s, plan.h_bytes));
        void* pws = slot_ptr(s, 2 * plan.h_bytes);
        void* qws = slot_ptr(s, 2 * plan.h_bytes + plan.p_bytes);
        // H and U of this slot are free once its previous group's sweeps are done
        if (sl && groups >= n_slots && hipStreamWaitEvent(hs, sl->free, 0) != hipSuccess) return GPTQ_ERR_HIP;
        zero_f32(H, d * d, hs);
        GPTQ_LAUNCH_CHECK();
        if ((st = hessian_launch(H, L[i].X, L[i].x_dtype, L[i].n_tokens, d, L[i].ldx, hws, plan.hw_bytes, hs)) !=
            GPTQ_OK)
            return st;
        if (sl && (hipEventRecord(sl->hdone, hs) != hipSuccess || hipStreamWaitEvent(ss, sl->hdone, 0) != hipSuccess))
            return GPTQ_ERR_HIP;
        if ((st = prep_launch(H, U, d, percdamp, pws, plan.p_bytes, info + 2 * i, ss, sl ? &sl->aux : nullptr)) !=
            GPTQ_OK)
            return st;
        for (int l = i; l < j; ++l)
            if ((st = quant_launch(L[l].W, L[l].w_dtype, L[l].d_row, d, U, prm, L[l].codes, L[l].scales_f16,
                                   L[l].zeros_f16, qws, plan.q_bytes, info + 2 * l + 1, ss)) != GPTQ_OK)
                return st;
        if (sl && hipEventRecord(sl->free, ss) != hipSuccess) return GPTQ_ERR_HIP;
        ++groups;
    }
    if (ctx) {
        // the caller's stream resumes after every slot and the Hessian stream
        for (int s = 0; s < n_slots && s < groups; ++s)
            if (hipStreamWaitEvent(caller, ctx->slot[s].free, 0) != hipSuccess) return GPTQ_ERR_HIP;
        if (hipEventRecord(ctx->hs_done, hs) != hipSuccess || hipStreamWaitEvent(caller, ctx->hs_done, 0) != hipSuccess)
            return GPTQ_ERR_HIP;
    }
    return GPTQ_OK;
}

// ---------------------------------------------------------------- the context

static void context_release(gptq_context* c) {
    auto es = [](hipEvent_t& e) { if (e) (void)hipEventDestroy(e); e = nullptr; };
    auto ss = [](hipStream_t& s) { if (s) (void)hipStreamDestroy(s); s = nullptr; };
    ss(c->prep.s); es(c->prep.fork); es(c->prep.join);
    ss(c->hs); es(c->start); es(c->hs_done);
    for (auto& sl : c->slot) {
        ss(sl.s); ss(sl.aux.s); es(sl.aux.fork); es(sl.aux.join); es(sl.hdone); es(sl.free);
    }
}

gptq_status context_create(int n_slots, gptq_context** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GPTQ_ERR_HIP;
    gptq_context* c = new (std::nothrow) gptq_context;
    if (c == nullptr) return GPTQ_ERR_HIP;
    c->device = dev;
    c->n_slots = n_slots;
    // every stream at the default priority, non-blocking with respect to the null stream
    auto ev = [](hipEvent_t* e) { return hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess; };
    auto st = [](hipStream_t* s) { return hipStreamCreateWithFlags(s, hipStreamNonBlocking) == hipSuccess; };
    bool ok = st(&c->prep.s) && ev(&c->prep.fork) && ev(&c->prep.join) && st(&c->hs) && ev(&c->start) &&
              ev(&c->hs_done);
    for (int s = 0; ok && s < n_slots; ++s) {
        gptq_context::Slot& sl = c->slot[s];
        ok = st(&sl.s) && st(&sl.aux.s) && ev(&sl.aux.fork) && ev(&sl.aux.join) && ev(&sl.hdone) && ev(&sl.free);
    }
    if (!ok) {
        context_release(c);
        delete c;
        return GPTQ_ERR_HIP;
    }
    *out = c;
    return GPTQ_OK;
}

gptq_status context_destroy(gptq_context* c) {
    if (c == nullptr) return GPTQ_OK;
    int cur = -1;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != c->device;
    if (switch_dev && hipSetDevice(c->device) != hipSuccess) return GPTQ_ERR_HIP;
    // the work already queued on the context's streams completes first
    auto drain = [](hipStream_t s) { if (s) (void)hipStreamSynchronize(s); };
    drain(c->prep.s);
    drain(c->hs);
    for (auto& sl : c->slot) { drain(sl.s); drain(sl.aux.s); }
    context_release(c);
    if (switch_dev) (void)hipSetDevice(cur);
    delete c;
    return GPTQ_OK;
}

}  // namespace gptq
