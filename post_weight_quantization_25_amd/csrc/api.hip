// C ABI of the GPTQ layer quantizer: argument validation, workspace sizing and
// dispatch to the gfx950 kernels.  See include/gptq.h for the contract.

#include "common.h"
#include "kernels.h"

using namespace gptq;

static bool valid_dtype(gptq_dtype t) { return t == GPTQ_F32 || t == GPTQ_BF16 || t == GPTQ_F16; }

static gptq_status check_params(const gptq_params* p, int64_t d_col) {
    if (p == nullptr) return GPTQ_ERR_INVALID_ARG;
    if (p->bits != 3 && p->bits != 4 && p->bits != 8) return GPTQ_ERR_UNSUPPORTED;
    if (p->block_size != 128) return GPTQ_ERR_UNSUPPORTED;
    if (p->sym < 0 || p->sym > 3) return GPTQ_ERR_INVALID_ARG;
    if (p->sym >= 2 && p->bits != 4) return GPTQ_ERR_UNSUPPORTED;   // E2M1 is a 4-bit grid
    if (p->group_size < -1) return GPTQ_ERR_INVALID_ARG;   // -1: per tensor, 0: per row
    if (p->group_size > 0) {
        if (p->block_size % p->group_size != 0 || d_col % p->group_size != 0) return GPTQ_ERR_INVALID_ARG;
        if (p->group_size != 32 && p->group_size != 64 && p->group_size != 128) return GPTQ_ERR_UNSUPPORTED;
    }
    if (p->bits <= 4 && (d_col & 1)) return GPTQ_ERR_INVALID_ARG;
    if (p->bits == 3 && (d_col & 7)) return GPTQ_ERR_INVALID_ARG;   // 3-bit rows: whole 8-code groups
    return GPTQ_OK;
}

#pragma GCC visibility push(default)
extern "C" {

size_t gptq_hessian_workspace_size(int64_t n_tokens, int64_t d_col) {
    if (n_tokens <= 0 || d_col <= 0) return 0;
    return hessian_ws_bytes(n_tokens, d_col);
}

gptq_status gptq_hessian_accumulate(float* H, const void* X, gptq_dtype x_dtype, int64_t n_tokens, int64_t d_col,
                                    int64_t ldx, void* ws, size_t ws_bytes, void* stream) {
    if (n_tokens < 0 || d_col < 0) return GPTQ_ERR_INVALID_ARG;
    if (!valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
    if (n_tokens == 0 || d_col == 0) return GPTQ_OK;
    if (H == nullptr || X == nullptr || ldx < d_col) return GPTQ_ERR_INVALID_ARG;
    if (d_col > 65536) return GPTQ_ERR_UNSUPPORTED;
    return hessian_launch(H, X, x_dtype, n_tokens, d_col, ldx, ws, ws_bytes, (hipStream_t)stream);
}

size_t gptq_prepare_hinv_workspace_size(int64_t d_col) {
    if (d_col <= 0) return 0;
    return prep_ws_bytes(d_col);
}

size_t gptq_prepare_hinv_workspace(int64_t d_col, gptq_dtype u_dtype) {
    return u_dtype == GPTQ_F32 ? gptq_prepare_hinv_workspace_size(d_col) : 0;
}

gptq_status gptq_context_create(int32_t n_slots, gptq_context** ctx) {
    if (ctx == nullptr || n_slots < 1 || n_slots > GPTQ_LAYERS_MAX_SLOTS) return GPTQ_ERR_INVALID_ARG;
    return context_create(n_slots, ctx);
}

gptq_status gptq_context_destroy(gptq_context* ctx) { return context_destroy(ctx); }

gptq_status gptq_context_set_wait_limit(gptq_context* ctx, int32_t polls) {
    if (ctx == nullptr || polls < 0) return GPTQ_ERR_INVALID_ARG;
    ctx->prep.wait_polls = polls;
    for (auto& sl : ctx->slot) sl.aux.wait_polls = polls;
    return GPTQ_OK;
}

// A context serves the device it was made on.
static gptq_status check_context(const gptq_context* ctx) {
    if (ctx == nullptr) return GPTQ_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GPTQ_ERR_HIP;
    return dev == ctx->device ? GPTQ_OK : GPTQ_ERR_INVALID_ARG;
}

gptq_status gptq_prepare_hinv(const float* H, float* U, int64_t d_col, float percdamp, void* ws, size_t ws_bytes,
                              int32_t* info, gptq_context* ctx, void* stream) {
    if (d_col < 0 || !(percdamp >= 0.f)) return GPTQ_ERR_INVALID_ARG;
    if (d_col == 0) return GPTQ_OK;
    if (H == nullptr || U == nullptr || info == nullptr) return GPTQ_ERR_INVALID_ARG;
    if (d_col > 65535) return GPTQ_ERR_UNSUPPORTED;
    if (ws == nullptr || ws_bytes < prep_ws_bytes(d_col)) return GPTQ_ERR_WORKSPACE;
    const gptq_status st = check_context(ctx);
    if (st != GPTQ_OK) return st;
    return prep_launch(H, U, d_col, percdamp, ws, ws_bytes, info, (hipStream_t)stream, ctx ? &ctx->prep : nullptr);
}

size_t gptq_quantize_workspace_size(int64_t d_row, int64_t d_col, const gptq_params* p) {
    (void)p;
    if (d_row <= 0 || d_col <= 0) return 0;
    return quant_ws_bytes(d_row, d_col);
}

size_t gptq_quantize_workspace(int64_t d_row, int64_t d_col, const gptq_params* p) {
    return gptq_quantize_workspace_size(d_row, d_col, p);
}

gptq_status gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                                const gptq_params* p, uint8_t* codes, uint16_t* scales_f16, uint16_t* zeros_f16,
                                void* ws, size_t ws_bytes, int32_t* info, void* stream) {
    if (d_row < 0 || d_col < 0 || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_params(p, d_col);
    if (st != GPTQ_OK) return st;
    if (d_row == 0 || d_col == 0) return GPTQ_OK;
    if (!W || !U || !codes || !scales_f16 || !zeros_f16 || !info) return GPTQ_ERR_INVALID_ARG;
    if (d_row > QUANT_MAX_ROWS || d_col > 65535) return GPTQ_ERR_UNSUPPORTED;
    return quant_launch(W, w_dtype, d_row, d_col, U, *p, codes, scales_f16, zeros_f16, ws, ws_bytes, info,
                        (hipStream_t)stream);
}

gptq_status gptq_quantize_layer_noalloc(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col,
                                        const float* U, const gptq_params* p, uint8_t* codes, uint16_t* scales_f16,
                                        uint16_t* zeros_f16, int32_t* info, void* stream) {
    if (d_row < 0 || d_col < 0 || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_params(p, d_col);
    if (st != GPTQ_OK) return st;
    if (d_row == 0 || d_col == 0) return GPTQ_OK;
    if (!W || !U || !codes || !scales_f16 || !zeros_f16 || !info) return GPTQ_ERR_INVALID_ARG;
    if (d_row > QUANT_MAX_ROWS || d_col > 65535) return GPTQ_ERR_UNSUPPORTED;
    if (quant_ws_bytes(d_row, d_col) > GPTQ_NOALLOC_SCRATCH_BYTES) return GPTQ_ERR_UNSUPPORTED;
    return quant_launch_noalloc(W, w_dtype, d_row, d_col, U, *p, codes, scales_f16, zeros_f16, info,
                                (hipStream_t)stream);
}

// p == nullptr: shapes only (the workspace size), no settings and no pointers checked.
static gptq_status check_layers(const gptq_layer* L, int32_t n, const gptq_params* p, int32_t n_slots) {
    if (n < 0 || (n > 0 && L == nullptr)) return GPTQ_ERR_INVALID_ARG;
    if (n_slots < 1 || n_slots > GPTQ_LAYERS_MAX_SLOTS) return GPTQ_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
        const gptq_layer& l = L[i];
        if (l.n_tokens < 1 || l.d_row < 1 || l.d_col < 1 || l.ldx < l.d_col) return GPTQ_ERR_INVALID_ARG;
        if (!valid_dtype(l.x_dtype) || !valid_dtype(l.w_dtype)) return GPTQ_ERR_INVALID_ARG;
        if (p) {
            if (!l.X || !l.W || !l.codes || !l.scales_f16 || !l.zeros_f16) return GPTQ_ERR_INVALID_ARG;
            const gptq_status st = check_params(p, l.d_col);
            if (st != GPTQ_OK) return st;
        }
        if (l.d_row > QUANT_MAX_ROWS || l.d_col > 65535) return GPTQ_ERR_UNSUPPORTED;
    }
    return GPTQ_OK;
}

size_t gptq_quantize_layers_workspace_size(const gptq_layer* layers, int32_t n_layers, int32_t n_slots) {
    if (check_layers(layers, n_layers, nullptr, n_slots) != GPTQ_OK || n_layers == 0) return 0;
    return layers_ws_bytes(layers, n_layers, n_slots);
}

gptq_status gptq_quantize_layers(const gptq_layer* layers, int32_t n_layers, float percdamp, const gptq_params* p,
                                 int32_t n_slots, void* ws, size_t ws_bytes, int32_t* info, gptq_context* ctx,
                                 void* stream) {
    if (p == nullptr || !(percdamp >= 0.f)) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_layers(layers, n_layers, p, n_slots);
    if (st != GPTQ_OK) return st;
    if (ctx && n_slots > ctx->n_slots) return GPTQ_ERR_INVALID_ARG;
    if (n_layers == 0) return GPTQ_OK;
    if (info == nullptr) return GPTQ_ERR_INVALID_ARG;
    if ((st = check_context(ctx)) != GPTQ_OK) return st;
    return layers_launch(layers, n_layers, percdamp, *p, n_slots, ws, ws_bytes, info, ctx, (hipStream_t)stream);
}

size_t gptq_obq_workspace_size(int64_t d_row, int64_t d_col) {
    if (d_row <= 0 || d_col <= 0 || d_col > OBQ_MAXD) return 0;
    return obq_ws_bytes(d_row, d_col);
}

gptq_status gptq_obq_layer(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                           const gptq_params* p, uint8_t* codes, uint16_t* scales_f16, uint16_t* zeros_f16,
                           void* ws, size_t ws_bytes, int32_t* info, void* stream) {
    if (d_row < 0 || d_col < 0 || !valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_params(p, d_col);
    if (st != GPTQ_OK) return st;
    if (p->group_size != 0) return GPTQ_ERR_UNSUPPORTED;   // one group per row
    if (p->sym >= 2) return GPTQ_ERR_UNSUPPORTED;          // integer grids only (no E2M1)
    if (d_row == 0 || d_col == 0) return GPTQ_OK;
    if (!W || !U || !codes || !scales_f16 || !zeros_f16 || !info) return GPTQ_ERR_INVALID_ARG;
    if (d_col > OBQ_MAXD || d_row > 2147483647LL / 64) return GPTQ_ERR_UNSUPPORTED;
    return obq_launch(W, w_dtype, d_row, d_col, U, *p, codes, scales_f16, zeros_f16, ws, ws_bytes, info,
                      (hipStream_t)stream);
}

gptq_status gptq_dequantize(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* zeros_f16,
                            int64_t d_row, int64_t d_col, int32_t bits, int32_t group_size, void* W_out,
                            gptq_dtype out_dtype, void* stream) {
    if (group_size == -1) group_size = 0;   // per tensor is stored as one (equal) group per row
    if (d_row < 0 || d_col < 0 || !valid_dtype(out_dtype) || group_size < 0) return GPTQ_ERR_INVALID_ARG;
    if (bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_UNSUPPORTED;
    if (group_size > 0 && d_col % group_size != 0) return GPTQ_ERR_INVALID_ARG;
    if (bits <= 4 && (d_col & 1)) return GPTQ_ERR_INVALID_ARG;
    if (bits == 3 && (d_col & 7)) return GPTQ_ERR_INVALID_ARG;
    if (d_row == 0 || d_col == 0) return GPTQ_OK;
    if (!codes || !scales_f16 || !zeros_f16 || !W_out) return GPTQ_ERR_INVALID_ARG;
    if (d_col > 2147483647LL) return GPTQ_ERR_UNSUPPORTED;   // group counts are 32-bit
    return dequant_launch(codes, scales_f16, zeros_f16, d_row, d_col, bits, group_size, W_out, out_dtype,
                          (hipStream_t)stream);
}

gptq_status gptq_dequantize_e2m1(const uint8_t* codes, const uint16_t* scales_f16, int64_t d_row, int64_t d_col,
                                 int32_t group_size, void* W_out, gptq_dtype out_dtype, void* stream) {
    if (group_size == -1) group_size = 0;
    if (d_row < 0 || d_col < 0 || !valid_dtype(out_dtype) || group_size < 0 || (d_col & 1)) return GPTQ_ERR_INVALID_ARG;
    if (group_size > 0 && d_col % group_size != 0) return GPTQ_ERR_INVALID_ARG;
    if (d_row == 0 || d_col == 0) return GPTQ_OK;
    if (!codes || !scales_f16 || !W_out) return GPTQ_ERR_INVALID_ARG;
    if (d_col > 2147483647LL) return GPTQ_ERR_UNSUPPORTED;   // group counts are 32-bit
    // the zero array is not read on this grid: pass the scales in its place
    return dequant_launch(codes, scales_f16, scales_f16, d_row, d_col, 4, group_size, W_out, out_dtype,
                          (hipStream_t)stream, true);
}

gptq_status gptq_quantized_linear(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* zeros_f16,
                                  int64_t d_row, int64_t d_col, int32_t bits, int32_t group_size, const void* x,
                                  gptq_dtype x_dtype, int64_t n_tokens, int64_t ldx, void* y, gptq_dtype y_dtype,
                                  void* stream) {
    if (group_size == -1) group_size = 0;   // per tensor is stored as one (equal) group per row
    if (d_row < 0 || d_col < 0 || n_tokens < 0 || group_size < 0) return GPTQ_ERR_INVALID_ARG;
    if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return GPTQ_ERR_INVALID_ARG;
    if (bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_UNSUPPORTED;
    if (group_size > 0 && d_col % group_size != 0) return GPTQ_ERR_INVALID_ARG;
    if (bits <= 4 && (d_col & 1)) return GPTQ_ERR_INVALID_ARG;
    if (bits == 3 && (d_col & 7)) return GPTQ_ERR_INVALID_ARG;
    if (d_row == 0 || d_col == 0 || n_tokens == 0) return GPTQ_OK;
    if (!codes || !scales_f16 || !zeros_f16 || !x || !y || ldx < d_col) return GPTQ_ERR_INVALID_ARG;
    if (d_row > 2147483647LL / 64 || d_col > 2147483647LL / 64 || n_tokens > LINEAR_MAX_TOKENS)
        return GPTQ_ERR_UNSUPPORTED;
    return linear_launch(codes, scales_f16, zeros_f16, d_row, d_col, bits, group_size, x, x_dtype, n_tokens, ldx, y,
                         y_dtype, (hipStream_t)stream);
}

const char* gptq_status_string(gptq_status s) {
    switch (s) {
        case GPTQ_OK: return "ok";
        case GPTQ_ERR_INVALID_ARG: return "invalid argument";
        case GPTQ_ERR_UNSUPPORTED: return "unsupported setting or size";
        case GPTQ_ERR_WORKSPACE: return "workspace missing or too small";
        case GPTQ_ERR_HIP: return "HIP runtime error";
        case GPTQ_ERR_NOT_PD: return "damped Hessian is not positive definite";
        case GPTQ_ERR_NONFINITE: return "non-finite input or scale outside the fp16 normal range";
    }
    return "unknown status";
}

}  // extern "C"
#pragma GCC visibility pop
