// Host-side launchers of the GPTQ kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gptq.h"

namespace gptq {

void fill_i32(int32_t* p, int n, int v, hipStream_t s);

size_t hessian_ws_bytes(int64_t n_tokens, int64_t d_col);
gptq_status hessian_launch(float* H, const void* X, gptq_dtype dt, int64_t n, int64_t d, int64_t ldx,
                           void* ws, size_t ws_bytes, hipStream_t stream);

// Auxiliary stream of the factorization (the inverse's row blocks run on it beside the
// chain) with the events that fork it from and join it to the caller's stream.
// Bound of a factorization step's wait for the next diagonal block, in polls of about
// 128 clocks (1 << 25: about 2 s at 2 GHz; the factorization of one block takes
// microseconds).
constexpr int32_t PREP_WAIT_POLLS = 1 << 25;
struct PrepAux {
    hipStream_t s = nullptr; hipEvent_t fork = nullptr, join = nullptr;
    int32_t wait_polls = PREP_WAIT_POLLS;
};

size_t prep_ws_bytes(int64_t d_col);
// aux: an auxiliary stream and its events, used by this call alone (from a caller-owned
// context); nullptr: every kernel on `stream`.
gptq_status prep_launch(const float* H, float* U, int64_t d, float percdamp, void* ws, size_t ws_bytes,
                        int32_t* info, hipStream_t stream, const PrepAux* aux);

void zero_f32(float* p, int64_t n, hipStream_t s);

size_t quant_ws_bytes(int64_t d_row, int64_t d_col);
gptq_status quant_launch(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                         const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                         void* ws, size_t ws_bytes, int32_t* info, hipStream_t stream);

// gptq_quantize_layer with the library's own per-device scratch in place of a workspace
gptq_status quant_launch_noalloc(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                                 const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                 int32_t* info, hipStream_t stream);

size_t layers_ws_bytes(const gptq_layer* layers, int n, int n_slots);
gptq_status layers_launch(const gptq_layer* layers, int n, float percdamp, const gptq_params& p, int n_slots,
                          void* ws, size_t ws_bytes, int32_t* info, gptq_context* ctx, hipStream_t stream);
gptq_status context_create(int n_slots, gptq_context** out);
gptq_status context_destroy(gptq_context* ctx);

constexpr int OBQ_MAXD = 2048;   // widest row the OBQ kernel keeps in LDS
// Most rows of a quantizer call: the trailing-update launches put the 128-row tiles of W
// on the grid's y extent (at most 65535).
constexpr int64_t QUANT_MAX_ROWS = (int64_t)65535 * 128;
// Most tokens of a quantized-linear call: its matrix-core launches put tiles of up to 64
// tokens on the grid's y extent.
constexpr int64_t LINEAR_MAX_TOKENS = (int64_t)65535 * 64;
size_t obq_ws_bytes(int64_t d_row, int64_t d_col);
gptq_status obq_launch(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                       const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros, void* ws,
                       size_t ws_bytes, int32_t* info, hipStream_t stream);

gptq_status dequant_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t d_row,
                           int64_t d_col, int bits, int group_size, void* out, gptq_dtype out_dtype,
                           hipStream_t stream, bool fp4 = false);

gptq_status linear_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t d_row,
                          int64_t d_col, int bits, int group_size, const void* x, gptq_dtype x_dtype, int64_t n_tok,
                          int64_t ldx, void* y, gptq_dtype y_dtype, hipStream_t stream);

}  // namespace gptq

// The caller-owned execution context (opaque in the C header): the streams and events
// that let one call overlap its own phases.  Made by gptq_context_create on one device,
// freed by gptq_context_destroy; the library keeps no other state between calls.
struct gptq_context {
    int device = -1;
    int n_slots = 0;
    gptq::PrepAux prep;                          // gptq_prepare_hinv's auxiliary stream
    hipStream_t hs = nullptr;                    // gptq_quantize_layers: the Hessians
    hipEvent_t start = nullptr, hs_done = nullptr;
    struct Slot {
        hipStream_t s = nullptr;                 // factorization and sweeps of a group
        gptq::PrepAux aux;                       // that factorization's auxiliary stream
        hipEvent_t hdone = nullptr, free = nullptr;
    } slot[GPTQ_LAYERS_MAX_SLOTS];
};
