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
struct PrepAux { hipStream_t s = nullptr; hipEvent_t fork = nullptr, join = nullptr; };

size_t prep_ws_bytes(int64_t d_col);
// own_aux: the caller's auxiliary stream and events, used by this call alone (the caller
// serializes calls that share them); nullptr: the device's own, under a lock.
gptq_status prep_launch(const float* H, float* U, int64_t d, float percdamp, void* ws, size_t ws_bytes,
                        int32_t* info, hipStream_t stream, PrepAux* own_aux = nullptr);

void zero_f32(float* p, int64_t n, hipStream_t s);

size_t quant_ws_bytes(int64_t d_row, int64_t d_col);
gptq_status quant_launch(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                         const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                         void* ws, size_t ws_bytes, int32_t* info, hipStream_t stream);

size_t layers_ws_bytes(const gptq_layer* layers, int n, int n_slots);
gptq_status layers_launch(const gptq_layer* layers, int n, float percdamp, const gptq_params& p, int n_slots,
                          void* ws, size_t ws_bytes, int32_t* info, hipStream_t stream);

constexpr int OBQ_MAXD = 2048;   // widest row the OBQ kernel keeps in LDS
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
