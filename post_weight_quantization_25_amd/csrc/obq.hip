// OBQ: every row quantized on its own, its weights in a greedy order, with the inverse
// Hessian of its remaining weights updated after each weight.  This is the method the
// GPTQ pages compare against (GPTQ summary page, OBQ background): O(d_row d_col^3)
// work against GPTQ's shared order and shared inverse.
//
// One workgroup per row; at most OBQ_SLOTS workgroups, each taking rows in turn with
// its own d_col x d_col copy F of H^-1 in the workspace.  The row's grid (one group
// per row) is fixed first from its original values, as the per-row sweep does.  Per
// step, over the live (not yet quantized) weights:
//   1. added error (w_j - q(w_j))^2 / F_jj of every live j; the smallest wins (ties to
//      the lowest index);
//   2. row j of F is staged in LDS (F is symmetric, so it is also column j);
//   3. the other live weights move by -(w_j - q(w_j)) / F_jj * F[j][i];
//   4. F -= F[:, j] F[j, :] / F_jj on the live rows (every column: rows and columns of
//      quantized weights hold zeros, which the update keeps), row and column j set to 0;
//   5. j leaves the live list.
// Arithmetic is fp32 (H^-1 = U^T U formed with fp64 sums).  The whole F is read and
// written once per step on the live rows: sum over steps of live x d_col elements.

#include "common.h"
#include "kernels.h"
#include "quant_internal.h"

namespace gptq {

constexpr int OBQ_T = 256;
constexpr int OBQ_SLOTS = 256;

// H^-1 = U^T U for U upper triangular (from the factorization of the damped H).
__global__ void obq_hinv_kernel(const float* U, int64_t d, float* Hinv) {
    const int64_t i = blockIdx.y, j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= d) return;
    const int64_t m = i < j ? i : j;
    double s = 0.0;
    for (int64_t k = 0; k <= m; ++k) s += (double)U[k * d + i] * (double)U[k * d + j];
    Hinv[i * d + j] = (float)s;
}

template <int BITS, bool SYM, gptq_dtype DT>
__global__ __launch_bounds__(OBQ_T) void obq_kernel(const void* W, int64_t d_row, int d, const float* Hinv,
                                                    float* Fbase, uint8_t* codes, int64_t code_ld,
                                                    uint16_t* scales, uint16_t* zeros, int32_t* info) {
    constexpr int QMIN = SYM ? -((1 << (BITS - 1)) - 1) : 0;
    constexpr int QMAX = SYM ? ((1 << (BITS - 1)) - 1) : (1 << BITS) - 1;
    constexpr int ZOFF = SYM ? (1 << (BITS - 1)) : 0;
    __shared__ float w[OBQ_MAXD], rowj[OBQ_MAXD];
    __shared__ int live[OBQ_MAXD], pos[OBQ_MAXD];
    __shared__ uint8_t u[OBQ_MAXD];
    __shared__ float rs[OBQ_T], smx[OBQ_T];
    __shared__ int ri[OBQ_T];
    __shared__ uint16_t sp[2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    float* F = Fbase + (int64_t)blockIdx.x * d * d;
    const int64_t dd = (int64_t)d * d;

    for (int64_t r = blockIdx.x; r < d_row; r += gridDim.x) {
        // the row, its range and its own copy of H^-1
        float mn = INFINITY, mx = -INFINITY;
        for (int c = tid; c < d; c += OBQ_T) {
            const float v = load_as_f32<DT>(W, r * d + c);
            w[c] = v; live[c] = c; pos[c] = c;
            mn = fminf(mn, v); mx = fmaxf(mx, v);
        }
        for (int64_t e = tid; e < dd; e += OBQ_T) F[e] = Hinv[e];
        rs[tid] = mn; smx[tid] = mx;
        __syncthreads();
        for (int st = OBQ_T / 2; st > 0; st >>= 1) {
            if (tid < st) { rs[tid] = fminf(rs[tid], rs[tid + st]); smx[tid] = fmaxf(smx[tid], smx[tid + st]); }
            __syncthreads();
        }
        if (tid == 0) {
            range_params<BITS, SYM>(rs[0], smx[0], info, sp[0], sp[1]);
            scales[r] = sp[0]; zeros[r] = sp[1];
        }
        __syncthreads();
        const float s16 = f16_bits_to_f32(sp[0]);
        const float zq = f16_bits_to_f32(sp[1]) - (float)ZOFF;   // Z on the (signed or unsigned) grid

        for (int L = d; L > 0; --L) {
            // 1. the live weight that adds the least error
            float best = INFINITY;
            int bj = 0x7fffffff;
            for (int t = tid; t < L; t += OBQ_T) {
                const int j = live[t];
                const float wj = w[j];
                const float q = fminf(fmaxf(rintf(wj / s16) + zq, (float)QMIN), (float)QMAX);
                const float e = wj - s16 * (q - zq);
                const float sc = e * e / F[(int64_t)j * d + j];
                if (sc < best || (sc == best && j < bj)) { best = sc; bj = j; }
            }
            rs[tid] = best; ri[tid] = bj;
            __syncthreads();
            for (int st = OBQ_T / 2; st > 0; st >>= 1) {
                if (tid < st) {
                    const float o = rs[tid + st];
                    const int oi = ri[tid + st];
                    if (o < rs[tid] || (o == rs[tid] && oi < ri[tid])) { rs[tid] = o; ri[tid] = oi; }
                }
                __syncthreads();
            }
            const int j = ri[0];
            // 2. row j of F
            for (int c = tid; c < d; c += OBQ_T) rowj[c] = F[(int64_t)j * d + c];
            __syncthreads();
            // 3. the code of j and the move of the other live weights
            const float wj = w[j];
            const float qj = fminf(fmaxf(rintf(wj / s16) + zq, (float)QMIN), (float)QMAX);
            const float err = (wj - s16 * (qj - zq)) / rowj[j];
            if (tid == 0) u[j] = (uint8_t)((int)qj + ZOFF);
            for (int t = tid; t < L; t += OBQ_T) {
                const int i = live[t];
                if (i != j) w[i] = fmaf(-err, rowj[i], w[i]);
            }
            // 4. j leaves the inverse: one wave per live row, lanes across the columns
            const float inv = 1.f / rowj[j];
            for (int rr = wave; rr < L; rr += OBQ_T / 64) {
                const int i = live[rr];
                float* Fi = F + (int64_t)i * d;
                if (i == j) {
                    for (int k = lane; k < d; k += 64) Fi[k] = 0.f;
                } else {
                    const float a = rowj[i] * inv;
                    for (int k = lane; k < d; k += 64) Fi[k] = (k == j) ? 0.f : fmaf(-a, rowj[k], Fi[k]);
                }
            }
            __syncthreads();
            // 5. j leaves the live list (the last live index takes its place)
            if (tid == 0) {
                const int p = pos[j], last = live[L - 1];
                live[p] = last; pos[last] = p;
            }
            __syncthreads();
        }
        // the row's codes: the 3-bit stream (three bytes per 8 codes), two per byte (first
        // in the low nibble) or one per byte
        uint8_t* crow = codes + r * code_ld;
        if (BITS == 3) {
            for (int g8 = tid; g8 < d / 8; g8 += OBQ_T) {
                uint32_t v = 0;
                for (int k = 0; k < 8; ++k) v |= (uint32_t)(u[8 * g8 + k] & 7) << (3 * k);
                crow[3 * g8] = (uint8_t)v;
                crow[3 * g8 + 1] = (uint8_t)(v >> 8);
                crow[3 * g8 + 2] = (uint8_t)(v >> 16);
            }
        } else if (BITS <= 4) {
            for (int c = tid; c < d / 2; c += OBQ_T) crow[c] = (uint8_t)(u[2 * c] | (u[2 * c + 1] << 4));
        } else {
            for (int c = tid; c < d; c += OBQ_T) crow[c] = u[c];
        }
        __syncthreads();
    }
}

size_t obq_ws_bytes(int64_t d_row, int64_t d_col) {
    if (d_row <= 0 || d_col <= 0) return 0;
    const int64_t slots = d_row < OBQ_SLOTS ? d_row : OBQ_SLOTS;
    return (size_t)(slots + 1) * d_col * d_col * sizeof(float);
}

template <int BITS, bool SYM>
static void obq_go(const void* W, gptq_dtype wt, int64_t d_row, int d, const float* Hinv, float* F, int slots,
                   uint8_t* codes, int64_t code_ld, uint16_t* scales, uint16_t* zeros, int32_t* info, hipStream_t s) {
    switch (wt) {
        case GPTQ_F32:
            obq_kernel<BITS, SYM, GPTQ_F32><<<slots, OBQ_T, 0, s>>>(W, d_row, d, Hinv, F, codes, code_ld, scales, zeros, info);
            break;
        case GPTQ_BF16:
            obq_kernel<BITS, SYM, GPTQ_BF16><<<slots, OBQ_T, 0, s>>>(W, d_row, d, Hinv, F, codes, code_ld, scales, zeros, info);
            break;
        default:
            obq_kernel<BITS, SYM, GPTQ_F16><<<slots, OBQ_T, 0, s>>>(W, d_row, d, Hinv, F, codes, code_ld, scales, zeros, info);
            break;
    }
}

gptq_status obq_launch(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                       const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros, void* ws,
                       size_t ws_bytes, int32_t* info, hipStream_t s) {
    if (ws == nullptr || ws_bytes < obq_ws_bytes(d_row, d_col)) return GPTQ_ERR_WORKSPACE;
    const int slots = (int)(d_row < OBQ_SLOTS ? d_row : OBQ_SLOTS);
    float* Hinv = reinterpret_cast<float*>(ws);
    float* F = Hinv + d_col * d_col;
    fill_i32(info, 1, 0, s);
    GPTQ_LAUNCH_CHECK();
    obq_hinv_kernel<<<dim3((unsigned)((d_col + 255) / 256), (unsigned)d_col), 256, 0, s>>>(U, d_col, Hinv);
    GPTQ_LAUNCH_CHECK();
    const int64_t code_ld = p.bits == 3 ? d_col / 8 * 3 : p.bits <= 4 ? d_col / 2 : d_col;
    const int d = (int)d_col;
#define OG(B, S) obq_go<B, S>(W, w_dtype, d_row, d, Hinv, F, slots, codes, code_ld, scales, zeros, info, s)
    if (p.bits == 4) { if (p.sym) OG(4, true); else OG(4, false); }
    else if (p.bits == 3) { if (p.sym) OG(3, true); else OG(3, false); }
    else if (p.bits == 8) { if (p.sym) OG(8, true); else OG(8, false); }
    else return GPTQ_ERR_UNSUPPORTED;
#undef OG
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
