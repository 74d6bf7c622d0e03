// The GPTQ column sweep on one layer: fused group scale/zero, quantization,
// error compensation inside 128-column blocks, code packing, and the lazy
// trailing update of the later columns.
//
// GPTQ summary page: OBQ background (quantize one weight, then update the
// remaining full-precision weights to compensate, in the direction given by the
// inverse Hessian); "Innovation 1" (one fixed column order for all rows, so the
// inverse Hessian is shared); "Innovation 2" (B = 128 columns are processed with
// updates kept local to the block, then one large matrix update of the rest);
// "Innovation 3" (rows of the Cholesky factor U of the inverse give the updates).
// Quantization concepts guide: "Mapping values to fewer bits" (S, Z, quantize),
// "Choose granularity" (per-group scales along a row), "Data types - int8 and
// int4" (two codes per byte, first in the low nibble).
//
// Sweep kernel layout: a workgroup owns 64 rows of the block; each row is held
// by 4 lanes of one quad, lane q holding columns q, q+4, ..., q+124 in registers
// (column-cyclic, so the triangular work stays balanced).  The block's diagonal
// 128 x 128 part of U is staged in LDS, permuted so that a lane reads its four
// next coefficients with one 16-byte LDS read.  The quantization error of column
// j is broadcast inside the quad with a DPP quad_perm.  Group min/max use DPP
// quad reductions.  The trailing update W[:, b1:] -= E U[b0:b1, b1:] runs on
// v_mfma_f32_16x16x4_f32 (fp32 operands).

#include <utility>

#include "common.h"
#include "kernels.h"

namespace gptq {

constexpr int QB = 128;
constexpr int QROWS = 64;
constexpr int QT = 256;

template <int I, int N, typename F>
GPTQ_DEV void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

GPTQ_DEV bool normal_f16_scale(float s) { return s >= 6.103515625e-05f && s <= 65504.f; }

struct SweepArgs {
    const float* Wws; int64_t d_row, d_col;
    const float* U;
    int64_t b0; int nb;
    float* E;                       // d_row x 128
    uint8_t* codes; int64_t code_ld;
    uint16_t* scales; uint16_t* zeros; int n_groups;
    int32_t* info;
    int group;                      // 32, 64, 128 (power of two), or 0 = per-row params precomputed
    int qmin, qmax, zoff;           // grid and stored-code offset
    int sym; int packed;            // packed: two codes per byte
};

__global__ __launch_bounds__(QT) void sweep_kernel(SweepArgs a) {
    __shared__ __attribute__((aligned(16))) float Up[QB][4][32];  // Up[j][q][i] = U[b0+j][b0+4i+q]
    __shared__ uint8_t cl[QROWS][QB];
    __shared__ int bad_any;

    const int tid = threadIdx.x;
    const int q = tid & 3;
    const int rl = tid >> 2;
    const int64_t row = (int64_t)blockIdx.x * QROWS + rl;
    const bool rv = row < a.d_row;
    const int nb = a.nb;
    const int G = a.group;
    const float fqmin = (float)a.qmin, fqmax = (float)a.qmax, fzoff = (float)a.zoff;
    if (tid == 0) bad_any = 0;

    for (int idx = tid; idx < QB * QB; idx += QT) {
        const int j = idx >> 7, c = idx & 127;
        Up[j][c & 3][c >> 2] = (j < nb && c < nb) ? a.U[(a.b0 + j) * a.d_col + a.b0 + c] : 0.f;
    }
    float w[32], e[32], uc[32];
    const float* wrow = a.Wws + (rv ? row : 0) * a.d_col + a.b0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int c = 4 * i + q;
        w[i] = (rv && c < nb) ? wrow[c] : 0.f;
        e[i] = 0.f;
    }
    float s16f = 1.f, zf = 0.f;
    bool bad = false;
    if (G == 0 && rv) {
        s16f = f16_bits_to_f32(a.scales[row * a.n_groups]);
        zf = f16_bits_to_f32(a.zeros[row * a.n_groups]) - fzoff;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const f32x4_t u4 = *reinterpret_cast<const f32x4_t*>(&Up[0][q][4 * m]);
#pragma unroll
        for (int k = 0; k < 4; ++k) uc[4 * m + k] = u4[k];
    }

    static_for<0, QB>([&](auto JC) {
        constexpr int j = decltype(JC)::value;
        constexpr int qj = j & 3, ij = j >> 2;
        constexpr int ijn = (j + 1) >> 2;
        if (j >= nb) return;
        // prefetch the coefficients of step j + 1 (slots >= its own slot)
        float un[32];
        if constexpr (j + 1 < QB) {
#pragma unroll
            for (int m = ijn >> 2; m < 8; ++m) {
                const f32x4_t u4 = *reinterpret_cast<const f32x4_t*>(&Up[j + 1][q][4 * m]);
#pragma unroll
                for (int k = 0; k < 4; ++k) un[4 * m + k] = u4[k];
            }
        }
        if (G > 0 && (j & (G - 1)) == 0) {
            // group scale/zero from the current values of columns j .. j+G-1
            const int iend = (j + G) >> 2;
            float s, mn = 0.f;
            if (a.sym) {
                float am = 0.f;
#pragma unroll
                for (int i = j / 4; i < 32; ++i) if (i < iend) am = fmaxf(am, fabsf(w[i]));
                am = fmaxf(am, quad_perm<QP_XOR1>(am));
                am = fmaxf(am, quad_perm<QP_XOR2>(am));
                s = am > 0.f ? am / fqmax : 1.f;
            } else {
                float mx = w[j / 4];
                mn = w[j / 4];
#pragma unroll
                for (int i = j / 4 + 1; i < 32; ++i)
                    if (i < iend) { mn = fminf(mn, w[i]); mx = fmaxf(mx, w[i]); }
                mn = fminf(mn, quad_perm<QP_XOR1>(mn));
                mn = fminf(mn, quad_perm<QP_XOR2>(mn));
                mx = fmaxf(mx, quad_perm<QP_XOR1>(mx));
                mx = fmaxf(mx, quad_perm<QP_XOR2>(mx));
                if (mn == mx) { mn = fminf(mn, 0.f); mx = fmaxf(mx, 0.f); }
                s = (mx > mn) ? (mx - mn) / (fqmax - fqmin) : 1.f;
            }
            s16f = f16_bits_to_f32(f32_to_f16_bits(s));
            if (!normal_f16_scale(s16f)) { bad = true; s16f = 1.f; }
            zf = a.sym ? 0.f : fqmin - rintf(mn / s16f);
            if (q == 0 && rv) {
                const int64_t g = (a.b0 + j) / G;
                a.scales[row * a.n_groups + g] = f32_to_f16_bits(s16f);
                a.zeros[row * a.n_groups + g] = f32_to_f16_bits(zf + fzoff);
            }
        }
        // quantize column j (its owner is lane qj of the quad, slot ij)
        const float wv = w[ij];
        const float t = wv / s16f;
        const float qv = fminf(fmaxf(rintf(t + zf), fqmin), fqmax);
        const float wq = s16f * (qv - zf);
        const float err = (wv - wq) / uc[ij];
        const float errb = quad_bcast<qj>(err);
        if (q == qj) {
            e[ij] = err;
            cl[rl][j] = (uint8_t)((int)qv + a.zoff);
            if (!(fabsf(err) <= 3.0e38f)) bad = true;
        }
        // compensate the later columns of the block; U is upper triangular, so the
        // coefficients of earlier columns in slot ij are zero or hit finished columns
#pragma unroll
        for (int i = ij; i < 32; ++i) w[i] = fmaf(-errb, uc[i], w[i]);
        if constexpr (j + 1 < QB) {
#pragma unroll
            for (int i = ijn; i < 32; ++i) uc[i] = un[i];
        }
        __builtin_amdgcn_sched_barrier(0);
    });

    if (rv) {
        float* erow = a.E + row * QB;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int c = 4 * i + q;
            if (c < nb) erow[c] = e[i];
        }
    }
    if (bad && rv) atomicOr(&bad_any, 1);
    __syncthreads();
    if (tid == 0 && bad_any) *a.info = -1;

    // pack the block's codes: two per byte (column 2k in the low nibble) or one per byte
    const int per = a.packed ? 2 : 1;
    const int nbytes = nb / per;
    const int rowbytes = QB / per;
    for (int idx = tid; idx < QROWS * rowbytes; idx += QT) {
        const int r = idx / rowbytes, bidx = idx % rowbytes;
        const int64_t grow = (int64_t)blockIdx.x * QROWS + r;
        if (grow >= a.d_row || bidx >= nbytes) continue;
        const uint8_t v = a.packed ? (uint8_t)((cl[r][2 * bidx] & 0xF) | ((cl[r][2 * bidx + 1] & 0xF) << 4))
                                   : cl[r][bidx];
        a.codes[grow * a.code_ld + a.b0 / per + bidx] = v;
    }
}

// --------------------------------------------------------------------------
// One scale/zero per row (group_size 0): from the original row, before any update.
template <int BITS, bool SYM>
__global__ __launch_bounds__(256) void row_params_kernel(const float* Wws, int64_t d_col, uint16_t* scales,
                                                         uint16_t* zeros, int32_t* info) {
    constexpr int QMIN = SYM ? -((1 << (BITS - 1)) - 1) : 0;
    constexpr int QMAX = SYM ? ((1 << (BITS - 1)) - 1) : (1 << BITS) - 1;
    constexpr int ZOFF = SYM ? (1 << (BITS - 1)) : 0;
    __shared__ float smn[256], smx[256];
    const int64_t row = blockIdx.x;
    const float* w = Wws + row * d_col;
    float mn = INFINITY, mx = -INFINITY;
    for (int64_t c = threadIdx.x; c < d_col; c += 256) {
        const float v = w[c];
        mn = fminf(mn, v); mx = fmaxf(mx, v);
    }
    smn[threadIdx.x] = mn; smx[threadIdx.x] = mx;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if ((int)threadIdx.x < st) {
            smn[threadIdx.x] = fminf(smn[threadIdx.x], smn[threadIdx.x + st]);
            smx[threadIdx.x] = fmaxf(smx[threadIdx.x], smx[threadIdx.x + st]);
        }
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    mn = smn[0]; mx = smx[0];
    float s, zf = 0.f;
    if (SYM) {
        const float am = fmaxf(fabsf(mn), fabsf(mx));
        s = am > 0.f ? am / (float)QMAX : 1.f;
    } else {
        if (mn == mx) { mn = fminf(mn, 0.f); mx = fmaxf(mx, 0.f); }
        s = (mx > mn) ? (mx - mn) / (float)(QMAX - QMIN) : 1.f;
    }
    float s16f = f16_bits_to_f32(f32_to_f16_bits(s));
    if (!normal_f16_scale(s16f)) { *info = -1; s16f = 1.f; }
    if (!SYM) zf = (float)QMIN - rintf(mn / s16f);
    scales[row] = f32_to_f16_bits(s16f);
    zeros[row] = f32_to_f16_bits(zf + (float)ZOFF);
}

// W (any dtype) -> fp32 working copy; flags non-finite values.
template <gptq_dtype DT>
__global__ void convert_kernel(const void* W, int64_t n, float* out, int32_t* info) {
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const float v = load_as_f32<DT>(W, i);
        if (!isfinite(v)) bad = 1;
        out[i] = v;
    }
    if (bad) *info = -1;
}

// --------------------------------------------------------------------------
// Trailing lazy update on fp32 MFMA: W[:, b1:] -= E[:, :nb] U[b0:b0+nb, b1:].
constexpr int TB = 64, TK = 32, TLD = TB + 4;

struct TrailArgs {
    float* Wws; int64_t d_row, d_col;
    const float* E; const float* U;
    int64_t b0, b1; int nb;
};

__global__ __launch_bounds__(256) void trail_kernel(TrailArgs a) {
    __shared__ float Es[TK][TLD];
    __shared__ float Us[TK][TLD];
    const int64_t m0 = (int64_t)blockIdx.y * TB;
    const int64_t n0 = a.b1 + (int64_t)blockIdx.x * TB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{};
    for (int k0 = 0; k0 < a.nb; k0 += TK) {
        for (int idx = tid; idx < TB * TK; idx += 256) {
            const int m = idx / TK, k = idx % TK;  // E rows, k contiguous
            const int64_t gm = m0 + m;
            Es[k][m] = (gm < a.d_row && k0 + k < a.nb) ? a.E[gm * QB + k0 + k] : 0.f;
            const int kk = idx / TB, n = idx % TB;  // U rows, n contiguous
            const int64_t gn = n0 + n;
            Us[kk][n] = (gn < a.d_col && k0 + kk < a.nb) ? a.U[(a.b0 + k0 + kk) * a.d_col + gn] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; kk += 4) {
            float fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = Es[kk + (lane >> 4)][wr * 32 + i * 16 + (lane & 15)];
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = Us[kk + (lane >> 4)][wc * 32 + j * 16 + (lane & 15)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t gm = m0 + wr * 32 + i * 16 + 4 * (lane >> 4) + e;
                const int64_t gn = n0 + wc * 32 + j * 16 + (lane & 15);
                if (gm < a.d_row && gn < a.d_col) a.Wws[gm * a.d_col + gn] -= acc[i][j][e];
            }
}

// --------------------------------------------------------------------------
// Host side
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t quant_ws_bytes(int64_t d_row, int64_t d_col) {
    if (d_row <= 0 || d_col <= 0) return 0;
    return align256((size_t)d_row * d_col * sizeof(float)) + align256((size_t)d_row * QB * sizeof(float));
}

static gptq_status launch_row_params(int bits, bool sym, const float* Wws, int64_t d_row, int64_t d_col,
                                     uint16_t* scales, uint16_t* zeros, int32_t* info, hipStream_t s) {
    dim3 grid((unsigned)d_row);
#define RP(B, S) row_params_kernel<B, S><<<grid, 256, 0, s>>>(Wws, d_col, scales, zeros, info)
    if (bits == 4) { if (sym) RP(4, true); else RP(4, false); }
    else if (bits == 3) { if (sym) RP(3, true); else RP(3, false); }
    else if (bits == 8) { if (sym) RP(8, true); else RP(8, false); }
    else return GPTQ_ERR_UNSUPPORTED;
#undef RP
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

gptq_status quant_launch(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                         const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                         void* ws, size_t ws_bytes, int32_t* info, hipStream_t s) {
    if (ws == nullptr || ws_bytes < quant_ws_bytes(d_row, d_col)) return GPTQ_ERR_WORKSPACE;
    float* Wws = reinterpret_cast<float*>(ws);
    float* E = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256((size_t)d_row * d_col * sizeof(float)));
    const int G = p.group_size;
    const int n_groups = (G == 0) ? 1 : (int)(d_col / G);

    fill_i32(info, 1, 0, s);
    GPTQ_LAUNCH_CHECK();
    const int64_t n = d_row * d_col;
    const unsigned cgrid = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
    switch (w_dtype) {
        case GPTQ_F32: convert_kernel<GPTQ_F32><<<cgrid, 256, 0, s>>>(W, n, Wws, info); break;
        case GPTQ_BF16: convert_kernel<GPTQ_BF16><<<cgrid, 256, 0, s>>>(W, n, Wws, info); break;
        case GPTQ_F16: convert_kernel<GPTQ_F16><<<cgrid, 256, 0, s>>>(W, n, Wws, info); break;
        default: return GPTQ_ERR_UNSUPPORTED;
    }
    GPTQ_LAUNCH_CHECK();
    gptq_status st;
    if (G == 0) {
        st = launch_row_params(p.bits, p.sym != 0, Wws, d_row, d_col, scales, zeros, info, s);
        if (st != GPTQ_OK) return st;
    }
    SweepArgs sa;
    sa.Wws = Wws; sa.d_row = d_row; sa.d_col = d_col; sa.U = U; sa.E = E;
    sa.codes = codes; sa.code_ld = (p.bits <= 4) ? d_col / 2 : d_col;
    sa.scales = scales; sa.zeros = zeros; sa.n_groups = n_groups; sa.info = info;
    sa.group = G; sa.sym = p.sym != 0; sa.packed = p.bits <= 4;
    sa.qmin = sa.sym ? -((1 << (p.bits - 1)) - 1) : 0;
    sa.qmax = sa.sym ? ((1 << (p.bits - 1)) - 1) : (1 << p.bits) - 1;
    sa.zoff = sa.sym ? (1 << (p.bits - 1)) : 0;
    const dim3 sgrid((unsigned)((d_row + QROWS - 1) / QROWS));
    for (int64_t b0 = 0; b0 < d_col; b0 += QB) {
        const int nb = (int)std::min<int64_t>(QB, d_col - b0);
        sa.b0 = b0; sa.nb = nb;
        sweep_kernel<<<sgrid, QT, 0, s>>>(sa);
        GPTQ_LAUNCH_CHECK();
        const int64_t b1 = b0 + nb;
        if (b1 < d_col) {
            TrailArgs ta{Wws, d_row, d_col, E, U, b0, b1, nb};
            dim3 tgrid((unsigned)((d_col - b1 + TB - 1) / TB), (unsigned)((d_row + TB - 1) / TB));
            trail_kernel<<<tgrid, 256, 0, s>>>(ta);
            GPTQ_LAUNCH_CHECK();
        }
    }
    return GPTQ_OK;
}

// --------------------------------------------------------------------------
// Dequantization: W_out = S16 (u - z).
template <int BITS, gptq_dtype OT>
__global__ void dequant_kernel(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t d_row,
                               int64_t d_col, int G, void* out) {
    const int64_t row = blockIdx.y;
    const int64_t chunks = (d_col + 7) / 8;
    const int64_t code_ld = (BITS <= 4) ? d_col / 2 : d_col;
    const int n_groups = (G == 0) ? 1 : (int)(d_col / G);
    for (int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ch < chunks; ch += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c0 = ch * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t c = c0 + e;
            if (c >= d_col) { v[e] = 0.f; continue; }
            uint32_t u;
            if constexpr (BITS <= 4) {
                const uint8_t b = codes[row * code_ld + (c >> 1)];
                u = (c & 1) ? (b >> 4) : (b & 0xF);
            } else {
                u = codes[row * code_ld + c];
            }
            const int g = (G == 0) ? 0 : (int)(c / G);
            const float s = f16_bits_to_f32(scales[row * n_groups + g]);
            const float z = f16_bits_to_f32(zeros[row * n_groups + g]);
            v[e] = s * ((float)u - z);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t c = c0 + e;
            if (c >= d_col) break;
            if constexpr (OT == GPTQ_F32) reinterpret_cast<float*>(out)[row * d_col + c] = v[e];
            else if constexpr (OT == GPTQ_BF16) reinterpret_cast<uint16_t*>(out)[row * d_col + c] = f32_to_bf16_bits(v[e]);
            else reinterpret_cast<uint16_t*>(out)[row * d_col + c] = f32_to_f16_bits(v[e]);
        }
    }
}

template <int BITS>
static gptq_status dq_dt(gptq_dtype ot, dim3 grid, hipStream_t s, const uint8_t* codes, const uint16_t* scales,
                         const uint16_t* zeros, int64_t d_row, int64_t d_col, int G, void* out) {
    switch (ot) {
        case GPTQ_F32: dequant_kernel<BITS, GPTQ_F32><<<grid, 256, 0, s>>>(codes, scales, zeros, d_row, d_col, G, out); break;
        case GPTQ_BF16: dequant_kernel<BITS, GPTQ_BF16><<<grid, 256, 0, s>>>(codes, scales, zeros, d_row, d_col, G, out); break;
        case GPTQ_F16: dequant_kernel<BITS, GPTQ_F16><<<grid, 256, 0, s>>>(codes, scales, zeros, d_row, d_col, G, out); break;
        default: return GPTQ_ERR_UNSUPPORTED;
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

gptq_status dequant_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t d_row,
                           int64_t d_col, int bits, int group_size, void* out, gptq_dtype out_dtype,
                           hipStream_t s) {
    const int64_t chunks = (d_col + 7) / 8;
    dim3 grid((unsigned)std::min<int64_t>((chunks + 255) / 256, 64), (unsigned)d_row);
    if (bits <= 4) return dq_dt<4>(out_dtype, grid, s, codes, scales, zeros, d_row, d_col, group_size, out);
    return dq_dt<8>(out_dtype, grid, s, codes, scales, zeros, d_row, d_col, group_size, out);
}

}  // namespace gptq
