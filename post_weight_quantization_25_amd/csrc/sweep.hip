// The GPTQ column sweep inside one 128-column block: fused group scale / zero
// point, quantization, error compensation of the later columns of the block,
// and the error block E for the lazy trailing update.
//
// GPTQ summary page: OBQ background (quantize one weight, then update the
// remaining full-precision weights to compensate, in the direction given by the
// inverse Hessian); "Innovation 1" (one column order for all rows); "Innovation
// 2" (updates kept local to a block of B = 128 columns); "Innovation 3" (rows of
// the Cholesky factor U of the inverse give the updates).  Quantization concepts
// guide: "Mapping values to fewer bits", "Choose granularity".
//
// Layout: a workgroup owns 16 rows of the block; each row is held by the 16
// lanes of one DPP row, lane q holding columns q, q+16, ..., q+112 in registers
// (column-cyclic, so the triangular work stays balanced).  The block's diagonal
// 128 x 128 part of U is staged in LDS, permuted so that a lane reads its eight
// coefficients of the next step with two 16-byte LDS reads (prefetched one step
// ahead).  The quantization error of column j is broadcast along the row with
// DPP row_newbcast; group min/max use DPP butterfly reductions.

#include <utility>

#include "quant_internal.h"

namespace gptq {

constexpr int SSLOTS = QB / SL;     // columns per lane: q, q+16, ..., q+112

GPTQ_DEV bool normal_f16_scale(float s) { return s >= 6.103515625e-05f && s <= 65504.f; }

template <int SRC>
GPTQ_DEV float row_bcast(float v) {  // DPP row_newbcast: lane SRC of each 16-lane row to the whole row
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + SRC, 0xf, 0xf, false));
}
template <int CTRL>
GPTQ_DEV float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
GPTQ_DEV float row_min(float v) {
    v = fminf(v, quad_perm<QP_XOR1>(v));
    v = fminf(v, quad_perm<QP_XOR2>(v));
    v = fminf(v, dpp_f<DPP_HALF_MIRROR>(v));
    return fminf(v, dpp_f<DPP_MIRROR>(v));
}
GPTQ_DEV float row_max(float v) {
    v = fmaxf(v, quad_perm<QP_XOR1>(v));
    v = fmaxf(v, quad_perm<QP_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
    return fmaxf(v, dpp_f<DPP_MIRROR>(v));
}

__global__ __launch_bounds__(QT) void sweep_kernel(SweepArgs a) {
    __shared__ __attribute__((aligned(16))) float Up[QB][SL][SSLOTS];  // Up[j][q][i] = U[b0+j][b0+q+16i]
    __shared__ float invd[QB];                                         // 1 / U[b0+j][b0+j]
    __shared__ __attribute__((aligned(16))) uint8_t cl[SROWS][QB];
    __shared__ __attribute__((aligned(16))) uint16_t ehs[SROWS][QB], els[SROWS][QB];   // E split, staged
    __shared__ int bad_any;

    const int tid = threadIdx.x;
    const int q = tid & (SL - 1);
    const int rl = tid >> 4;
    const int64_t row = (int64_t)blockIdx.x * SROWS + rl;
    const bool rv = row < a.d_row;
    const int nb = a.nb;
    const int G = a.group;
    const float fqmin = (float)a.qmin, fqmax = (float)a.qmax, fzoff = (float)a.zoff;
    if (tid == 0) bad_any = 0;

    float w[SSLOTS], e[SSLOTS];
    int cv[SSLOTS];
    const float* wrow = a.Wws + (rv ? row : 0) * a.d_col + a.b0;
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) {
        const int c = SL * i + q;
        w[i] = (rv && c < nb) ? wrow[c] : 0.f;
        e[i] = 0.f;
        cv[i] = 0;
    }
    // stage U's diagonal block: all loads of a thread first (16-byte loads when rows
    // are 16-byte aligned), then the permuted LDS stores
    constexpr int NV = QB * QB / 4 / QT;   // float4 per thread
    f32x4_t uv[NV];
    const bool vec = nb == QB && ((a.d_col & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.U) & 15) == 0);
    if (vec) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + QT * v;       // float4 index: 32 per row of 128
            const int j = idx >> 5, c4 = (idx & 31) * 4;
            uv[v] = *reinterpret_cast<const f32x4_t*>(a.U + (a.b0 + j) * a.d_col + a.b0 + c4);
        }
    } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + QT * v;
            const int j = idx >> 5, c4 = (idx & 31) * 4;
            const float* src = a.U + (a.b0 + j) * a.d_col + a.b0 + c4;
#pragma unroll
            for (int e = 0; e < 4; ++e) uv[v][e] = (j < nb && c4 + e < nb) ? src[e] : 0.f;
        }
    }
    // the reciprocal pivots: one division in each of the first 128 threads
    const float udiag = (tid < nb) ? a.U[(a.b0 + tid) * a.d_col + a.b0 + tid] : 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = tid + QT * v;
        const int j = idx >> 5, c4 = (idx & 31) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = c4 + e;
            Up[j][c & (SL - 1)][c >> 4] = uv[v][e];
        }
    }
    if (tid < QB) invd[tid] = (tid < nb) ? 1.0f / udiag : 0.f;
    // s16f, r16f = 1 / s16f and the zero point zf of the current group; the code is
    // rne(t) + zf clamped to [qmin, qmax], i.e. rne(t) clamped to [lo, hi]
    float s16f = 1.f, r16f = 1.f, zf = 0.f;
    bool bad = false;
    if (G == 0 && rv) {
        s16f = f16_bits_to_f32(a.scales[row * a.n_groups]);
        r16f = 1.0f / s16f;
        zf = f16_bits_to_f32(a.zeros[row * a.n_groups]) - fzoff;
    }
    float lo = fqmin - zf, hi = fqmax - zf;
    __syncthreads();
    // U coefficients of the current and the next step, alternating by step parity
    float ucA[SSLOTS], ucB[SSLOTS];
    {
        const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(&Up[0][q][0]);
        const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(&Up[0][q][4]);
#pragma unroll
        for (int k = 0; k < 4; ++k) { ucA[k] = u0[k]; ucA[4 + k] = u1[k]; }
    }
    float idc = invd[0];

    // All 128 steps run: past nb (the last block of a width that is not a multiple of
    // 128) the weights, U and 1 / U[j][j] are 0, so those steps change nothing.
    static_for<0, QB>([&](auto JC) {
        constexpr int j = decltype(JC)::value;
        constexpr int qj = j & (SL - 1), ij = j >> 4;
        float* uc = (j & 1) ? ucB : ucA;
        float* un = (j & 1) ? ucA : ucB;
        // prefetch the coefficients of step j + 1, only the slots it uses (a loaded
        // value left unused lets the compiler reuse its register while the load is in
        // flight, which costs a wait every step)
        float idn = 0.f;
        if constexpr (j + 1 < QB) {
            constexpr int i1 = (j + 1) >> 4;
            if constexpr (i1 == 0) {
                const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(&Up[j + 1][q][0]);
#pragma unroll
                for (int k = 0; k < 4; ++k) un[k] = u0[k];
            } else {
#pragma unroll
                for (int k = i1; k < 4; ++k) un[k] = Up[j + 1][q][k];
            }
            if constexpr (i1 <= 4) {
                const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(&Up[j + 1][q][4]);
#pragma unroll
                for (int k = 0; k < 4; ++k) un[4 + k] = u1[k];
            } else {
#pragma unroll
                for (int k = i1; k < SSLOTS; ++k) un[k] = Up[j + 1][q][k];
            }
            idn = invd[j + 1];
        }
        __builtin_amdgcn_sched_barrier(0);   // issue the prefetch at the top of the step
        // a group starts at a multiple of its size (32, 64 or 128), so only every 32nd
        // step carries the group code
        if constexpr ((j & 31) == 0) {
            if (G > 0 && (j & (G - 1)) == 0) {
                // group scale/zero from the current values of columns j .. j+G-1
                const int iend = (j + G) >> 4;
                float sc, mn = 0.f;
                if (a.sym) {
                    float am = 0.f;
#pragma unroll
                    for (int i = ij; i < SSLOTS; ++i) if (i < iend) am = fmaxf(am, fabsf(w[i]));
                    am = row_max(am);
                    sc = am > 0.f ? am / fqmax : 1.f;
                } else {
                    float mx = w[ij];
                    mn = w[ij];
#pragma unroll
                    for (int i = ij + 1; i < SSLOTS; ++i)
                        if (i < iend) { mn = fminf(mn, w[i]); mx = fmaxf(mx, w[i]); }
                    mn = row_min(mn);
                    mx = row_max(mx);
                    if (mn == mx) { mn = fminf(mn, 0.f); mx = fmaxf(mx, 0.f); }
                    sc = (mx > mn) ? (mx - mn) / (fqmax - fqmin) : 1.f;
                }
                s16f = f16_bits_to_f32(f32_to_f16_bits(sc));
                if (!normal_f16_scale(s16f)) { bad = true; s16f = 1.f; }
                r16f = 1.0f / s16f;
                zf = a.sym ? 0.f : fqmin - rintf(mn / s16f);
                lo = fqmin - zf;
                hi = fqmax - zf;
                if (q == 0 && rv && a.b0 + j < a.d_col) {
                    const int64_t g = (a.b0 + j) / G;
                    a.scales[row * a.n_groups + g] = f32_to_f16_bits(s16f);
                    a.zeros[row * a.n_groups + g] = f32_to_f16_bits(zf + fzoff);
                }
            }
        }
        // quantize column j (owner: lane qj of the row, slot ij).  t = w / S16 correctly
        // rounded: q0 = w r with r = 1 / S16 correctly rounded, then one correction with
        // the exact residual w - q0 S16 (Markstein); equal to the IEEE quotient.  The code
        // is rne(t) + zf clamped to the grid (zf is an integer, so this is exact).
        const float wv = w[ij];
        const float q0 = wv * r16f;
        const float t = fmaf(fmaf(-q0, s16f, wv), r16f, q0);
        const float qd = __builtin_amdgcn_fmed3f(rintf(t), lo, hi);
        const float err = fmaf(-s16f, qd, wv) * idc;
        const float errb = row_bcast<qj>(err);
        const bool own = (q == qj);
        e[ij] = own ? err : e[ij];
        cv[ij] = own ? (int)(qd + zf) + a.zoff : cv[ij];
        // compensate the later columns; U is upper triangular, so in slot ij the lanes
        // holding columns <= j get a zero coefficient (or touch a finished column).
        // The slot of the next column first: it is on the critical path.
        constexpr int in = ((j + 1) >> 4) < SSLOTS ? ((j + 1) >> 4) : SSLOTS - 1;
        w[in] = fmaf(-errb, uc[in], w[in]);
#pragma unroll
        for (int i = ij; i < SSLOTS; ++i)
            if (i != in) w[i] = fmaf(-errb, uc[i], w[i]);
        idc = idn;
    });

    // a non-finite weight, scale or error shows up in the block's errors
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) bad = bad || !(fabsf(e[i]) <= 3.0e38f);
    // the trailing update multiplies on bf16 MFMA with a three-term split: the split
    // is formed here once (hi = bf16(e), lo = bf16(e - hi)) instead of in every
    // workgroup of the product; it and the codes are staged in LDS and written as
    // whole 16- / 4-byte pieces
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) {
        const int c = SL * i + q;
        const uint16_t h = f32_to_bf16_bits(e[i]);
        ehs[rl][c] = h;
        els[rl][c] = f32_to_bf16_bits(e[i] - bf16_bits_to_f32(h));
        cl[rl][c] = (uint8_t)cv[i];
    }
    if (bad && rv) atomicOr(&bad_any, 1);
    // LDS only: the global stores above and below need not have landed
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (tid == 0 && bad_any) *a.info = -1;

    const int per = a.packed ? 2 : 1;
    {
        // E: thread t writes 8 columns of row t / 16
        const int r = tid >> 4, c8 = (tid & 15) * 8;
        const int64_t grow = (int64_t)blockIdx.x * SROWS + r;
        if (grow < a.d_row) {
            uint16_t* hrow = a.Ehi + grow * a.lde;
            uint16_t* lrow = a.Elo + grow * a.lde;
            if (nb == QB && (a.lde & 7) == 0 && ((reinterpret_cast<uintptr_t>(a.Ehi) & 15) == 0) &&
                ((reinterpret_cast<uintptr_t>(a.Elo) & 15) == 0)) {
                *reinterpret_cast<u32x4_t*>(hrow + c8) = *reinterpret_cast<const u32x4_t*>(&ehs[r][c8]);
                *reinterpret_cast<u32x4_t*>(lrow + c8) = *reinterpret_cast<const u32x4_t*>(&els[r][c8]);
            } else {
                for (int c = c8; c < c8 + 8 && c < nb; ++c) { hrow[c] = ehs[r][c]; lrow[c] = els[r][c]; }
            }
        }
        // codes: two per byte (column 2k in the low nibble) or one per byte; thread t
        // writes 8 columns of row t / 16
        if (grow < a.d_row) {
            uint8_t* crow = a.codes + grow * a.code_ld + a.b0 / per;
            const bool whole = nb == QB && ((reinterpret_cast<uintptr_t>(crow) & (a.packed ? 3 : 7)) == 0);
            if (a.packed) {
                uint32_t v = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v |= (uint32_t)((cl[r][c8 + 2 * k] & 0xF) | ((cl[r][c8 + 2 * k + 1] & 0xF) << 4)) << (8 * k);
                if (whole) *reinterpret_cast<uint32_t*>(crow + c8 / 2) = v;
                else
                    for (int k = 0; k < 4 && c8 + 2 * k < nb; ++k) crow[c8 / 2 + k] = (uint8_t)(v >> (8 * k));
            } else {
                if (whole) {
                    *reinterpret_cast<uint2*>(crow + c8) = *reinterpret_cast<const uint2*>(&cl[r][c8]);
                } else {
                    for (int k = 0; k < 8 && c8 + k < nb; ++k) crow[c8 + k] = cl[r][c8 + k];
                }
            }
        }
    }
}

gptq_status sweep_launch(const SweepArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.d_row + SROWS - 1) / SROWS));
    sweep_kernel<<<grid, QT, 0, s>>>(a);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
