// The GPTQ column sweep over one super-block of up to four 128-column blocks: fused
// group scale / zero point, quantization, error compensation of the later columns of
// the block, the error block E for the lazy trailing update, and, after each block,
// that block's update of the rest of the super-block.
//
// GPTQ summary page: OBQ background (quantize one weight, then update the
// remaining full-precision weights to compensate, in the direction given by the
// inverse Hessian); "Innovation 1" (one column order for all rows); "Innovation
// 2" (updates kept local to a block of B = 128 columns); "Innovation 3" (rows of
// the Cholesky factor U of the inverse give the updates).  Quantization concepts
// guide: "Mapping values to fewer bits", "Choose granularity".
//
// Layout: a workgroup owns 16 rows; their values in the super-block's columns stay in
// LDS for the whole launch.  In a block each row is held by the 16 lanes of one DPP
// row, lane q holding columns q, q+16, ..., q+112 in registers (column-cyclic, so
// the triangular work stays balanced).  The block's diagonal
// 128 x 128 part of U is staged in LDS, permuted so that a lane reads its eight
// coefficients of the next step with two 16-byte LDS reads (prefetched one step
// ahead).  The quantization error of column j is broadcast along the row with
// DPP row_newbcast; group min/max use DPP butterfly reductions.
// After a block, its errors E (16 x 128, scaled by powers of two and split into fp16
// hi + lo, staged in LDS, then held in registers) update the rest of the super-block in
// LDS, W[:, later] -= E U[block, later], on v_mfma_f32_16x16x32_f16 with three products
// (hi hi + hi lo + lo hi, fp32 accumulation, then divided by the row's scale); the U
// operands come straight from global memory in registers, from the transposed scaled
// fp16 copy of the super-block's diagonal block of U (eight consecutive k of one column
// per 16-byte load), loaded while the block's steps run.  Rows are independent, so no
// other workgroup is involved.

#include <type_traits>
#include <utility>

#include "quant_internal.h"

namespace gptq {

constexpr int SSLOTS = QB / SL;     // columns per lane: q, q+16, ..., q+112
constexpr int WL_LD = QSB + 4;      // LDS row pitch of the super-block's W (floats)
constexpr int UT_N = 64;            // columns of U per update chunk


template <int SRC>
GPTQ_DEV float row_bcast(float v) {  // DPP row_newbcast: lane SRC of each 16-lane row to the whole row
    // (every lane reads a valid source, so no old value is needed)
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + SRC, 0xf, 0xf, false));
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

// The U operands of one 64-column chunk of a block's update for this lane (wave w:
// columns n0 + 16 w .. + 15): for each 32-k step, lane l holds column n0 + 16 w + l % 16
// at k = b0 + 32 kk + 8 (l / 16) .. + 7, hi and lo, from the operand-ordered copy of
// the diagonal block (always QSB x QSB, zero past d_col, so no bounds checks): one
// contiguous 1 KB piece per wave and operand.
constexpr int NKK = QB / 32;
struct UChunk { f16x8_t h[NKK], l[NKK]; };

GPTQ_DEV void load_uchunk(const SweepArgs& a, int64_t b0, int64_t n0, int wave, int lane, UChunk& u) {
    const int64_t o = ((((n0 - a.s0) >> 4) + wave) * (QSB / 32) + ((b0 - a.s0) >> 5)) * 512 + 8 * lane;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        u.h[kk] = *reinterpret_cast<const f16x8_t*>(a.Uthi + o + 512 * kk);
        u.l[kk] = *reinterpret_cast<const f16x8_t*>(a.Utlo + o + 512 * kk);
    }
}

// Workgroup barrier that orders LDS accesses only (every barrier of the sweep guards
// LDS data): global loads issued before it stay in flight across it.
GPTQ_DEV void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A block's diagonal 128 x 128 part of U into registers, in the order of its LDS copy:
// thread t holds the (row j, lane q) pairs p = t + QT m, each as the eight values
// U[b0 + j][b0 + q + 16 i] that lane q uses in step j (zero past nb), and, in the first
// 128 threads, the pivot U[b0 + t][b0 + t].  Pair p's row j lies in 16 m .. 16 m + 15, and
// step j touches only slots i >= j / 16 = m, so slots i < m are never read: not loaded.
constexpr int NPAIR = QB * SL / QT;
struct UDiag { float v[NPAIR][SSLOTS]; float piv; };

template <bool FULL>
GPTQ_DEV void load_udiag(const SweepArgs& a, int64_t b0, int nb, int tid, UDiag& u) {
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) {
        const int pr = tid + QT * m;
        const int j = pr >> 4, qq = pr & (SL - 1);
        const float* src = a.U + (b0 + j) * a.d_col + b0 + qq;
#pragma unroll
        for (int i = 0; i < SSLOTS; ++i) {
            static_assert(QT == 16 * SL, "pair p = t + QT m has row j in 16 m .. 16 m + 15");
            if (i < m) u.v[m][i] = 0.f;
            else u.v[m][i] = (FULL || (j < nb && qq + SL * i < nb)) ? src[SL * i] : 0.f;
        }
    }
    u.piv = (tid < nb) ? a.U[(b0 + tid) * a.d_col + b0 + tid] : 0.f;
}

// U chunks of one block's update of the rest of the super-block (at most QSB - QB columns)
constexpr int NCH = (QSB - QB) / UT_N;

// FULL: a whole super-block with every row, block and pointer aligned for 16-byte
// accesses (checked on the host), so that every load and store takes its vector form
// with no edge code around it.
template <bool FULL, bool FP4>
__global__ __launch_bounds__(QT) void sweep_kernel(SweepArgs a) {
    // Up[j][q][i] = U[b0+j][b0+q+16i]
    __shared__ __attribute__((aligned(16))) float Up[QB][SL][SSLOTS];
    __shared__ float invd[QB];                                         // 1 / U[b0+j][b0+j]
    __shared__ __attribute__((aligned(16))) float Wl[SROWS][WL_LD];    // the super-block's W
    __shared__ __attribute__((aligned(16))) uint8_t cl[SROWS][QB];
    // E split, staged; rows padded by 16 bytes so that the 16 rows of an operand read
    // fall on distinct banks
    __shared__ __attribute__((aligned(16))) uint16_t ehs[SROWS][QB + 8], els[SROWS][QB + 8];
    __shared__ float einv[SROWS];                                      // 1 / es of the rows
    __shared__ int bad_any;

    const int tid = threadIdx.x;
    const int q = tid & (SL - 1);
    const int rl = tid >> 4;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t row = (int64_t)blockIdx.x * SROWS + rl;
    const bool rv = row < a.d_row;
    const int nsb = (int)(a.s1 - a.s0);
    const int G = a.group;
    const float fqmin = (float)a.qmin, fqmax = (float)a.qmax, fzoff = (float)a.zoff;
    if (tid == 0) bad_any = 0;
    const float es_row = rv ? a.es[row] : 1.f;
    if (q == 0) einv[rl] = 1.0f / es_row;

    // the super-block's W for the workgroup's rows: thread t loads row t / 16,
    // columns 4 (t % 16) + 64 m (16-byte loads when rows are aligned)
    {
        constexpr int NW = QSB / 64;
        const float* src = a.Wws + (rv ? row : 0) * a.d_col + a.s0;
        const bool vec = FULL || nsb == QSB && ((a.d_col & 3) == 0) && ((a.s0 & 3) == 0) &&
                         ((reinterpret_cast<uintptr_t>(a.Wws) & 15) == 0);
        f32x4_t v[NW];
#pragma unroll
        for (int m = 0; m < NW; ++m) {
            const int c = 4 * q + 64 * m;
            if (vec) {
                v[m] = rv ? *reinterpret_cast<const f32x4_t*>(src + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[m][e] = (rv && c + e < nsb) ? src[c + e] : 0.f;
            }
        }
#pragma unroll
        for (int m = 0; m < NW; ++m) *reinterpret_cast<f32x4_t*>(&Wl[rl][4 * q + 64 * m]) = v[m];
    }

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

    UDiag ud;
    for (int64_t b0 = a.s0; b0 < a.s1; b0 += QB) {
    const int nb = (int)((a.s1 - b0) < QB ? (a.s1 - b0) : QB);
    const int cb = (int)(b0 - a.s0);       // the block's first column in Wl
    float w[SSLOTS], e[SSLOTS];
    // the code of each owned column, kept as a float and converted once at the block end,
    // off the steps' path: for the integer grids q + zf, for E2M1 the signed grid value
    using CodeT = float;
    CodeT cv[SSLOTS];
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) {
        e[i] = 0.f;
        cv[i] = 0;
    }
    // stage U's diagonal block (loaded ahead, during the previous block, except for
    // the first block) permuted into Up, and the reciprocal pivots
    if (b0 == a.s0) load_udiag<FULL>(a, b0, nb, tid, ud);
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) {
        const int pr = tid + QT * m;
        const int j = pr >> 4, qq = pr & (SL - 1);
        *reinterpret_cast<f32x4_t*>(&Up[j][qq][0]) = f32x4_t{ud.v[m][0], ud.v[m][1], ud.v[m][2], ud.v[m][3]};
        *reinterpret_cast<f32x4_t*>(&Up[j][qq][4]) = f32x4_t{ud.v[m][4], ud.v[m][5], ud.v[m][6], ud.v[m][7]};
    }
    if (tid < QB) invd[tid] = (tid < nb) ? 1.0f / ud.piv : 0.f;
    // every U chunk of this block's update: the loads are in flight during the steps
    const int64_t bn = b0 + QB;                       // the next block
    UChunk uch[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
        if (bn + UT_N * ch < a.s1) load_uchunk(a, b0, bn + UT_N * ch, wave, lane, uch[ch]);
    // U's row scales of this lane's columns (for the scaled errors), also in flight
    float usc[SSLOTS];
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) usc[i] = (FULL || SL * i + q < nb) ? a.us[b0 + SL * i + q] : 1.f;
    // the block's W from LDS (updated by the earlier blocks of the super-block); the
    // barrier before the U staging of the first block orders the W stores above
    if (b0 == a.s0) lds_barrier();
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) {
        const int c = SL * i + q;
        w[i] = (c < nb) ? Wl[rl][cb + c] : 0.f;
    }
    lds_barrier();
    // U coefficients of the current and the next step, alternating by step parity
    float ucA[SSLOTS], ucB[SSLOTS];
    {
        const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(&Up[0][q][0]);
        const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(&Up[0][q][4]);
#pragma unroll
        for (int k = 0; k < 4; ++k) { ucA[k] = u0[k]; ucA[4 + k] = u1[k]; }
    }
    // 1 / U[j][j] of this lane's columns j = q + 16 i: the owner of column j divides its
    // error with its own copy, so no step reads the reciprocal
    float idv[SSLOTS];
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) idv[i] = invd[SL * i + q];

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
        }
        __builtin_amdgcn_sched_barrier(0);   // issue the prefetch at the top of the step
        // a group starts at a multiple of its size (32, 64 or 128), so only every 32nd
        // step carries the group code
        if constexpr ((j & 31) == 0) {
            if (G > 0 && (j & (G - 1)) == 0) {
                // group scale/zero from the current values of columns j .. j+G-1
                const int iend = (j + G) >> 4;
                float sc, mn = 0.f;
                if (FP4 || a.sym) {
                    float am = 0.f;
#pragma unroll
                    for (int i = ij; i < SSLOTS; ++i) if (i < iend) am = fmaxf(am, fabsf(w[i]));
                    am = row_max(am);
                    sc = am > 0.f ? range_scale16(true, 0.f, 0.f, am, fqmax, FP4 && a.mx) : 1.f;
                } else {
                    float mx = w[ij];
                    mn = w[ij];
#pragma unroll
                    for (int i = ij + 1; i < SSLOTS; ++i)
                        if (i < iend) { mn = fminf(mn, w[i]); mx = fmaxf(mx, w[i]); }
                    mn = row_min(mn);
                    mx = row_max(mx);
                    if (mn == mx) { mn = fminf(mn, 0.f); mx = fmaxf(mx, 0.f); }
                    sc = (mx > mn) ? range_scale16(false, mn, mx, 0.f, fqmax - fqmin, false) : 1.f;
                }
                s16f = sc;   // an fp16 value
                if (!normal_f16_scale(s16f)) { bad = true; s16f = 1.f; }
                r16f = 1.0f / s16f;
                zf = (FP4 || a.sym) ? 0.f : fqmin - rintf(mn / s16f);
                lo = fqmin - zf;
                hi = fqmax - zf;
                if (q == 0 && rv && b0 + j < a.d_col) {
                    const int64_t g = (b0 + j) / G;
                    a.scales[row * a.n_groups + g] = f32_to_f16_bits(s16f);
                    a.zeros[row * a.n_groups + g] = f32_to_f16_bits(zf + fzoff);
                }
            }
        }
        // quantize column j (owner: lane qj of the row, slot ij).  t = w / S16 correctly
        // rounded: q0 = w r with r = 1 / S16 correctly rounded, then one correction with
        // the exact residual w - q0 S16 (Markstein); equal to the IEEE quotient, whose
        // rounding to an integer is that of the exact w / S16 wherever |t| < 4096 (there a
        // half-integer times S16 is an fp32 number, so t cannot reach or cross one that
        // w / S16 is not).  The code
        // is rne(t) + zf clamped to the grid (zf is an integer, so this is exact).
        const float wv = w[ij];
        const float q0 = wv * r16f;
        const float t = fmaf(fmaf(-q0, s16f, wv), r16f, q0);
        float qd;
        CodeT code;
        if constexpr (FP4) {
            // nearest E2M1 value (ties to the even mantissa, 6 beyond): steps of 0.5
            // below 2, of 1 below 4, of 2 above.  Every candidate is formed and then
            // selected, so the step has no branches (written as nested conditional
            // expressions, the compiler branched on them)
            const float m = fabsf(t);
            const float v_lo = 0.5f * rintf(2.f * m), v_mid = rintf(m), v_hi = fminf(2.f * rintf(0.5f * m), 6.f);
            float v = m < 4.f ? v_mid : v_hi;
            v = m < 2.f ? v_lo : v;
            qd = copysignf(v, t);
            code = qd;
        } else {
            qd = __builtin_amdgcn_fmed3f(rintf(t), lo, hi);
            code = qd + zf;
        }
        const float err = fmaf(-s16f, qd, wv) * idv[ij];
        const float errb = row_bcast<qj>(err);
        const bool own = (q == qj);
        e[ij] = own ? err : e[ij];
        cv[ij] = own ? code : cv[ij];
        // keep both selects in this step (left alone, the compiler moves every step's
        // selects after the last step, holding 128 values live and putting that work on
        // the block's path)
        asm volatile("" : "+v"(e[ij]), "+v"(cv[ij]));
        // compensate the later columns; U is upper triangular, so in slot ij the lanes
        // holding columns <= j get a zero coefficient (or touch a finished column).
        // The slot of the next column first: it is on the critical path.
        constexpr int in = ((j + 1) >> 4) < SSLOTS ? ((j + 1) >> 4) : SSLOTS - 1;
        w[in] = fmaf(-errb, uc[in], w[in]);
#pragma unroll
        for (int i = ij; i < SSLOTS; ++i)
            if (i != in) w[i] = fmaf(-errb, uc[i], w[i]);
    });

    // the next block's diagonal U: the loads are in flight during the error staging and
    // this block's update of the rest of the super-block
    if (bn < a.s1) load_udiag<FULL>(a, bn, (int)((a.s1 - bn) < QB ? (a.s1 - bn) : QB), tid, ud);
    // a non-finite weight, scale or error shows up in the block's errors
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) bad = bad || !(fabsf(e[i]) <= 3.0e38f);
    // the trailing update multiplies on fp16 MFMA with a three-term split of the scaled
    // errors x = e es_r / us_k: the split is formed here once (hi = fp16(x), lo =
    // fp16(x - hi)) instead of in every workgroup of the product; it and the codes are
    // staged in LDS and written as whole 16- / 4-byte pieces
#pragma unroll
    for (int i = 0; i < SSLOTS; ++i) {
        const int c = SL * i + q;
        const float x = (c < nb) ? e[i] * (es_row / usc[i]) : 0.f;
        bad = bad || !(fabsf(x) < 65504.f);
        const uint16_t h = f32_to_f16_bits(x);
        ehs[rl][c] = h;
        els[rl][c] = f32_to_f16_bits(x - f16_bits_to_f32(h));
        if constexpr (FP4) {
            // sign bit 8 | magnitude index (0 .. 7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6); a zero
            // value has no sign bit
            const float v = fabsf(cv[i]);
            int idx = v < 4.f ? (int)v + 2 : (int)(0.5f * v) + 4;
            idx = v < 2.f ? (int)(2.f * v) : idx;
            cl[rl][c] = (uint8_t)(idx + (cv[i] < 0.f ? 8 : 0));
        } else {
            cl[rl][c] = (uint8_t)((int)cv[i] + a.zoff);
        }
    }
    if (bad && rv) atomicOr(&bad_any, 1);
    // the global stores above and below need not have landed
    lds_barrier();
    if (tid == 0 && bad_any) *a.info = -1;

    const int per = a.packed ? 2 : 1;
    {
        // E: thread t writes 8 columns of row t / 16
        const int r = tid >> 4, c8 = (tid & 15) * 8;
        const int64_t grow = (int64_t)blockIdx.x * SROWS + r;
        if (grow < a.d_row) {
            uint16_t* hrow = a.Ehi + grow * a.lde + cb;
            uint16_t* lrow = a.Elo + grow * a.lde + cb;
            if (FULL || nb == QB && (a.lde & 7) == 0 && ((reinterpret_cast<uintptr_t>(hrow) & 15) == 0) &&
                ((reinterpret_cast<uintptr_t>(lrow) & 15) == 0)) {
                *reinterpret_cast<u32x4_t*>(hrow + c8) = *reinterpret_cast<const u32x4_t*>(&ehs[r][c8]);
                *reinterpret_cast<u32x4_t*>(lrow + c8) = *reinterpret_cast<const u32x4_t*>(&els[r][c8]);
            } else {
                for (int c = c8; c < c8 + 8 && c < nb; ++c) { hrow[c] = ehs[r][c]; lrow[c] = els[r][c]; }
            }
        }
        // codes: the 3-bit stream (three bytes per 8 columns; block widths are multiples
        // of 8), two per byte (column 2k in the low nibble) or one per byte; thread t writes
        // 8 columns of row t / 16
        if (a.bits3) {
            if (grow < a.d_row && c8 < nb) {
                uint8_t* crow = a.codes + grow * a.code_ld + (b0 + c8) / 8 * 3;
                uint32_t v = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) v |= (uint32_t)(cl[r][c8 + k] & 7) << (3 * k);
                crow[0] = (uint8_t)v;
                crow[1] = (uint8_t)(v >> 8);
                crow[2] = (uint8_t)(v >> 16);
            }
        } else if (grow < a.d_row) {
            uint8_t* crow = a.codes + grow * a.code_ld + b0 / per;
            const bool whole = FULL || nb == QB && ((reinterpret_cast<uintptr_t>(crow) & (a.packed ? 3 : 7)) == 0);
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

    // the rest of the super-block: W[:, n0 ..] -= E U[b0 .. b0 + 127, n0 ..], 64 columns of
    // U at a time; wave w updates 16 rows x 16 columns of each chunk (its own columns of
    // Wl, so the chunks need no barrier between them)
    if (bn < a.s1) {
        f16x8_t eh[NKK], el[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int mr = lane & 15, ka = 32 * kk + 8 * (lane >> 4);
            eh[kk] = *reinterpret_cast<const f16x8_t*>(&ehs[mr][ka]);
            el[kk] = *reinterpret_cast<const f16x8_t*>(&els[mr][ka]);
        }
        float ri[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ri[r] = einv[4 * (lane >> 4) + r];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            const int64_t n0 = bn + UT_N * ch;
            if (n0 >= a.s1) break;
            f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(eh[kk], uch[ch].h[kk], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(eh[kk], uch[ch].l[kk], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(el[kk], uch[ch].h[kk], acc, 0, 0, 0);
            }
            // D layout: lane l holds column l % 16, rows 4 (l / 16) .. + 3
            const int nc = (int)(n0 - a.s0) + 16 * wave + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) Wl[4 * (lane >> 4) + r][nc] = fmaf(-acc[r], ri[r], Wl[4 * (lane >> 4) + r][nc]);
        }
        lds_barrier();   // the next block reads these columns of Wl
    }
    }   // blocks of the super-block
}

gptq_status sweep_launch(const SweepArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.d_row + SROWS - 1) / SROWS));
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool full = a.s1 - a.s0 == QSB && (a.d_col & 15) == 0 && (a.lde & 7) == 0 && (a.code_ld & 7) == 0 &&
                      al16(a.Wws) && al16(a.U) && al16(a.Ehi) && al16(a.Elo) &&
                      al16(a.codes);
    if (a.fp4) {
        if (full) sweep_kernel<true, true><<<grid, QT, 0, s>>>(a);
        else sweep_kernel<false, true><<<grid, QT, 0, s>>>(a);
    } else {
        if (full) sweep_kernel<true, false><<<grid, QT, 0, s>>>(a);
        else sweep_kernel<false, false><<<grid, QT, 0, s>>>(a);
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
