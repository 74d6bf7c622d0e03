// Internal declarations shared by the quantization kernels.
#pragma once
#include "common.h"

namespace gptq {

// A scale is usable when fp16 holds it as a normal number.
GPTQ_DEV bool normal_f16_scale(float s) { return s >= 6.103515625e-05f && s <= 65504.f; }

// S16 and the stored zero of one range: [mn, mx] (asymmetric; a constant range is
// widened to include 0) or its absolute maximum (symmetric); *info = -1 when the scale
// is not a normal fp16 number.
// The smallest power of two not below x > 0 (exact: from the exponent of x).
GPTQ_DEV float pow2_ceil(float x) {
    int e;
    const float m = frexpf(x, &e);   // x = m 2^e, m in [0.5, 1)
    return ldexpf(1.f, m == 0.5f ? e - 1 : e);
}

// FP4: the E2M1 grid (largest magnitude 6), one scale, stored zero 0; pow2: the scale
// rounded up to a power of two (MXFP4).
template <int BITS, bool SYM, bool FP4 = false>
GPTQ_DEV void range_params(float mn, float mx, int32_t* info, uint16_t& s_out, uint16_t& z_out, bool pow2 = false) {
    constexpr int QMIN = SYM ? -((1 << (BITS - 1)) - 1) : 0;
    constexpr int QMAX = FP4 ? 6 : SYM ? ((1 << (BITS - 1)) - 1) : (1 << BITS) - 1;
    constexpr int ZOFF = (SYM && !FP4) ? (1 << (BITS - 1)) : 0;
    float s, zf = 0.f;
    if (SYM || FP4) {
        const float am = fmaxf(fabsf(mn), fabsf(mx));
        s = am > 0.f ? am / (float)QMAX : 1.f;
    } else {
        if (mn == mx) { mn = fminf(mn, 0.f); mx = fmaxf(mx, 0.f); }
        s = (mx > mn) ? (mx - mn) / (float)(QMAX - QMIN) : 1.f;
    }
    if (FP4 && pow2) s = pow2_ceil(s);
    float s16f = f16_bits_to_f32(f32_to_f16_bits(s));
    if (!normal_f16_scale(s16f)) { *info = -1; s16f = 1.f; }
    if (!SYM && !FP4) zf = (float)QMIN - rintf(mn / s16f);
    s_out = f32_to_f16_bits(s16f);
    z_out = f32_to_f16_bits(zf + (float)ZOFF);
}


constexpr int QB = 128;             // lazy-update block width (columns)
constexpr int QT = 256;             // threads per sweep workgroup
constexpr int SL = 16;              // lanes per row in the sweep (one DPP row)
constexpr int SROWS = QT / SL;      // rows per sweep workgroup
// Super-block of the deferred trailing update: the sweep of its blocks and the updates
// inside it run in one launch; the columns after it get one product with K = QSB.
constexpr int QSB = 512;

struct SweepArgs {
    const float* Wws; int64_t d_row, d_col;
    const float* U;                 // fp32 U (the diagonal blocks for the sweep)
    // this super-block's diagonal QSB x QSB part of U, row k scaled by us_k and split into
    // fp16 hi + lo, zero past d_col, in MFMA B-operand order (the updates inside the
    // super-block)
    const uint16_t* Uthi; const uint16_t* Utlo;
    int64_t s0, s1;                 // the super-block: columns s0 .. s1 - 1 (s1 - s0 <= QSB)
    uint16_t* Ehi; uint16_t* Elo;   // the super-block's errors e, scaled to x = e es_r / us_k, as
    int64_t lde;                    // fp16 hi + lo (hi = fp16(x), lo = fp16(x - hi)): d_row x QSB,
                                    // row stride lde
    const float* es;                // es_r per row and us_k per column (exact powers of two)
    const float* us;
    uint8_t* codes; int64_t code_ld;
    uint16_t* scales; uint16_t* zeros; int n_groups;
    int32_t* info;
    int group;                      // 32, 64, 128 (power of two), or 0 = per-row params precomputed
    int qmin, qmax, zoff;           // grid and stored-code offset
    int sym; int packed;            // packed: two codes per byte
    int bits3;                      // 3-bit stream: eight codes in three bytes
    int fp4;                        // E2M1 grid (sign bit 8 | magnitude index), zero 0
    int mx;                         // with fp4: power-of-two group scales (MXFP4)
};

gptq_status sweep_launch(const SweepArgs& a, hipStream_t s);

}  // namespace gptq
