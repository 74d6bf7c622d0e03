// Internal declarations shared by the quantization kernels.
#pragma once
#include "common.h"

namespace gptq {

// A scale is usable when fp16 holds it as a normal number.
GPTQ_DEV bool normal_f16_scale(float s) { return s >= 6.103515625e-05f && s <= 65504.f; }

// The smallest power of two not below x > 0 (exact: from the exponent of x).
GPTQ_DEV float pow2_ceil(float x) {
    int e;
    const float m = frexpf(x, &e);   // x = m 2^e, m in [0.5, 1)
    return ldexpf(1.f, m == 0.5f ? e - 1 : e);
}

// The scale, the zero point and the codes are roundings of exact quotients, and the
// kernels decide them exactly from their own fp32 values.  For a quotient x / d of an fp32
// x by a d that is a small integer or an fp16 value, the correctly rounded fp32 quotient
// already rounds the same way as x / d: a rounding boundary b (an fp16 midpoint, or a
// half-integer below 4096 in magnitude) has at most 13 significant bits, so b d is an
// fp32 number, x != b d puts x at least one ulp of b d away, and x / d more than half an
// ulp of b away from b; the fp32 quotient can then neither reach b nor cross it.  Only a
// range mx - mn that is itself rounded needs more:
//
// fp16 (nearest even) of x / den, x = xh + xl > 0 with xl the rounding error of xh, den a
// positive integer up to 255.  The fp16 rounding c of the fp32 quotient s can be wrong
// only where x / den and s lie on either side of the midpoint m between c and c's fp16
// neighbour n on the side of s, or s is m itself.  m has at most 13 significant bits, so
// den m is exact, xh - den m is exact (both within a factor 2 of each other), and the
// rounded sum (xh - den m) + xl has the sign of x - den m.
GPTQ_DEV float f16_of_quotient(float xh, float xl, float den) {
    const float s = xh / den;
    const uint16_t h = f32_to_f16_bits(s);
    const float c = f16_bits_to_f32(h);
    if (s == c || h == 0 || h >= 0x7BFF) return c;   // exact, or at the ends of the range
    const uint16_t hn = s > c ? (uint16_t)(h + 1) : (uint16_t)(h - 1);
    const float n = f16_bits_to_f32(hn);
    const float m = 0.5f * (c + n);
    const float r = (xh - den * m) + xl;
    if (r == 0.f) return (h & 1) ? n : c;            // x / den = m: the even neighbour
    return ((r > 0.f) == (n > c)) ? n : c;
}

// fp16 scale of a range, before the check that it is a normal fp16 number: (mx - mn) /
// (qmax - qmin) for the asymmetric grid (mx > mn; the difference taken exactly as a
// rounded value plus its error), am / qmax for the symmetric and E2M1 grids (am > 0);
// pow2 (MXFP4, qmax = 6): the smallest power of two not below am / 6 (exact from the
// fp32 quotient by the argument above, with the powers of two as boundaries).
GPTQ_DEV float range_scale16(bool absmax, float mn, float mx, float am, float qspan, bool pow2) {
    if (absmax) return f16_bits_to_f32(f32_to_f16_bits(pow2 ? pow2_ceil(am / qspan) : am / qspan));
    const float xh = mx - mn;
    const float bb = xh - mx;
    const float xl = (mx - (xh - bb)) + (-mn - bb);   // xh + xl = mx - mn exactly
    return f16_of_quotient(xh, xl, qspan);
}

// S16 and the stored zero of one range: [mn, mx] (asymmetric; a constant range is
// widened to include 0) or its absolute maximum (symmetric); *info = -1 when the scale
// is not a normal fp16 number.  FP4: the E2M1 grid (largest magnitude 6), one scale,
// stored zero 0; pow2: the scale rounded up to a power of two (MXFP4).
template <int BITS, bool SYM, bool FP4 = false>
GPTQ_DEV void range_params(float mn, float mx, int32_t* info, uint16_t& s_out, uint16_t& z_out, bool pow2 = false) {
    constexpr int QMIN = SYM ? -((1 << (BITS - 1)) - 1) : 0;
    constexpr int QMAX = FP4 ? 6 : SYM ? ((1 << (BITS - 1)) - 1) : (1 << BITS) - 1;
    constexpr int ZOFF = (SYM && !FP4) ? (1 << (BITS - 1)) : 0;
    float s16f, zf = 0.f;
    if (SYM || FP4) {
        const float am = fmaxf(fabsf(mn), fabsf(mx));
        s16f = am > 0.f ? range_scale16(true, 0.f, 0.f, am, (float)QMAX, FP4 && pow2) : 1.f;
    } else {
        if (mn == mx) { mn = fminf(mn, 0.f); mx = fmaxf(mx, 0.f); }
        s16f = (mx > mn) ? range_scale16(false, mn, mx, 0.f, (float)(QMAX - QMIN), false) : 1.f;
    }
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
