// The layer's product on its quantized weights, read straight from the stored format:
// y[t][r] = sum_c x[t][c] What[r][c], What[r][c] = S16[r][g] (u[r][c] - z[r][g]), with
// fp32 accumulation.
//
// GPTQ summary page, layer-wise objective (the layer computes W X; with activations
// stored tokens x d_col the output is X W^T) and its results on inference with the
// packed weights; Quantization concepts guide, "Mapping values to fewer bits"
// (x ~= S (q - Z)) and "Data types - int8 and int4" (two int4 values per byte, the
// first in the low nibble; 3-bit codes as a stream, eight in three bytes, the first in
// the lowest bits).
//
// Decode-shaped (one to a few tokens, linear_kernel): the product streams the codes
// once and is bound by their bytes.  A workgroup of four waves owns 4 LROWS rows
// (LROWS per wave); the 64 lanes of a wave take 32-column chunks in turn (lane l:
// chunks l, l + 64, ..), so each wave reads a row's codes as contiguous 1 KB pieces.
// Per chunk the group's scale and zero are loaded once; the 32 products x (u - z) are
// summed in fp32 and scaled by S once (S is factored out of the chunk).  The lanes'
// partial sums of a row are added with a butterfly over the wave.
//
// Batched tokens (linear_mfma_kernel): per token the decode kernel spends an fp32
// multiply-add per weight, so beyond a few tokens the products move to the matrix
// cores (v_mfma_f32_16x16x32 in the activations' own 16-bit type): the activations
// are the A operand (16 tokens), the codes, decoded to u - z in that type, the B
// operand (16 rows), so the decoding is paid once per weight for all the tokens of a
// tile.  u - z is exact in bf16 (f16) when the zero is an integer of magnitude at most
// 240 (2032); otherwise the remainder d - bf16(d) goes through a second product.

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gptq {

struct LinArgs {
    const uint8_t* codes; int64_t code_ld;            // bytes per row
    const uint16_t* scales; const uint16_t* zeros;    // fp16, d_row x n_groups
    int n_groups; int64_t G;                          // group width in columns (d_col when per row)
    const void* x; int64_t ldx; int64_t n_tok;
    void* y; int64_t ldy;
    int64_t d_row, d_col;
};

#ifndef LIN_ROWS
#define LIN_ROWS 2
#endif
constexpr int LROWS = LIN_ROWS;              // rows per wave
#ifndef LIN_WAVES
#define LIN_WAVES 4
#endif
constexpr int LWAVES = LIN_WAVES;
constexpr int LCH = 32;                      // columns per chunk
#ifndef LIN_MFMA_MIN_TOK
#define LIN_MFMA_MIN_TOK 2                   // fewest tokens taken by the batched kernel
#endif

template <gptq_dtype DT>
GPTQ_DEV void load_x8(const void* base, int64_t idx, float (&v)[8]) {   // 8 values, 16-byte aligned
    if constexpr (DT == GPTQ_F32) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(base) + idx);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(base) + idx + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
    } else {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(base) + idx);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint16_t lo = (uint16_t)(w[e] & 0xffffu), hi = (uint16_t)(w[e] >> 16);
            if constexpr (DT == GPTQ_BF16) { v[2 * e] = bf16_bits_to_f32(lo); v[2 * e + 1] = bf16_bits_to_f32(hi); }
            else { v[2 * e] = f16_bits_to_f32(lo); v[2 * e + 1] = f16_bits_to_f32(hi); }
        }
    }
}

template <gptq_dtype YT>
GPTQ_DEV void store_y(void* y, int64_t idx, float v) {
    if constexpr (YT == GPTQ_F32) reinterpret_cast<float*>(y)[idx] = v;
    else if constexpr (YT == GPTQ_BF16) reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_bits(v);
    else reinterpret_cast<uint16_t*>(y)[idx] = f32_to_f16_bits(v);
}

GPTQ_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Code e (0 .. 31) of a 32-column chunk held in words w: CB = 4, word 2 (e / 8) + (e & 1)
// holds column e in byte (e & 7) / 2 (the nibbles split into even and odd bytes); CB = 3,
// the 96-bit stream of the chunk, code e in bits 3e .. 3e + 2; CB = 8, byte e & 3 of word
// e / 4.
template <int CB>
GPTQ_DEV uint32_t chunk_code(const uint32_t* w, int e) {
    if constexpr (CB == 3) {
        const int bit = 3 * e, k = bit >> 5, sh = bit & 31;
        return sh <= 29 ? (w[k] >> sh) & 7u : ((w[k] >> sh) | (w[k + 1] << (32 - sh))) & 7u;
    } else if constexpr (CB == 4) {
        return (w[2 * (e >> 3) + (e & 1)] >> (8 * ((e & 7) >> 1))) & 0xFFu;
    } else {
        return (w[e >> 2] >> (8 * (e & 3))) & 0xFFu;
    }
}

// Fast path: d_col a multiple of 32, rows of codes 16-byte (3-bit: 4-byte) and of x
// 16-byte aligned.  NT tokens per pass; CB = code bits as stored: 4 (two codes per byte,
// 16 bytes per chunk), 3 (the 3-bit stream, 12 bytes per chunk) or 8 (32 bytes).
template <int CB, int NT, gptq_dtype XT, gptq_dtype YT>
__global__ __launch_bounds__(64 * LWAVES) void linear_kernel(LinArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = ((int64_t)blockIdx.x * LWAVES + wave) * LROWS;
    const int nch = (int)(a.d_col / LCH);
    for (int64_t t0 = 0; t0 < a.n_tok; t0 += NT) {
        float acc[LROWS][NT];
#pragma unroll
        for (int i = 0; i < LROWS; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[i][t] = 0.f;
        for (int j = lane; j < nch; j += 64) {
            const int64_t c0 = (int64_t)j * LCH;
            float xv[NT][LCH];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int64_t tt = (t0 + t < a.n_tok) ? t0 + t : a.n_tok - 1;   // a repeated token past the end
#pragma unroll
                for (int q = 0; q < LCH / 8; ++q) {
                    float v8[8];
                    load_x8<XT>(a.x, tt * a.ldx + c0 + 8 * q, v8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) xv[t][8 * q + e] = v8[e];
                }
            }
            const int g = (int)(c0 / a.G);
            // every row's codes, scale and zero first (rows past the end re-read the last
            // row; their sums are not stored), so the loads are in flight together
            uint32_t cw[LROWS][8];
            float S[LROWS], z[LROWS];
#pragma unroll
            for (int i = 0; i < LROWS; ++i) {
                const int64_t r = (r0 + i < a.d_row) ? r0 + i : a.d_row - 1;
                const uint8_t* crow = a.codes + r * a.code_ld;
                if constexpr (CB == 3) {
                    const uint32_t* w = reinterpret_cast<const uint32_t*>(crow + c0 / 8 * 3);
#pragma unroll
                    for (int e = 0; e < 3; ++e) cw[i][e] = w[e];
                } else if constexpr (CB == 4) {
                    // nibbles 0, 2, 4, .. and 1, 3, 5, .. of a word as bytes
                    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(crow + c0 / 2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        cw[i][2 * e] = w[e] & 0x0F0F0F0Fu;
                        cw[i][2 * e + 1] = (w[e] >> 4) & 0x0F0F0F0Fu;
                    }
                } else {
                    const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(crow + c0);
                    const u32x4_t w1 = *reinterpret_cast<const u32x4_t*>(crow + c0 + 16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { cw[i][e] = w0[e]; cw[i][4 + e] = w1[e]; }
                }
                S[i] = f16_bits_to_f32(a.scales[r * a.n_groups + g]);
                z[i] = f16_bits_to_f32(a.zeros[r * a.n_groups + g]);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep every load above the arithmetic
#pragma unroll
            for (int i = 0; i < LROWS; ++i) {
                float s[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) s[t] = 0.f;
#pragma unroll
                for (int e = 0; e < LCH; ++e) {
                    const float d = (float)chunk_code<CB>(cw[i], e) - z[i];   // exact: small integers
#pragma unroll
                    for (int t = 0; t < NT; ++t) s[t] = fmaf(xv[t][e], d, s[t]);
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[i][t] = fmaf(S[i], s[t], acc[i][t]);
            }
        }
#pragma unroll
        for (int i = 0; i < LROWS; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float v = wave_sum(acc[i][t]);
                const int64_t r = r0 + i;
                if (lane == 0 && r < a.d_row && t0 + t < a.n_tok) store_y<YT>(a.y, (t0 + t) * a.ldy + r, v);
            }
    }
}

// General path (any even d_col, any alignment): one thread per (row, token), columns in
// order; the same arithmetic per group.
template <int CB, gptq_dtype XT, gptq_dtype YT>
__global__ __launch_bounds__(256) void linear_any_kernel(LinArgs a) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= a.d_row) return;
    const uint8_t* crow = a.codes + r * a.code_ld;
    for (int64_t t = blockIdx.y; t < a.n_tok; t += gridDim.y) {
        float acc = 0.f;
        for (int64_t c0 = 0; c0 < a.d_col; c0 += a.G) {
            const int g = (int)(c0 / a.G);
            const float S = f16_bits_to_f32(a.scales[r * a.n_groups + g]);
            const float z = f16_bits_to_f32(a.zeros[r * a.n_groups + g]);
            const int64_t c1 = (c0 + a.G < a.d_col) ? c0 + a.G : a.d_col;
            float s = 0.f;
            for (int64_t c = c0; c < c1; ++c) {
                const uint32_t u = CB == 3 ? code3(load_u24(crow + c / 8 * 3), (int)(c & 7))
                                   : CB == 4 ? (crow[c >> 1] >> (4 * (c & 1))) & 0xFu : crow[c];
                s = fmaf(load_as_f32<XT>(a.x, t * a.ldx + c), (float)u - z, s);
            }
            acc = fmaf(S, s, acc);
        }
        store_y<YT>(a.y, t * a.ldy + r, acc);
    }
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

#ifndef LIN_MW
#define LIN_MW 8
#endif
#ifndef LIN_CPW1
#define LIN_CPW1 2
#endif
#ifndef LIN_CPW2
#define LIN_CPW2 1
#endif
#ifndef LIN_CPW4
#define LIN_CPW4 1
#endif
#ifndef LIN_NTT_MAX
#define LIN_NTT_MAX 4
#endif
#ifndef LIN_RB
#define LIN_RB 2
#endif
constexpr int MW = LIN_MW;   // waves per workgroup of the batched kernel, each a share of the chunks
constexpr int MCK = 128;     // columns per chunk: four 32-deep products, one scale

// Batched kernel: a workgroup owns 16 RB rows and 16 NTT tokens; its waves take the
// rows' 128-column chunks in turn (wave w: chunks w, w + 8, ..).  Within a chunk lane l
// reads the 16 code bytes 16 (l / 16) .. + 15 of row l % 16 of each 16-row block
// (columns 32 (l / 16) .. + 31) and the same 32 columns of token l % 16 of each token
// tile; product t of the chunk takes columns 32 (l / 16) + 8 t .. + 7 from every lane,
// so over its four products the chunk's 128 columns each enter once (the order of a
// sum's terms is the only thing this changes).  Each activation fragment serves the RB
// row blocks, so the activations are read from L2 once per 16 RB rows.  Requires 4-bit
// (16 bytes per lane, 16-byte aligned rows) or 3-bit codes (12 bytes per lane, 4-byte
// aligned rows), 16-bit activations, d_col and the group width multiples of 128,
// 16-byte aligned activation rows.
template <int CB, int NTT, int RB, gptq_dtype XT, gptq_dtype YT>
__global__ __launch_bounds__(64 * MW) void linear_mfma_kernel(LinArgs a) {
    typedef std::conditional_t<XT == GPTQ_BF16, bf16x8_t, f16x8_t> frag_t;
    typedef std::conditional_t<XT == GPTQ_BF16, __bf16, _Float16> elem_t;
    constexpr float ZMAX = XT == GPTQ_BF16 ? 240.f : 2032.f;   // |u - z| <= 255 (2047): exact
    constexpr int CPW = NTT == 1 ? LIN_CPW1 : NTT == 2 ? LIN_CPW2 : LIN_CPW4;  // chunks per wave per pass
    __shared__ float red[MW][NTT * RB][4][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n16 = lane & 15, q = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * 16 * RB;
    const uint8_t* crow[RB];
    int64_t rr[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int64_t row = row0 + 16 * rb + n16;
        rr[rb] = row < a.d_row ? row : a.d_row - 1;              // rows past the end re-read the last
        crow[rb] = a.codes + rr[rb] * a.code_ld + (CB == 3 ? 12 : 16) * q;
    }
    const int64_t tok0 = (int64_t)blockIdx.y * 16 * NTT;
    const uint16_t* xrow[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        int64_t t = tok0 + 16 * tt + n16;
        t = t < a.n_tok ? t : a.n_tok - 1;                      // a repeated token past the end
        xrow[tt] = reinterpret_cast<const uint16_t*>(a.x) + t * a.ldx + 32 * q;
    }
    const int nck = (int)(a.d_col / MCK);
    const int cpg = (int)(a.G / MCK);
    f32x4_t acc[NTT][RB];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[tt][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = wave; c0 < nck; c0 += MW * CPW) {
        u32x4_t cw[CPW][RB], xw[CPW][NTT][4];
        float S[CPW][RB], z[CPW][RB];
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const int c = c0 + MW * j < nck ? c0 + MW * j : c0;  // chunks past the end re-read c0
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                if constexpr (CB == 3) {
                    const uint32_t* w = reinterpret_cast<const uint32_t*>(crow[rb] + (int64_t)c * (MCK / 8 * 3));
                    cw[j][rb] = u32x4_t{w[0], w[1], w[2], 0u};
                } else {
                    cw[j][rb] = *reinterpret_cast<const u32x4_t*>(crow[rb] + (int64_t)c * (MCK / 2));
                }
                const int64_t gi = rr[rb] * a.n_groups + c / cpg;
                S[j][rb] = f16_bits_to_f32(a.scales[gi]);
                z[j][rb] = f16_bits_to_f32(a.zeros[gi]);
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    xw[j][tt][t] = *reinterpret_cast<const u32x4_t*>(xrow[tt] + (int64_t)c * MCK + 8 * t);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep every load above the arithmetic
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            if (c0 + MW * j >= nck) break;   // wave-uniform
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const bool exact = z[j][rb] == rintf(z[j][rb]) && fabsf(z[j][rb]) <= ZMAX;
                const bool need_lo = __ballot(!exact) != 0;
                f32x4_t cs[NTT];
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) cs[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // element e of the operand is column 8 t + e of the lane's 32: 4-bit, the
                    // low nibble of byte e / 2 for even e, the high nibble for odd e; 3-bit,
                    // code e of the 24-bit group t of the lane's 96-bit stream
                    float d[8];
                    if constexpr (CB == 3) {
                        const u32x4_t cc = cw[j][rb];
                        const uint32_t g24 = t == 0 ? cc[0] & 0xFFFFFFu
                                           : t == 1 ? ((cc[0] >> 24) | (cc[1] << 8)) & 0xFFFFFFu
                                           : t == 2 ? ((cc[1] >> 16) | (cc[2] << 16)) & 0xFFFFFFu
                                                    : cc[2] >> 8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) d[e] = (float)code3(g24, e) - z[j][rb];
                    } else {
                        const uint32_t w = cw[j][rb][t];
                        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            d[2 * b] = (float)((lo >> (8 * b)) & 0xFFu) - z[j][rb];
                            d[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu) - z[j][rb];
                        }
                    }
                    frag_t bh;
#pragma unroll
                    for (int e = 0; e < 8; ++e) bh[e] = (elem_t)d[e];
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt) {
                        const frag_t xa = __builtin_bit_cast(frag_t, xw[j][tt][t]);
                        if constexpr (XT == GPTQ_BF16) cs[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bh, cs[tt], 0, 0, 0);
                        else cs[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, bh, cs[tt], 0, 0, 0);
                    }
                    if (need_lo) {
                        frag_t bl;
#pragma unroll
                        for (int e = 0; e < 8; ++e) bl[e] = (elem_t)(d[e] - (float)bh[e]);
#pragma unroll
                        for (int tt = 0; tt < NTT; ++tt) {
                            const frag_t xa = __builtin_bit_cast(frag_t, xw[j][tt][t]);
                            if constexpr (XT == GPTQ_BF16) cs[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bl, cs[tt], 0, 0, 0);
                            else cs[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, bl, cs[tt], 0, 0, 0);
                        }
                    }
                }
                // lane l holds the sums of row l % 16 of block rb for tokens 4 (l / 16) + i
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[tt][rb][i] = fmaf(S[j][rb], cs[tt][i], acc[tt][rb][i]);
            }
        }
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][tt * RB + rb][i][lane] = acc[tt][rb][i];
    __syncthreads();
    // output o: token tile o / (256 RB), row block (o / 256) % RB, token m = (o / 16) % 16
    // of the tile, row n = o % 16; its partial sums sit in lane n + 16 (m / 4), register
    // m % 4, of every wave
    for (int o = threadIdx.x; o < NTT * RB * 256; o += 64 * MW) {
        const int tr = o >> 8, m = (o >> 4) & 15, n = o & 15;
        const int tt = tr / RB, rb = tr % RB;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < MW; ++w) v += red[w][tr][m & 3][n + 16 * (m >> 2)];
        const int64_t t = tok0 + 16 * tt + m, r = row0 + 16 * rb + n;
        if (t < a.n_tok && r < a.d_row) store_y<YT>(a.y, t * a.ldy + r, v);
    }
}

template <int CB, gptq_dtype XT, gptq_dtype YT>
static void launch_mfma(const LinArgs& a, hipStream_t s) {
    // 16 tokens or fewer: 16-row workgroups (enough of them to fill the device); beyond,
    // 32-row workgroups, so that each activation fragment serves two row blocks and the
    // activations are read from L2 half as often; 64-row workgroups once there are
    // enough of them
    const unsigned g16 = (unsigned)((a.d_row + 15) / 16), g32 = (unsigned)((a.d_row + 31) / 32);
    if (a.n_tok <= 16 || LIN_NTT_MAX == 1)
        linear_mfma_kernel<CB, 1, 1, XT, YT><<<dim3(g16, (unsigned)((a.n_tok + 15) / 16)), 64 * MW, 0, s>>>(a);
    else if (a.n_tok <= 32)
        linear_mfma_kernel<CB, 1, LIN_RB, XT, YT><<<dim3(LIN_RB == 2 ? g32 : g16, (unsigned)((a.n_tok + 15) / 16)), 64 * MW, 0, s>>>(a);
    else if (a.n_tok <= 64 || LIN_NTT_MAX == 2)
        linear_mfma_kernel<CB, 2, LIN_RB, XT, YT><<<dim3(LIN_RB == 2 ? g32 : g16, (unsigned)((a.n_tok + 31) / 32)), 64 * MW, 0, s>>>(a);
    else if ((int64_t)((a.d_row + 63) / 64) * ((a.n_tok + 63) / 64) >= 256)
        // enough 64-row x 64-token workgroups to fill the device: each activation fragment
        // serves four row blocks (1 workgroup per CU: 128 KB of LDS for the reduction)
        linear_mfma_kernel<CB, 4, 4, XT, YT><<<dim3((unsigned)((a.d_row + 63) / 64), (unsigned)((a.n_tok + 63) / 64)), 64 * MW, 0, s>>>(a);
    else linear_mfma_kernel<CB, 4, LIN_RB, XT, YT><<<dim3(LIN_RB == 2 ? g32 : g16, (unsigned)((a.n_tok + 63) / 64)), 64 * MW, 0, s>>>(a);
}

template <int CB, gptq_dtype XT, gptq_dtype YT>
static gptq_status launch3(const LinArgs& a, int path, hipStream_t s) {
    if constexpr (CB != 8 && XT != GPTQ_F32) {
        if (path == 2) {
            launch_mfma<CB, XT, YT>(a, s);
            GPTQ_LAUNCH_CHECK();
            return GPTQ_OK;
        }
    }
    const bool fast = path >= 1;
    if (!fast) {
        const unsigned ty = (unsigned)(a.n_tok < 65535 ? a.n_tok : 65535);
        linear_any_kernel<CB, XT, YT><<<dim3((unsigned)((a.d_row + 255) / 256), ty), 256, 0, s>>>(a);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    const dim3 grid((unsigned)((a.d_row + LWAVES * LROWS - 1) / (LWAVES * LROWS)));
    if (a.n_tok == 1) linear_kernel<CB, 1, XT, YT><<<grid, 64 * LWAVES, 0, s>>>(a);
    else if (a.n_tok == 2) linear_kernel<CB, 2, XT, YT><<<grid, 64 * LWAVES, 0, s>>>(a);
    else linear_kernel<CB, 4, XT, YT><<<grid, 64 * LWAVES, 0, s>>>(a);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

template <int CB, gptq_dtype XT>
static gptq_status launch2(const LinArgs& a, gptq_dtype yt, int path, hipStream_t s) {
    switch (yt) {
        case GPTQ_F32: return launch3<CB, XT, GPTQ_F32>(a, path, s);
        case GPTQ_BF16: return launch3<CB, XT, GPTQ_BF16>(a, path, s);
        case GPTQ_F16: return launch3<CB, XT, GPTQ_F16>(a, path, s);
    }
    return GPTQ_ERR_UNSUPPORTED;
}

template <int CB>
static gptq_status launch1(const LinArgs& a, gptq_dtype xt, gptq_dtype yt, int path, hipStream_t s) {
    switch (xt) {
        case GPTQ_F32: return launch2<CB, GPTQ_F32>(a, yt, path, s);
        case GPTQ_BF16: return launch2<CB, GPTQ_BF16>(a, yt, path, s);
        case GPTQ_F16: return launch2<CB, GPTQ_F16>(a, yt, path, s);
    }
    return GPTQ_ERR_UNSUPPORTED;
}

gptq_status linear_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t d_row,
                          int64_t d_col, int bits, int group_size, const void* x, gptq_dtype x_dtype, int64_t n_tok,
                          int64_t ldx, void* y, gptq_dtype y_dtype, hipStream_t s) {
    LinArgs a;
    const int cb = bits == 3 ? 3 : bits == 4 ? 4 : 8;     // code bits as stored
    a.codes = codes; a.code_ld = cb == 3 ? d_col / 8 * 3 : cb == 4 ? d_col / 2 : d_col;
    a.scales = scales; a.zeros = zeros;
    a.G = group_size == 0 ? d_col : group_size;
    a.n_groups = (int)(d_col / a.G);
    a.x = x; a.ldx = ldx; a.n_tok = n_tok;
    a.y = y; a.ldy = d_row;
    a.d_row = d_row; a.d_col = d_col;
    const size_t xsz = x_dtype == GPTQ_F32 ? 4 : 2;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    // whole 32-column chunks inside one group, every chunk of codes 16-byte aligned (3-bit:
    // 4-byte; its chunks are 12 bytes) and of x 16-byte aligned
    const int cal = cb == 3 ? 4 : 16;
    const bool fast = d_col % LCH == 0 && a.G % LCH == 0 && (a.code_ld % cal) == 0 &&
                      (reinterpret_cast<uintptr_t>(codes) % cal) == 0 && al16(x) && ((size_t)ldx * xsz) % 16 == 0;
    // batched tokens on the matrix cores: 3- or 4-bit codes, 16-bit activations, whole
    // 128-column chunks inside one group
    const bool mfma = fast && cb != 8 && x_dtype != GPTQ_F32 && n_tok >= LIN_MFMA_MIN_TOK && d_col % MCK == 0 &&
                      a.G % MCK == 0;
    const int path = mfma ? 2 : fast ? 1 : 0;
    return cb == 3 ? launch1<3>(a, x_dtype, y_dtype, path, s)
         : cb == 4 ? launch1<4>(a, x_dtype, y_dtype, path, s) : launch1<8>(a, x_dtype, y_dtype, path, s);
}

}  // namespace gptq
