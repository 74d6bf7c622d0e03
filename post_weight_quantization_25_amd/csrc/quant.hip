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
// The in-block column sweep is in sweep.hip.  This file holds the per-row
// scale/zero of group_size 0, the working-copy conversion, the trailing lazy
// update W[:, b1:] -= E U[b0:b1, b1:] on v_mfma_f32_32x32x16_bf16 with both
// operands split into bf16 hi + lo (three products, fp32 accumulation), the
// host-side block loop, and dequantization.

#include <mutex>

#include "kernels.h"
#include "quant_internal.h"

namespace gptq {


// --------------------------------------------------------------------------
// One scale/zero per row (group_size 0): from the original row, before any update.
template <int BITS, bool SYM, bool FP4>
__global__ __launch_bounds__(256) void row_params_kernel(const float* Wws, int64_t d_col, uint16_t* scales,
                                                         uint16_t* zeros, int32_t* info, int pow2 = 0) {
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
    range_params<BITS, SYM, FP4>(smn[0], smx[0], info, scales[row], zeros[row], pow2 != 0);
}

// Per-tensor granularity (one range for the whole matrix; Quantization concepts
// guide, "Choose granularity"): min and max of every block's share of the working
// copy, then one block reduces the partial ranges and gives every row the same S16
// and zero.
__global__ __launch_bounds__(256) void tensor_minmax_kernel(const float* Wws, int64_t n, float* part) {
    __shared__ float smn[256], smx[256];
    float mn = INFINITY, mx = -INFINITY;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const float v = Wws[i];
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
    if (threadIdx.x == 0) { part[2 * blockIdx.x] = smn[0]; part[2 * blockIdx.x + 1] = smx[0]; }
}

template <int BITS, bool SYM, bool FP4>
__global__ __launch_bounds__(256) void tensor_params_kernel(const float* part, int nb, int64_t d_row,
                                                            uint16_t* scales, uint16_t* zeros, int32_t* info,
                                                            int pow2 = 0) {
    __shared__ float smn[256], smx[256];
    __shared__ uint16_t sz[2];
    float mn = INFINITY, mx = -INFINITY;
    for (int i = threadIdx.x; i < nb; i += 256) { mn = fminf(mn, part[2 * i]); mx = fmaxf(mx, part[2 * i + 1]); }
    smn[threadIdx.x] = mn; smx[threadIdx.x] = mx;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if ((int)threadIdx.x < st) {
            smn[threadIdx.x] = fminf(smn[threadIdx.x], smn[threadIdx.x + st]);
            smx[threadIdx.x] = fmaxf(smx[threadIdx.x], smx[threadIdx.x + st]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) range_params<BITS, SYM, FP4>(smn[0], smx[0], info, sz[0], sz[1], pow2 != 0);
    __syncthreads();
    for (int64_t r = threadIdx.x; r < d_row; r += 256) { scales[r] = sz[0]; zeros[r] = sz[1]; }
}

// W (any dtype) -> fp32 working copy, one workgroup per row; flags non-finite values and
// writes the row's error scale es_r = 2^(17 - e), |W[r][:]| < 2^e (frexp of the row's
// largest magnitude): the scaled errors E[r][k] es_r / us_k of the trailing update then
// stay well inside fp16's normal range (|E| / us_k is about |err| max_j |U[k][j]| /
// U[k][k] 2^-13.5, and the errors are a fraction of the row's magnitude).  Eight values
// per thread and step with 16-byte accesses when the rows are 16-byte aligned; otherwise
// one value at a time.
template <gptq_dtype DT>
__global__ __launch_bounds__(256) void convert_kernel(const void* W, int64_t d_col, float* out, float* es,
                                                      int32_t* info) {
    __shared__ float red[4];
    constexpr int EB = (DT == GPTQ_F32) ? 4 : 2;
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const char* src = reinterpret_cast<const char*>(W) + row * d_col * EB;
    float* dst = out + row * d_col;
    const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0) && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0);
    const int64_t n8 = vec ? d_col / 8 : 0;
    int bad = 0;
    float m = 0.f;
    for (int64_t i = tid; i < n8; i += 256) {
        float v[8];
        if constexpr (DT == GPTQ_F32) {
            const f32x4_t a = reinterpret_cast<const f32x4_t*>(src)[2 * i], b = reinterpret_cast<const f32x4_t*>(src)[2 * i + 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
        } else {
            const u32x4_t h = reinterpret_cast<const u32x4_t*>(src)[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t lo = (uint16_t)(h[e] & 0xFFFFu), hi = (uint16_t)(h[e] >> 16);
                v[2 * e] = (DT == GPTQ_BF16) ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
                v[2 * e + 1] = (DT == GPTQ_BF16) ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { bad |= !isfinite(v[e]); m = fmaxf(m, fabsf(v[e])); }
        f32x4_t* o = reinterpret_cast<f32x4_t*>(dst) + 2 * i;
        o[0] = f32x4_t{v[0], v[1], v[2], v[3]};
        o[1] = f32x4_t{v[4], v[5], v[6], v[7]};
    }
    for (int64_t c = 8 * n8 + tid; c < d_col; c += 256) {
        const float v = load_as_f32<DT>(W, row * d_col + c);
        bad |= !isfinite(v);
        m = fmaxf(m, fabsf(v));
        dst[c] = v;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    if (bad) *info = -1;
    __syncthreads();
    if (tid == 0) {
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        int e = 0;
        (void)frexpf(m, &e);
        es[row] = (m > 0.f && m <= 3.0e38f) ? ldexpf(1.f, 17 - e) : 1.f;
    }
}

// --------------------------------------------------------------------------
// Trailing lazy update: W[:, n_beg:n_end] -= E[:, :K] U[k0:k0+K, n_beg:n_end] on
// fp16 MFMA (v_mfma_f32_32x32x16_f16) with a three-term split of scaled fp32
// operands: x = hi + lo with hi = fp16(x), lo = fp16(x - hi), and
// E U ~= Ehi Uhi + Ehi Ulo + Elo Uhi (the dropped Elo Ulo and the residuals are
// ~2^-22 relative per product), accumulated in fp32.  fp16 keeps 11 bits where bf16
// keeps 8, but not its range, so both operands are scaled by exact powers of two that
// cancel: row k of U by us_k (its largest magnitude into [2^13, 2^14)), E[r][k] by
// es_r / us_k (es_r from row r's largest weight), and the product of row r by 1 / es_r.
// With bf16 (hi + lo) the per-product error was ~2^-17, which moved the values the
// codes are decided from by ~1e-6 of a step on the widest layers.
// 128 x 128 output tiles, four waves of 64 x 64 (2 x 2 MFMA 32 x 32 tiles); K in
// chunks of 32 staged in LDS as bf16: E row-major ([m][k], 8 consecutive k per
// 16-byte read), U as it lies in memory ([k][n]) and read transposed with
// ds_read_b64_tr_b16.  The next chunk is loaded into registers while the current
// one is multiplied.
constexpr int TB = 128, TK = 32;
constexpr int TE_LD = TK + 8;       // E rows in LDS: 40 bf16 = 80 B (conflict-free 16 B reads)
constexpr int TU_RS = TB + 16;      // U rows in LDS: 144 bf16 = 72 dwords (conflict-free transposed reads)

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

struct TrailArgs {
    float* Wws; int64_t d_row, d_col;
    const uint16_t* Ehi; const uint16_t* Elo; int64_t lde;   // scaled E block (fp16 hi + lo): d_row x K
    const uint16_t* Uhi; const uint16_t* Ulo;                // scaled U (fp16 hi + lo), d_col x d_col
    const float* erow;                                       // es_r per row (the product is divided by it)
    int64_t k0; int K;
    int64_t n_beg, n_end;
    int64_t m_beg;                                           // first row of the launch's tiles
};

struct TrailStage {
    uint16_t ehi[TB * TE_LD], elo[TB * TE_LD];
    uint16_t uhi[TK * TU_RS], ulo[TK * TU_RS];
};

// Per thread and chunk: E rows m = tid / 2, k = 16 (tid & 1) .. +15 and U rows
// k = tid / 8, n = 16 (tid & 7) .. +15, each as hi and lo: 8 x 16 bytes.
struct TrailRegs { u32x4_t e[2][2], u[2][2]; };   // [hi/lo][first/second 8 values]

GPTQ_DEV u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

GPTQ_DEV u32x4_t ld8_edge(const uint16_t* p, int valid) {   // 8 bf16, zero past `valid`
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < 8; ++e)
        if (e < valid) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
    return u32x4_t{w[0], w[1], w[2], w[3]};
}

GPTQ_DEV void trail_load(const TrailArgs& a, int64_t m0, int64_t n0, int kc, int tid, TrailRegs& r, bool full) {
    const int me = tid >> 1, ke = (tid & 1) * 16;
    const int ku = tid >> 3, nu = (tid & 7) * 16;
    const int64_t gm = m0 + me;
    const int64_t eo = gm * a.lde + kc + ke;
    const int64_t uo = (a.k0 + kc + ku) * a.d_col + n0 + nu;
    if (full) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            r.e[0][h] = ld16(a.Ehi + eo + 8 * h);
            r.e[1][h] = ld16(a.Elo + eo + 8 * h);
            r.u[0][h] = ld16(a.Uhi + uo + 8 * h);
            r.u[1][h] = ld16(a.Ulo + uo + 8 * h);
        }
        return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ve = (gm < a.d_row) ? a.K - (kc + ke + 8 * h) : 0;
        const int vu = (kc + ku < a.K) ? (int)(a.n_end - (n0 + nu + 8 * h)) : 0;
        r.e[0][h] = ld8_edge(a.Ehi + eo + 8 * h, ve);
        r.e[1][h] = ld8_edge(a.Elo + eo + 8 * h, ve);
        r.u[0][h] = ld8_edge(a.Uhi + uo + 8 * h, vu);
        r.u[1][h] = ld8_edge(a.Ulo + uo + 8 * h, vu);
    }
}

GPTQ_DEV void trail_store(TrailStage& st, int tid, const TrailRegs& r) {
    const int me = tid >> 1, ke = (tid & 1) * 16;
    const int ku = tid >> 3, nu = (tid & 7) * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<u32x4_t*>(&st.ehi[me * TE_LD + ke + 8 * h]) = r.e[0][h];
        *reinterpret_cast<u32x4_t*>(&st.elo[me * TE_LD + ke + 8 * h]) = r.e[1][h];
        *reinterpret_cast<u32x4_t*>(&st.uhi[ku * TU_RS + nu + 8 * h]) = r.u[0][h];
        *reinterpret_cast<u32x4_t*>(&st.ulo[ku * TU_RS + nu + 8 * h]) = r.u[1][h];
    }
}

// B operand (32 columns n x 16 k) from the [k][n] tile with two transposed reads:
// in each 16-lane group lane j addresses k = k0 + (j >> 2), n = n0 + 4 (j & 3) and lane
// i receives column n0 + i at k0 .. k0 + 3.
GPTQ_DEV f16x8_t trail_bfrag(const uint16_t* tile, int nc0, int kk, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int n = nc0 + (g & 1) * 16 + 4 * (j & 3);
    const int k = kk + (g >> 1) * 8 + (j >> 2);
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + k * TU_RS + n));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + (k + 4) * TU_RS + n));
    return __builtin_bit_cast(f16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

GPTQ_DEV void trail_mfma(const TrailStage& st, int wr, int wc, int lane, f32x16_t (&acc)[2][2]) {
#pragma unroll
    for (int kk = 0; kk < TK; kk += 16) {
        f16x8_t ah[2], al[2], bh[2], bl[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int m = wr * 64 + i * 32 + (lane & 31), k = kk + (lane >> 5) * 8;
            ah[i] = *reinterpret_cast<const f16x8_t*>(&st.ehi[m * TE_LD + k]);
            al[i] = *reinterpret_cast<const f16x8_t*>(&st.elo[m * TE_LD + k]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bh[j] = trail_bfrag(st.uhi, wc * 64 + j * 32, kk, lane);
            bl[j] = trail_bfrag(st.ulo, wc * 64 + j * 32, kk, lane);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bh[j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bl[j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bh[j], acc[i][j], 0, 0, 0);
            }
    }
}

__global__ __launch_bounds__(256) void trail_kernel(TrailArgs a) {
    __shared__ __attribute__((aligned(16))) TrailStage stg[2];
    const int64_t m0 = a.m_beg + (int64_t)blockIdx.y * TB;
    const int64_t n0 = a.n_beg + (int64_t)blockIdx.x * TB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
    const int nch = (a.K + TK - 1) / TK;
    // fast loads: the tile inside W, whole chunks of k, 16-byte aligned rows
    const bool fl = (m0 + TB <= a.d_row) && (n0 + TB <= a.n_end) && (a.K % TK == 0) && ((a.lde & 7) == 0) &&
                    ((a.d_col & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.Ehi) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(a.Elo) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(a.Uhi + a.k0 * a.d_col + n0) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(a.Ulo + a.k0 * a.d_col + n0) & 15) == 0);
    TrailRegs rg;
    trail_load(a, m0, n0, 0, tid, rg, fl);
    trail_store(stg[0], tid, rg);
    if (nch > 1) trail_load(a, m0, n0, TK, tid, rg, fl);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        trail_mfma(stg[c & 1], wr, wc, lane, acc);
        if (c + 1 < nch) trail_store(stg[(c + 1) & 1], tid, rg);
        if (c + 2 < nch) trail_load(a, m0, n0, (c + 2) * TK, tid, rg, fl);
        __syncthreads();
    }
    // W -= acc / es_row: all loads first, then all stores (a load after a store to the
    // same array would otherwise wait for that store's round trip)
    const bool full = (m0 + TB <= a.d_row) && (n0 + TB <= a.n_end);
    float* wbase = a.Wws + (m0 + wr * 64 + 4 * (lane >> 5)) * a.d_col + n0 + wc * 64 + (lane & 31);
    auto off = [&](int i, int j, int e) { return (int64_t)(i * 32 + 8 * (e >> 2) + (e & 3)) * a.d_col + j * 32; };
    auto rowm = [&](int i, int e) { return m0 + wr * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); };
    if (full) {
        // one accumulator tile (16 values per lane) at a time keeps the register count low
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float inv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) inv[e] = 1.0f / a.erow[rowm(i, e)];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float old[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) old[e] = wbase[off(i, j, e)];
#pragma unroll
                for (int e = 0; e < 16; ++e) wbase[off(i, j, e)] = fmaf(-acc[i][j][e], inv[e], old[e]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t gm = rowm(i, e);
                    const int64_t gn = n0 + wc * 64 + j * 32 + (lane & 31);
                    if (gm < a.d_row && gn < a.n_end)
                        a.Wws[gm * a.d_col + gn] = fmaf(-acc[i][j][e], 1.0f / a.erow[gm], a.Wws[gm * a.d_col + gn]);
                }
    }
}

// --------------------------------------------------------------------------
// Whole 128 x 128 tiles: the same product with the operands copied to LDS by direct
// global -> LDS loads (global_load_lds_dwordx4) into a ring of four 32-deep stages,
// issued three stages ahead, and the fragment reads of the next 16-deep slice
// overlapped with the MFMAs of the current one.  A stage holds E hi, E lo, U hi, U lo
// (8 KB each); wave w copies operand w.  E rows (64 bytes, four 16-byte chunks) are
// stored with chunk q at q ^ eswz(row) and read with 16-byte reads; U rows (256 bytes)
// with chunk c at tswz(row, c) and read with ds_read_b64_tr_b16; both are free of bank
// conflicts for 8- and 16-lane groups.
constexpr int TD_NSTG = 4;
constexpr int TD_OPE = TK * TB;                  // bf16 elements of one operand tile
constexpr int TD_STE = 4 * TD_OPE;               // one stage
constexpr int TD_DMA = TD_OPE * 2 / 1024;        // 1 KB loads per wave and stage
constexpr int TD_VM = (TD_NSTG - 2) * TD_DMA;    // loads left in flight at a stage wait
static_assert(TD_NSTG * TD_STE * 2 <= 160 * 1024, "LDS ring exceeds the workgroup's LDS");

GPTQ_DEV int eswz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
GPTQ_DEV int tswz(int k, int c) {
    const int r = k & 3;
    const int f = 2 * r + ((r ^ (r >> 1)) & 1);
    return c ^ (f << 1);
}

struct TrailCopy {
    uint32_t voff[TD_DMA];   // per-lane byte offsets of the wave's loads (row and chunk)
    const uint16_t* base;    // the wave's operand at stage 0 (wave-uniform)
    int64_t sstride;         // elements between stages
    uint32_t m0base;         // LDS byte address of the wave's operand tile in slot 0
};

GPTQ_DEV TrailCopy trail_copy_setup(const TrailArgs& a, const uint16_t* ring0, int64_t m0, int64_t n0, int wave,
                                    int lane) {
    TrailCopy tc;
    const int w = __builtin_amdgcn_readfirstlane(wave);
    tc.m0base = lds_addr(ring0) + (uint32_t)(w * TD_OPE * 2);
    if (w < 2) {   // E hi / lo: load i covers rows 16 i .. 16 i + 15, lane l row 16 i + l / 4
        tc.base = (w ? a.Elo : a.Ehi) + m0 * a.lde;
        tc.sstride = TK;
#pragma unroll
        for (int i = 0; i < TD_DMA; ++i) {
            const int r = 16 * i + (lane >> 2), q = (lane & 3) ^ eswz(r);
            tc.voff[i] = (uint32_t)(((int64_t)r * a.lde + 8 * q) * 2);
        }
    } else {       // U hi / lo: load i covers rows 4 i .. 4 i + 3, lane l row 4 i + l / 16
        tc.base = (w == 2 ? a.Uhi : a.Ulo) + a.k0 * a.d_col + n0;
        tc.sstride = (int64_t)TK * a.d_col;
#pragma unroll
        for (int i = 0; i < TD_DMA; ++i) {
            const int r = 4 * i + (lane >> 4), c = tswz(r, lane & 15);
            tc.voff[i] = (uint32_t)(((int64_t)r * a.d_col + 8 * c) * 2);
        }
    }
    return tc;
}

template <int SLOT>
GPTQ_DEV void trail_issue(const TrailCopy& tc, int st) {
    const uint16_t* sbase = tc.base + st * tc.sstride;
    static_for<0, TD_DMA>([&](auto I) {
        constexpr int i = decltype(I)::value;
        dma16<(uint32_t)(SLOT * TD_STE * 2 + i * 1024)>(tc.voff[i], sbase, tc.m0base);
    });
}

struct TdFrags { f16x8_t ah[2], al[2], bh[2], bl[2]; };

// B operand from a swizzled U tile (as trail_bfrag, with the chunk swizzle)
GPTQ_DEV f16x8_t td_bfrag(const uint16_t* tile, int nc0, int kk, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int n = nc0 + (g & 1) * 16 + 4 * (j & 3);
    const int k = kk + (g >> 1) * 8 + (j >> 2);
    const int c = n >> 3, half = (n >> 2) & 1;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(tile + k * TB + 8 * tswz(k, c) + 4 * half));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(tile + (k + 4) * TB + 8 * tswz(k + 4, c) + 4 * half));
    return __builtin_bit_cast(f16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// one wave's fragments for the 16-deep slice kk of a stage: A (rows wr * 64 + 32 i +
// lane % 32, k = kk + 8 (lane / 32) .. + 7) with 16-byte reads, B transposed
GPTQ_DEV void td_read(const uint16_t* stg, int kk, int wr, int wc, int lane, TdFrags& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = wr * 64 + i * 32 + (lane & 31), q = (kk >> 3) + (lane >> 5);
        const int o = m * TK + 8 * (q ^ eswz(m));
        f.ah[i] = *reinterpret_cast<const f16x8_t*>(stg + o);
        f.al[i] = *reinterpret_cast<const f16x8_t*>(stg + TD_OPE + o);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        f.bh[j] = td_bfrag(stg + 2 * TD_OPE, wc * 64 + j * 32, kk, lane);
        f.bl[j] = td_bfrag(stg + 3 * TD_OPE, wc * 64 + j * 32, kk, lane);
    }
}

// the three products, product-major (the four accumulators take turns)
GPTQ_DEV void td_mfma(const TdFrags& f, f32x16_t (&acc)[2][2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[i], f.bh[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[i], f.bl[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.al[i], f.bh[j], acc[i][j], 0, 0, 0);
    // 12 fragment reads of the next slice against 12 MFMAs: one each, in turn
    static_for<0, 12>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    });
}

__global__ __launch_bounds__(256, 1) void trail_dma_kernel(TrailArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_ring[TD_NSTG * TD_STE];
    const uint16_t* ring[TD_NSTG];
    static_for<0, TD_NSTG>([&](auto I) { ring[decltype(I)::value] = lds_ring + decltype(I)::value * TD_STE; });
    const int64_t m0 = a.m_beg + (int64_t)blockIdx.y * TB;
    const int64_t n0 = a.n_beg + (int64_t)blockIdx.x * TB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
    const int nst = a.K / TK;
    // loads of stages past the last re-load the last one (addresses stay inside the
    // operands), so that every step leaves the same number of loads in flight
    auto t0 = [&](int st) { return st < nst ? st : nst - 1; };
    const TrailCopy tc = trail_copy_setup(a, lds_ring, m0, n0, wave, lane);
    static_for<0, TD_NSTG - 1>([&](auto I) { trail_issue<decltype(I)::value>(tc, t0(decltype(I)::value)); });
    wait_vm_lgkm0<TD_VM>();
    __syncthreads();
    trail_issue<TD_NSTG - 1>(tc, t0(TD_NSTG - 1));
    TdFrags f0, f1;
    td_read(ring[0], 0, wr, wc, lane, f0);
    for (int st = 0; st < nst; st += TD_NSTG) {
        static_for<0, TD_NSTG>([&](auto U) {
            constexpr int u = decltype(U)::value;
            if (st + u < nst) {
                td_read(ring[u], 16, wr, wc, lane, f1);
                td_mfma(f0, acc);
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_lgkm0<TD_VM>();
                __syncthreads();
                trail_issue<u>(tc, t0(st + u + TD_NSTG));
                td_read(ring[(u + 1) % TD_NSTG], 0, wr, wc, lane, f0);
                td_mfma(f1, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    }
    __builtin_amdgcn_s_waitcnt(0);   // the trailing re-loads land before the workgroup ends
    // W -= acc / es_row (whole tile): all loads first, then all stores
    float* wbase = a.Wws + (m0 + wr * 64 + 4 * (lane >> 5)) * a.d_col + n0 + wc * 64 + (lane & 31);
    const float* ebase = a.erow + m0 + wr * 64 + 4 * (lane >> 5);
    auto off = [&](int i, int j, int e) { return (int64_t)(i * 32 + 8 * (e >> 2) + (e & 3)) * a.d_col + j * 32; };
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float inv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) inv[e] = 1.0f / ebase[i * 32 + 8 * (e >> 2) + (e & 3)];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float old[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) old[e] = wbase[off(i, j, e)];
#pragma unroll
            for (int e = 0; e < 16; ++e) wbase[off(i, j, e)] = fmaf(-acc[i][j][e], inv[e], old[e]);
        }
    }
}

// --------------------------------------------------------------------------
// Large products (whole 256 x 256 tiles): the same update on the Hessian kernel's load
// path.  Eight waves (two per SIMD), each accumulating a 64 x 128 sub-tile (2 x 4 MFMA
// 32 x 32 tiles, fp16, three products per k step); a ring of four 16-deep stages
// (E hi, E lo: 256 rows x 16 k; U hi, U lo: 16 k x 256 columns; 8 KB each) filled by
// direct global -> LDS loads issued three stages ahead; the fragments of the next stage
// are read while the MFMAs of the current one run.  Per MFMA a wave reads 512 bytes of
// LDS (the 128 x 128 kernel: 683) and the copy writes 171 (341).  E rows are stored as
// they lie (32 bytes, read with 16-byte reads); U rows (512 bytes) with their 16-byte
// chunks XOR-swizzled as in the Hessian kernel and read with ds_read_b64_tr_b16.
// Work mapping: the tiles in row-major order are cut into eight runs, one per XCD
// (workgroup L runs on XCD L % 8), so each XCD's L2 serves few rows of E.
constexpr int TG_BM = 256, TG_BK = 16, TG_NSTG = 4, TG_WAVES = 8;
constexpr int TG_WM = 64, TG_WN = 128;             // wave sub-tile: waves 4 (rows) x 2 (columns)
constexpr int TG_OPE = TG_BM * TG_BK;              // 16-bit elements of one operand of a stage
constexpr int TG_STE = 4 * TG_OPE;                 // a stage: E hi, E lo, U hi, U lo (32 KB)
constexpr int TG_DMA = 4;                          // 1 KB loads per wave and stage
constexpr int TG_VM = (TG_NSTG - 2) * TG_DMA;      // loads left in flight at a stage wait
static_assert(TG_NSTG * TG_STE * 2 <= 160 * 1024, "LDS ring exceeds the workgroup's LDS");

GPTQ_DEV int tg_swz(int k, int c) {       // the Hessian kernel's chunk swizzle of 512-byte rows
    const int r = k & 3;
    const int f = 2 * r + ((r ^ (r >> 1)) & 1);
    return c ^ (f << 1);
}

struct TgCopy {
    uint32_t voff[TG_DMA];   // per-lane byte offsets of the wave's loads
    const uint16_t* base;    // the wave's operand at stage 0 (wave-uniform)
    int64_t sstride;         // elements between stages
    uint32_t m0base;         // LDS byte address of the wave's share of the operand in slot 0
};

// Wave w copies 4 KB (half h = w & 1) of operand w / 2 (E hi, E lo, U hi, U lo).  E: load
// i covers rows 32 (4 h + i) .. + 31, lane l row + l / 2, chunk l & 1 (linear in LDS).
// U: load i covers k rows 2 (4 h + i), + 1, lane l row + l / 32, LDS chunk position l % 32
// holding chunk tg_swz(row, l % 32).
GPTQ_DEV TgCopy tg_copy_setup(const TrailArgs& a, const uint16_t* ring0, int64_t m0, int64_t n0, int wave, int lane) {
    TgCopy tc;
    const int w = __builtin_amdgcn_readfirstlane(wave);
    const int op = w >> 1, h = w & 1;
    tc.m0base = lds_addr(ring0) + (uint32_t)(op * TG_OPE * 2 + h * TG_DMA * 1024);
    if (op < 2) {
        tc.base = (op ? a.Elo : a.Ehi) + m0 * a.lde;
        tc.sstride = TG_BK;
#pragma unroll
        for (int i = 0; i < TG_DMA; ++i) {
            const int r = 32 * (TG_DMA * h + i) + (lane >> 1), q = lane & 1;
            tc.voff[i] = (uint32_t)(((int64_t)r * a.lde + 8 * q) * 2);
        }
    } else {
        tc.base = (op == 2 ? a.Uhi : a.Ulo) + a.k0 * a.d_col + n0;
        tc.sstride = (int64_t)TG_BK * a.d_col;
#pragma unroll
        for (int i = 0; i < TG_DMA; ++i) {
            const int r = 2 * (TG_DMA * h + i) + (lane >> 5), c = tg_swz(r, lane & 31);
            tc.voff[i] = (uint32_t)(((int64_t)r * a.d_col + 8 * c) * 2);
        }
    }
    return tc;
}

template <int SLOT>
GPTQ_DEV void tg_issue(const TgCopy& tc, int st) {
    const uint16_t* sbase = tc.base + st * tc.sstride;
    static_for<0, TG_DMA>([&](auto I) {
        constexpr int i = decltype(I)::value;
        dma16<(uint32_t)(SLOT * TG_STE * 2 + i * 1024)>(tc.voff[i], sbase, tc.m0base);
    });
}

struct TgFrags { f16x8_t ah[2], al[2], bh[4], bl[4]; };

// B operand (32 columns n x 16 k) from a swizzled [k][256] U tile (two transposed reads)
GPTQ_DEV f16x8_t tg_bfrag(const uint16_t* tile, int nc0, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int n = nc0 + (g & 1) * 16 + 4 * (j & 3);
    const int k = (g >> 1) * 8 + (j >> 2);
    const int c = n >> 3, half = (n >> 2) & 1;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(tile + k * TG_BM + 8 * tg_swz(k, c) + 4 * half));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(tile + (k + 4) * TG_BM + 8 * tg_swz(k + 4, c) + 4 * half));
    return __builtin_bit_cast(f16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

GPTQ_DEV void tg_read(const uint16_t* stg, int wr, int wc, int lane, TgFrags& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = wr * TG_WM + i * 32 + (lane & 31);
        const int o = m * TG_BK + 8 * (lane >> 5);
        f.ah[i] = *reinterpret_cast<const f16x8_t*>(stg + o);
        f.al[i] = *reinterpret_cast<const f16x8_t*>(stg + TG_OPE + o);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f.bh[j] = tg_bfrag(stg + 2 * TG_OPE, wc * TG_WN + j * 32, lane);
        f.bl[j] = tg_bfrag(stg + 3 * TG_OPE, wc * TG_WN + j * 32, lane);
    }
}

// the three products, product-major; the 20 fragment reads of the next stage are
// interleaved with these 24 MFMAs
GPTQ_DEV void tg_mfma(const TgFrags& f, f32x16_t (&acc)[2][4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[i], f.bh[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[i], f.bl[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.al[i], f.bh[j], acc[i][j], 0, 0, 0);
    static_for<0, 4>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    });
    static_for<0, 16>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    });
    static_for<0, 4>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); });
}

// a.n_beg: first column of the region; the grid enumerates nm x nn whole tiles
__global__ __launch_bounds__(64 * TG_WAVES, 1) void trail_big_kernel(TrailArgs a, int nm, int nn) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_ring[TG_NSTG * TG_STE];
    const uint16_t* ring[TG_NSTG];
    static_for<0, TG_NSTG>([&](auto I) { ring[decltype(I)::value] = lds_ring + decltype(I)::value * TG_STE; });
    const int T = nm * nn, L = blockIdx.x;
    const int tpx = (T + 7) / 8;
    const int tile = (L & 7) * tpx + (L >> 3);
    if (tile >= T) return;
    const int64_t m0 = a.m_beg + (int64_t)(tile / nn) * TG_BM;
    const int64_t n0 = a.n_beg + (int64_t)(tile % nn) * TG_BM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};
    const int nst = a.K / TG_BK;
    // loads of stages past the last re-load the last one (addresses stay inside the
    // operands), so that every step leaves the same number of loads in flight
    auto t0 = [&](int st) { return st < nst ? st : nst - 1; };
    const TgCopy tc = tg_copy_setup(a, lds_ring, m0, n0, wave, lane);
    static_for<0, TG_NSTG - 1>([&](auto I) { tg_issue<decltype(I)::value>(tc, t0(decltype(I)::value)); });
    wait_vm_lgkm0<TG_VM>();
    __syncthreads();
    tg_issue<TG_NSTG - 1>(tc, t0(TG_NSTG - 1));
    TgFrags f0, f1;
    tg_read(ring[0], wr, wc, lane, f0);
    for (int st = 0; st < nst; st += TG_NSTG) {
        static_for<0, TG_NSTG>([&](auto U) {
            constexpr int u = decltype(U)::value;
            if (st + u < nst) {
                // stage st + u + 1 has landed and every wave is done with slot u
                wait_vm_lgkm0<TG_VM>();
                __syncthreads();
                tg_issue<u>(tc, t0(st + u + TG_NSTG));
                TgFrags& cur = (u & 1) ? f1 : f0;
                TgFrags& nxt = (u & 1) ? f0 : f1;
                tg_read(ring[(u + 1) % TG_NSTG], wr, wc, lane, nxt);
                tg_mfma(cur, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    }
    __builtin_amdgcn_s_waitcnt(0);   // the trailing re-loads land before the workgroup ends
    // W -= acc / es_row: all loads of a 32 x 128 strip first, then its stores
    float* wbase = a.Wws + (m0 + wr * TG_WM + 4 * (lane >> 5)) * a.d_col + n0 + wc * TG_WN + (lane & 31);
    const float* ebase = a.erow + m0 + wr * TG_WM + 4 * (lane >> 5);
    auto off = [&](int i, int j, int e) { return (int64_t)(i * 32 + 8 * (e >> 2) + (e & 3)) * a.d_col + j * 32; };
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float inv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) inv[e] = 1.0f / ebase[i * 32 + 8 * (e >> 2) + (e & 3)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float old[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) old[e] = wbase[off(i, j, e)];
#pragma unroll
            for (int e = 0; e < 16; ++e) wbase[off(i, j, e)] = fmaf(-acc[i][j][e], inv[e], old[e]);
        }
    }
}

// Rows [m_beg, m_end) of the product: whole 128 x 128 tiles on the direct-load kernel
// when the operands allow 16-byte loads at every row (K a multiple of 32, row pitches
// multiples of 8 elements, aligned arrays); the partial last row and column of tiles (and
// everything otherwise) on trail_kernel.
static gptq_status trail_region(const TrailArgs& ta, int64_t m_beg, int64_t m_end, int64_t n_beg, int64_t n_end,
                                hipStream_t s) {
    if (n_end <= n_beg || m_end <= m_beg) return GPTQ_OK;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool dma = ta.K % TK == 0 && (ta.lde & 7) == 0 && (ta.d_col & 7) == 0 && (n_beg & 7) == 0 &&
                     ta.d_col < ((int64_t)1 << 25) && ta.lde < ((int64_t)1 << 20) && al16(ta.Ehi) && al16(ta.Elo) &&
                     al16(ta.Uhi) && al16(ta.Ulo);
    const int64_t mf = dma ? m_beg + ((m_end - m_beg) / TB) * TB : m_beg;        // rows of whole tiles
    const int64_t nf = dma ? n_beg + ((n_end - n_beg) / TB) * TB : n_beg;        // columns of whole tiles
    if (mf > m_beg && nf > n_beg) {
        TrailArgs t = ta;
        t.m_beg = m_beg; t.n_beg = n_beg;
        trail_dma_kernel<<<dim3((unsigned)((nf - n_beg) / TB), (unsigned)((mf - m_beg) / TB)), 256, 0, s>>>(t);
        GPTQ_LAUNCH_CHECK();
    }
    auto edge = [&](int64_t mb, int64_t me, int64_t nb, int64_t ne) -> gptq_status {
        if (me <= mb || ne <= nb) return GPTQ_OK;
        TrailArgs t = ta;
        t.m_beg = mb; t.d_row = me; t.n_beg = nb; t.n_end = ne;
        trail_kernel<<<dim3((unsigned)((ne - nb + TB - 1) / TB), (unsigned)((me - mb + TB - 1) / TB)), 256, 0, s>>>(t);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    };
    gptq_status st;
    if (mf > m_beg && nf > n_beg) {
        if ((st = edge(m_beg, mf, nf, n_end)) != GPTQ_OK) return st;     // last column of tiles
        return edge(mf, m_end, n_beg, n_end);                            // last row of tiles
    }
    return edge(m_beg, m_end, n_beg, n_end);
}

// W[:, n_beg:n_end] -= E U[k0:k0+K, n_beg:n_end]: whole 256 x 256 tiles on the large-tile
// kernel when the operands allow it (K a multiple of 16, 16-byte rows) and there are at
// least as many of them as compute units (fewer large tiles leave compute units idle that
// four times as many 128 x 128 tiles would fill: measured slower at 4096 x 4096), the
// rest by trail_region.
static gptq_status trail(const TrailArgs& ta, hipStream_t s) {
    if (ta.n_end <= ta.n_beg || ta.K <= 0 || ta.d_row <= 0) return GPTQ_OK;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool big = ta.K % TG_BK == 0 && (ta.lde & 7) == 0 && (ta.d_col & 7) == 0 && (ta.n_beg & 7) == 0 &&
                     ta.d_col < ((int64_t)1 << 25) && ta.lde < ((int64_t)1 << 20) && al16(ta.Ehi) && al16(ta.Elo) &&
                     al16(ta.Uhi) && al16(ta.Ulo);
    const int64_t mb = big ? (ta.d_row / TG_BM) * TG_BM : 0;
    const int64_t nb = big ? ta.n_beg + ((ta.n_end - ta.n_beg) / TG_BM) * TG_BM : ta.n_beg;
    if (mb > 0 && nb > ta.n_beg && (mb / TG_BM) * ((nb - ta.n_beg) / TG_BM) >= 256) {
        TrailArgs t = ta;
        t.m_beg = 0;
        const int nm = (int)(mb / TG_BM), nn = (int)((nb - ta.n_beg) / TG_BM);
        trail_big_kernel<<<(unsigned)(8 * ((nm * nn + 7) / 8)), 64 * TG_WAVES, 0, s>>>(t, nm, nn);
        GPTQ_LAUNCH_CHECK();
        gptq_status st;
        if ((st = trail_region(ta, 0, mb, nb, ta.n_end, s)) != GPTQ_OK) return st;     // last column of tiles
        return trail_region(ta, mb, ta.d_row, ta.n_beg, ta.n_end, s);                 // last row of tiles
    }
    return trail_region(ta, 0, ta.d_row, ta.n_beg, ta.n_end, s);
}

// --------------------------------------------------------------------------
// Host side
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Two levels of deferral of the trailing update.  Inside a super-block (QSB columns)
// every 128-column block updates only the rest of the super-block (in the sweep
// kernel).  Inside a macro-block (QMB columns, QMB / QSB super-blocks) every
// super-block then updates only the rest of the macro-block (K = QSB); the columns after
// the macro-block get one product with K = QMB, with the errors of all its super-blocks.
// The fp32 working copy of the later columns is therefore read and written once per
// macro-block instead of once per super-block.  The regrouping of the rank-1 updates is
// exact in exact arithmetic, as for the 128-column lazy blocks.
constexpr int QMB = 2048;
static_assert(QMB % QSB == 0, "a macro-block holds whole super-blocks");

// Workspace: fp32 working copy of W | E hi | E lo (scaled fp16, d_row x QMB) | U hi |
// U lo (scaled fp16, d_col x d_col) | Ut hi | Ut lo (scaled fp16, one transposed QSB x QSB
// diagonal block of U per super-block) | es (fp32, d_row) | us (fp32, d_col).
static size_t ut_bytes(int64_t d_col) { return (size_t)((d_col + QSB - 1) / QSB) * QSB * QSB * 2; }

size_t quant_ws_bytes(int64_t d_row, int64_t d_col) {
    if (d_row <= 0 || d_col <= 0) return 0;
    return align256((size_t)d_row * d_col * sizeof(float)) + 2 * align256((size_t)d_row * QMB * 2) +
           2 * align256((size_t)d_col * d_col * 2) + 2 * align256(ut_bytes(d_col)) +
           align256((size_t)d_row * sizeof(float)) + align256((size_t)d_col * sizeof(float));
}

// The split of a scaled value into fp16 hi + lo (hi = fp16(x), lo = fp16(x - hi); x - hi
// is exact in fp32).
GPTQ_DEV void split_f16(float x, uint16_t& h, uint16_t& l) {
    h = f32_to_f16_bits(x);
    l = f32_to_f16_bits(x - f16_bits_to_f32(h));
}

// The diagonal QSB x QSB blocks of U, split into bf16 hi + lo, zero past d, in the
// order in which the updates inside a super-block read them as MFMA B operands: for
// column group g = n / 16 and k step s = k / 32, a 1 KB piece holds, for lane l =
// n % 16 + 16 ((k % 32) / 8), the eight values k = 32 s + 8 (l / 16) .. + 7 of column
// n, so that a wave reads each operand with one contiguous 16-byte-per-lane load.
// One workgroup per 64 x 64 tile, transposed through LDS.
__global__ __launch_bounds__(256) void udt_kernel(const float* U, int64_t d, const float* us, uint16_t* th,
                                                  uint16_t* tl) {
    __shared__ float t[64][65];
    const int b = blockIdx.y, tk = blockIdx.x / (QSB / 64), tn = blockIdx.x % (QSB / 64);
    const int64_t k0 = (int64_t)b * QSB + tk * 64, n0 = (int64_t)b * QSB + tn * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 4 * (tid & 15) + e;
            t[r][c] = (k0 + r < d && n0 + c < d) ? U[(k0 + r) * d + n0 + c] * us[k0 + r] : 0.f;
        }
    }
    __syncthreads();
    const int n = tid >> 2, kb = 16 * (tid & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int nb = tn * 64 + n, k = tk * 64 + kb + 8 * h;   // within the block
        const int64_t o = (int64_t)b * QSB * QSB +
                          ((int64_t)((nb >> 4) * (QSB / 32) + (k >> 5)) * 64 + (nb & 15) + 16 * ((k & 31) >> 3)) * 8;
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float u0 = t[kb + 8 * h + 2 * e][n], u1 = t[kb + 8 * h + 2 * e + 1][n];
            uint16_t h0, h1, l0, l1;
            split_f16(u0, h0, l0);
            split_f16(u1, h1, l1);
            ph[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            pl[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        *reinterpret_cast<u32x4_t*>(th + o) = u32x4_t{ph[0], ph[1], ph[2], ph[3]};
        *reinterpret_cast<u32x4_t*>(tl + o) = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
    }
}

// U -> scaled fp16 hi + lo, once per call: every workgroup of the trailing products reads
// the split instead of forming it again.  One workgroup per row k: the row's largest
// magnitude m < 2^e (frexp) gives us_k = 2^(14 - e), so the scaled row lies in
// (-2^14, 2^14) with its largest value at least 2^13 (U is upper triangular with a
// positive diagonal, so m > 0; only the columns from k's 8-column piece on are read for
// it, which also cover the zeros left of k).  Eight values per thread and step with
// 16-byte accesses when the arrays are aligned.
__global__ __launch_bounds__(256) void split_u_kernel(const float* U, int64_t d, uint16_t* hi, uint16_t* lo,
                                                      float* us) {
    __shared__ float red[4];
    const int64_t k = blockIdx.x;
    const int tid = threadIdx.x;
    const float* row = U + k * d;
    uint16_t* hrow = hi + k * d;
    uint16_t* lrow = lo + k * d;
    const bool vec = (d & 7) == 0 && ((reinterpret_cast<uintptr_t>(U) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(hi) & 15) == 0) && ((reinterpret_cast<uintptr_t>(lo) & 15) == 0);
    const int64_t n8 = vec ? d / 8 : 0;
    float m = 0.f;
    for (int64_t i = (k >> 3) + tid; i < n8; i += 256) {     // from the 8-column piece holding k
        const f32x4_t a = reinterpret_cast<const f32x4_t*>(row)[2 * i], b = reinterpret_cast<const f32x4_t*>(row)[2 * i + 1];
        m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3]))),
                           fmaxf(fmaxf(fabsf(b[0]), fabsf(b[1])), fmaxf(fabsf(b[2]), fabsf(b[3])))));
    }
    for (int64_t c = (n8 > 0 ? 8 * n8 : k) + tid; c < d; c += 256) m = fmaxf(m, fabsf(row[c]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    (void)frexpf(m, &e);
    const float sc = (m > 0.f && m <= 3.0e38f) ? ldexpf(1.f, 14 - e) : 1.f;
    if (tid == 0) us[k] = sc;
    for (int64_t i = tid; i < n8; i += 256) {
        const f32x4_t a = reinterpret_cast<const f32x4_t*>(row)[2 * i], b = reinterpret_cast<const f32x4_t*>(row)[2 * i + 1];
        const float u[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint16_t h0, h1, l0, l1;
            split_f16(u[2 * q] * sc, h0, l0);
            split_f16(u[2 * q + 1] * sc, h1, l1);
            ph[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            pl[q] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        reinterpret_cast<u32x4_t*>(hrow)[i] = u32x4_t{ph[0], ph[1], ph[2], ph[3]};
        reinterpret_cast<u32x4_t*>(lrow)[i] = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
    }
    for (int64_t c = 8 * n8 + tid; c < d; c += 256) split_f16(row[c] * sc, hrow[c], lrow[c]);
}

static gptq_status launch_row_params(int bits, bool sym, bool fp4, bool mx, const float* Wws, int64_t d_row, int64_t d_col,
                                     uint16_t* scales, uint16_t* zeros, int32_t* info, hipStream_t s) {
    dim3 grid((unsigned)d_row);
#define RP(B, S) row_params_kernel<B, S, false><<<grid, 256, 0, s>>>(Wws, d_col, scales, zeros, info)
    if (fp4) row_params_kernel<4, true, true><<<grid, 256, 0, s>>>(Wws, d_col, scales, zeros, info, mx ? 1 : 0);
    else if (bits == 4) { if (sym) RP(4, true); else RP(4, false); }
    else if (bits == 3) { if (sym) RP(3, true); else RP(3, false); }
    else if (bits == 8) { if (sym) RP(8, true); else RP(8, false); }
    else return GPTQ_ERR_UNSUPPORTED;
#undef RP
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

// Per-tensor: partial ranges of up to 1024 blocks (in the E area of the workspace, which
// the sweep only uses later on the same stream), then one block for S16 and the zero.
static gptq_status launch_tensor_params(int bits, bool sym, bool fp4, bool mx, const float* Wws, int64_t d_row, int64_t d_col,
                                        float* part, int nb, uint16_t* scales, uint16_t* zeros, int32_t* info,
                                        hipStream_t s) {
    tensor_minmax_kernel<<<nb, 256, 0, s>>>(Wws, d_row * d_col, part);
    GPTQ_LAUNCH_CHECK();
#define TP(B, S) tensor_params_kernel<B, S, false><<<1, 256, 0, s>>>(part, nb, d_row, scales, zeros, info)
    if (fp4) tensor_params_kernel<4, true, true><<<1, 256, 0, s>>>(part, nb, d_row, scales, zeros, info, mx ? 1 : 0);
    else if (bits == 4) { if (sym) TP(4, true); else TP(4, false); }
    else if (bits == 3) { if (sym) TP(3, true); else TP(3, false); }
    else if (bits == 8) { if (sym) TP(8, true); else TP(8, false); }
    else return GPTQ_ERR_UNSUPPORTED;
#undef TP
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

gptq_status quant_launch(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                         const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                         void* ws, size_t ws_bytes, int32_t* info, hipStream_t s) {
    if (ws == nullptr || ws_bytes < quant_ws_bytes(d_row, d_col)) return GPTQ_ERR_WORKSPACE;
    float* Wws = reinterpret_cast<float*>(ws);
    char* wp = reinterpret_cast<char*>(ws) + align256((size_t)d_row * d_col * sizeof(float));
    uint16_t* Ehi = reinterpret_cast<uint16_t*>(wp);
    wp += align256((size_t)d_row * QMB * 2);
    uint16_t* Elo = reinterpret_cast<uint16_t*>(wp);
    wp += align256((size_t)d_row * QMB * 2);
    uint16_t* Uhi = reinterpret_cast<uint16_t*>(wp);
    wp += align256((size_t)d_col * d_col * 2);
    uint16_t* Ulo = reinterpret_cast<uint16_t*>(wp);
    wp += align256((size_t)d_col * d_col * 2);
    uint16_t* Uthi = reinterpret_cast<uint16_t*>(wp);
    wp += align256(ut_bytes(d_col));
    uint16_t* Utlo = reinterpret_cast<uint16_t*>(wp);
    wp += align256(ut_bytes(d_col));
    float* es = reinterpret_cast<float*>(wp);
    wp += align256((size_t)d_row * sizeof(float));
    float* us = reinterpret_cast<float*>(wp);
    const int G = p.group_size;                 // -1: per tensor, 0: per row
    const int n_groups = (G <= 0) ? 1 : (int)(d_col / G);

    fill_i32(info, 1, 0, s);
    GPTQ_LAUNCH_CHECK();
    const unsigned cgrid = (unsigned)d_row;
    switch (w_dtype) {
        case GPTQ_F32: convert_kernel<GPTQ_F32><<<cgrid, 256, 0, s>>>(W, d_col, Wws, es, info); break;
        case GPTQ_BF16: convert_kernel<GPTQ_BF16><<<cgrid, 256, 0, s>>>(W, d_col, Wws, es, info); break;
        case GPTQ_F16: convert_kernel<GPTQ_F16><<<cgrid, 256, 0, s>>>(W, d_col, Wws, es, info); break;
        default: return GPTQ_ERR_UNSUPPORTED;
    }
    GPTQ_LAUNCH_CHECK();
    gptq_status st;
    if (G == 0) {
        st = launch_row_params(p.bits, p.sym != 0, p.sym >= 2, p.sym == 3, Wws, d_row, d_col, scales, zeros, info, s);
        if (st != GPTQ_OK) return st;
    } else if (G < 0) {
        // E holds d_row x QMB 16-bit values: room for 64 d_row partial ranges
        const int nb = (int)std::min<int64_t>(1024, 64 * d_row);
        st = launch_tensor_params(p.bits, p.sym != 0, p.sym >= 2, p.sym == 3, Wws, d_row, d_col, reinterpret_cast<float*>(Ehi), nb, scales,
                                  zeros, info, s);
        if (st != GPTQ_OK) return st;
    }
    SweepArgs sa;
    {
        split_u_kernel<<<(unsigned)d_col, 256, 0, s>>>(U, d_col, Uhi, Ulo, us);
        GPTQ_LAUNCH_CHECK();
        udt_kernel<<<dim3((QSB / 64) * (QSB / 64), (unsigned)((d_col + QSB - 1) / QSB)), 256, 0, s>>>(U, d_col, us,
                                                                                                    Uthi, Utlo);
        GPTQ_LAUNCH_CHECK();
    }
    sa.es = es; sa.us = us;
    sa.Wws = Wws; sa.d_row = d_row; sa.d_col = d_col; sa.U = U;
    sa.codes = codes; sa.code_ld = p.bits == 3 ? d_col / 8 * 3 : (p.bits <= 4) ? d_col / 2 : d_col;
    sa.bits3 = p.bits == 3;
    sa.scales = scales; sa.zeros = zeros; sa.n_groups = n_groups; sa.info = info;
    sa.group = G < 0 ? 0 : G;   // per tensor: every row's parameters are set, as per row
    sa.sym = p.sym != 0; sa.packed = p.bits <= 4;
    sa.fp4 = p.sym >= 2;
    sa.mx = p.sym == 3;
    sa.qmin = sa.sym ? -((1 << (p.bits - 1)) - 1) : 0;
    sa.qmax = sa.fp4 ? 6 : sa.sym ? ((1 << (p.bits - 1)) - 1) : (1 << p.bits) - 1;
    sa.zoff = (sa.sym && !sa.fp4) ? (1 << (p.bits - 1)) : 0;
    for (int64_t m0 = 0; m0 < d_col; m0 += QMB) {
        const int64_t m1 = std::min<int64_t>(m0 + QMB, d_col);
        for (int64_t s0 = m0; s0 < m1; s0 += QSB) {
            const int64_t s1 = std::min<int64_t>(s0 + QSB, m1);
            // the super-block's blocks, each followed by the update of the rest of the
            // super-block, in one launch; its errors go to columns s0 - m0 .. of E
            sa.s0 = s0; sa.s1 = s1; sa.Ehi = Ehi + (s0 - m0); sa.Elo = Elo + (s0 - m0); sa.lde = QMB;
            sa.Uthi = Uthi + (s0 / QSB) * QSB * QSB;
            sa.Utlo = Utlo + (s0 / QSB) * QSB * QSB;
            st = sweep_launch(sa, s);
            if (st != GPTQ_OK) return st;
            // the rest of the macro-block, K = s1 - s0
            TrailArgs tn{Wws, d_row, d_col, Ehi + (s0 - m0), Elo + (s0 - m0), QMB, Uhi, Ulo, es, s0, (int)(s1 - s0),
                         s1, m1, 0};
            if ((st = trail(tn, s)) != GPTQ_OK) return st;
        }
        // everything after the macro-block, K = m1 - m0
        TrailArgs tf{Wws, d_row, d_col, Ehi, Elo, QMB, Uhi, Ulo, es, m0, (int)(m1 - m0), m1, d_col, 0};
        if ((st = trail(tf, s)) != GPTQ_OK) return st;
    }
    return GPTQ_OK;
}

// --------------------------------------------------------------------------
// Dequantization: W_out = S16 (u - z).
// Fast path (8 consecutive columns per thread, one group): one 4-byte (two codes per
// byte) or 8-byte load of codes, one scale / zero pair, 16-byte stores; it needs d_col
// and the group size to be multiples of 8 and aligned rows.  Otherwise element by element.
// E2M1 magnitude of a code's low 3 bits, negated when bit 3 is set.
GPTQ_DEV float e2m1_value(uint32_t u) {
    const uint32_t m = u & 7u;
    const float v = m < 4u ? 0.5f * (float)m : (m < 6u ? (float)(m - 2u) : 2.f * (float)(m - 4u));
    return (u & 8u) ? -v : v;
}

template <int BITS, gptq_dtype OT, bool FP4 = false>
__global__ void dequant_kernel(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t d_row,
                               int64_t d_col, int G, void* out) {
    const int64_t chunks = (d_col + 7) / 8;
    const int64_t code_ld = (BITS == 3) ? d_col / 8 * 3 : (BITS <= 4) ? d_col / 2 : d_col;
    const int n_groups = (G == 0) ? 1 : (int)(d_col / G);
    constexpr int OB = (OT == GPTQ_F32) ? 4 : 2;     // output bytes per value
    // rows beyond the grid's y extent (at most 65535) are taken in strides of it
    for (int64_t row = blockIdx.y; row < d_row; row += gridDim.y) {
        const bool fast = (d_col % 8 == 0) && (G % 8 == 0) &&
                          (BITS == 3 || ((reinterpret_cast<uintptr_t>(codes) & 7) == 0)) &&
                          ((reinterpret_cast<uintptr_t>(out) & 15) == 0) &&
                          (BITS == 3 || (code_ld * row) % ((BITS <= 4) ? 4 : 8) == 0) && ((d_col * OB) % 16 == 0);
        for (int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ch < chunks; ch += (int64_t)gridDim.x * blockDim.x) {
            const int64_t c0 = ch * 8;
            float v[8];
            if (fast) {
                uint32_t u[8];
                if constexpr (BITS == 3) {
                    const uint32_t g24 = load_u24(codes + row * code_ld + c0 / 8 * 3);
#pragma unroll
                    for (int e = 0; e < 8; ++e) u[e] = code3(g24, e);
                } else if constexpr (BITS <= 4) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + row * code_ld + c0 / 2);
#pragma unroll
                    for (int e = 0; e < 8; ++e) u[e] = (w >> (4 * e)) & 0xFu;
                } else {
                    const uint2 w = *reinterpret_cast<const uint2*>(codes + row * code_ld + c0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { u[e] = (w.x >> (8 * e)) & 0xFFu; u[4 + e] = (w.y >> (8 * e)) & 0xFFu; }
                }
                const int g = (G == 0) ? 0 : (int)(c0 / G);
                const float sc = f16_bits_to_f32(scales[row * n_groups + g]);
                const float z = f16_bits_to_f32(zeros[row * n_groups + g]);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = FP4 ? sc * e2m1_value(u[e]) : sc * ((float)u[e] - z);
                if constexpr (OT == GPTQ_F32) {
                    f32x4_t* o = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + row * d_col + c0);
                    o[0] = f32x4_t{v[0], v[1], v[2], v[3]};
                    o[1] = f32x4_t{v[4], v[5], v[6], v[7]};
                } else {
                    uint32_t p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = (OT == GPTQ_BF16) ? f32_to_bf16_bits(v[2 * e]) : f32_to_f16_bits(v[2 * e]);
                        const uint32_t hi = (OT == GPTQ_BF16) ? f32_to_bf16_bits(v[2 * e + 1]) : f32_to_f16_bits(v[2 * e + 1]);
                        p[e] = lo | (hi << 16);
                    }
                    *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + row * d_col + c0) = u32x4_t{p[0], p[1], p[2], p[3]};
                }
                continue;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t c = c0 + e;
                if (c >= d_col) { v[e] = 0.f; continue; }
                uint32_t u;
                if constexpr (BITS == 3) {
                    u = code3(load_u24(codes + row * code_ld + c / 8 * 3), (int)(c & 7));
                } else if constexpr (BITS <= 4) {
                    const uint8_t b = codes[row * code_ld + (c >> 1)];
                    u = (c & 1) ? (b >> 4) : (b & 0xF);
                } else {
                    u = codes[row * code_ld + c];
                }
                const int g = (G == 0) ? 0 : (int)(c / G);
                const float sc = f16_bits_to_f32(scales[row * n_groups + g]);
                const float z = f16_bits_to_f32(zeros[row * n_groups + g]);
                v[e] = FP4 ? sc * e2m1_value(u) : sc * ((float)u - z);
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
}

template <int BITS, bool FP4 = false>
static gptq_status dq_dt(gptq_dtype ot, dim3 grid, hipStream_t s, const uint8_t* codes, const uint16_t* scales,
                         const uint16_t* zeros, int64_t d_row, int64_t d_col, int G, void* out) {
    switch (ot) {
        case GPTQ_F32: dequant_kernel<BITS, GPTQ_F32, FP4><<<grid, 256, 0, s>>>(codes, scales, zeros, d_row, d_col, G, out); break;
        case GPTQ_BF16: dequant_kernel<BITS, GPTQ_BF16, FP4><<<grid, 256, 0, s>>>(codes, scales, zeros, d_row, d_col, G, out); break;
        case GPTQ_F16: dequant_kernel<BITS, GPTQ_F16, FP4><<<grid, 256, 0, s>>>(codes, scales, zeros, d_row, d_col, G, out); break;
        default: return GPTQ_ERR_UNSUPPORTED;
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

gptq_status dequant_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t d_row,
                           int64_t d_col, int bits, int group_size, void* out, gptq_dtype out_dtype,
                           hipStream_t s, bool fp4) {
    const int64_t chunks = (d_col + 7) / 8;
    dim3 grid((unsigned)std::min<int64_t>((chunks + 255) / 256, 64), (unsigned)std::min<int64_t>(d_row, 65535));
    if (fp4) return dq_dt<4, true>(out_dtype, grid, s, codes, scales, zeros, d_row, d_col, group_size, out);
    if (bits == 3) return dq_dt<3>(out_dtype, grid, s, codes, scales, zeros, d_row, d_col, group_size, out);
    if (bits <= 4) return dq_dt<4>(out_dtype, grid, s, codes, scales, zeros, d_row, d_col, group_size, out);
    return dq_dt<8>(out_dtype, grid, s, codes, scales, zeros, d_row, d_col, group_size, out);
}

// --------------------------------------------------------------------------
// Scratch of gptq_quantize_layer_noalloc, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops): a file-scope device array of fixed size in
// place of the caller's workspace.  Each GPU the library runs on holds its own copy
// until the process ends, and every call on that GPU shares it, keeping the last
// call's contents (nothing in it needs to start at zero: every value a kernel reads is
// written earlier in the same call).  Calls that overlap on one GPU race.  Host code
// never passes the array's name (a host-side stand-in): its device address is looked up
// once per device, with that device current, and that address is what the kernels get.
static __device__ __align__(256) unsigned char scratch[GPTQ_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
static std::once_flag scratch_once[SCRATCH_MAX_DEVICES];
static void* scratch_dev_ptr[SCRATCH_MAX_DEVICES];
static hipError_t scratch_err[SCRATCH_MAX_DEVICES];

static gptq_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return GPTQ_ERR_HIP;
    std::call_once(scratch_once[dev], [dev] {
        void* ptr = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        scratch_dev_ptr[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (scratch_err[dev] != hipSuccess || scratch_dev_ptr[dev] == nullptr) return GPTQ_ERR_HIP;
    *out = scratch_dev_ptr[dev];
    return GPTQ_OK;
}

gptq_status quant_launch_noalloc(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col, const float* U,
                                 const gptq_params& p, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                 int32_t* info, hipStream_t s) {
    if (quant_ws_bytes(d_row, d_col) > GPTQ_NOALLOC_SCRATCH_BYTES) return GPTQ_ERR_UNSUPPORTED;
    void* ws = nullptr;
    const gptq_status st = scratch_address(&ws);
    if (st != GPTQ_OK) return st;
    return quant_launch(W, w_dtype, d_row, d_col, U, p, codes, scales, zeros, ws, GPTQ_NOALLOC_SCRATCH_BYTES, info,
                        s);
}

}  // namespace gptq
