// H += 2 X^T X on gfx950 matrix cores.
//
// GPTQ summary page, statement of the one-layer procedure: the layer Hessian
// H = 2 X X^T (page layout d_col x tokens; here X is tokens x d_col, so H = 2 X^T X).
//
// bf16 X: a symmetric rank-k update on v_mfma_f32_32x32x16_bf16.  Only tiles
// on or above the diagonal are computed (256 x 256 output tiles, one workgroup of
// eight waves per CU, each wave accumulating a 64 x 128 sub-tile in 8 MFMAs).  X is stored
// token-major (channels contiguous), i.e. the contraction index is the strided
// one.  Tiles are copied to LDS as they lie in memory (coalesced 16-byte loads,
// conflict-free 16-byte LDS writes) and the MFMA operands, which need 8
// consecutive tokens of one channel per lane, are read with the gfx950
// transposing LDS read ds_read_b64_tr_b16.
// Global loads run one 64-token stage ahead of the MFMAs, LDS is double
// buffered.  The token range is split S ways; each XCD (workgroups are
// dealt round-robin to the 8 XCDs) owns a compact range of tiles and walks the
// splits in order, so all XCDs read the same token slab at about the same time.  Each work item writes its fp32
// partial tile; the last work item of a tile to finish (tile counter) sums the
// S partials in split order and updates H, so results are bitwise reproducible.
//
// fp32 / fp16 X: exact-product path on v_mfma_f32_16x16x4_f32, one WG per
// 64 x 64 upper tile over all tokens (no split).

#include <cmath>

#include "common.h"
#include "kernels.h"

namespace gptq {

// ----------------------------------------------------------------------------
// Tile enumeration: upper-triangle tiles grouped into 8 x 8 super-tiles.
__host__ __device__ inline void upper_tile(int idx, int nt, int& ti, int& tj) {
    constexpr int SG = 8;
    const int nT = (nt + SG - 1) / SG;
    for (int R = 0; R < nT; ++R) {
        const int r0 = R * SG, r1 = (r0 + SG < nt) ? r0 + SG : nt, h = r1 - r0;
        const int rowtot = h * nt - ((r0 + r1 - 1) * h) / 2;
        if (idx >= rowtot) { idx -= rowtot; continue; }
        const int dtot = h * (h + 1) / 2;
        if (idx < dtot) {
            int a = 0;
            while (idx >= h - a) { idx -= h - a; ++a; }
            ti = r0 + a; tj = r0 + a + idx; return;
        }
        idx -= dtot;
        for (int C = R + 1; C < nT; ++C) {
            const int c0 = C * SG, w = ((c0 + SG < nt) ? c0 + SG : nt) - c0;
            if (idx < h * w) { ti = r0 + idx / w; tj = c0 + idx % w; return; }
            idx -= h * w;
        }
    }
    ti = tj = -1;
}

// ----------------------------------------------------------------------------
// bf16 path
constexpr int HB_BM = 256;           // tile edge (channels)
constexpr int HB_BK = 64;            // tokens per LDS stage
constexpr int HB_RS = HB_BM + 16;    // LDS row = one token: 256 channels + pad (544 B = 136 dwords)
constexpr int HB_THREADS = 512;      // 8 waves: wave (wr, wc) owns rows wr*64.., columns wc*128..
constexpr int HB_SLICE = 32;         // rows per LDS-staged slice of the final reduction
constexpr int HB_TILE = HB_BK * HB_RS;  // bf16 elements of one operand stage

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

struct HessBf16Args {
    const uint16_t* X; int64_t n; int d; int64_t ldx;
    float* H; float* partials; int* counters;
    int nt; int T; int S; int64_t ks;  // tokens per split (multiple of HB_BK)
    int tpx;                           // tiles per XCD
};

// One thread's share of a stage: 8 chunks of 8 channels (16 B) from token rows
// k = kr + 8 i of the stage, channel chunk cc (lanes consecutive in cc: 512 B per row).
template <bool FULL>
GPTQ_DEV void load_stage(const HessBf16Args& a, int64_t t0, int64_t t_end, int c, int kr, u32x4_t (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t t = t0 + kr + 8 * i;
        if constexpr (FULL) {
            r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.X + t * a.ldx + c));
        } else {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (t < t_end) {
                if (c + 8 <= a.d) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.X + t * a.ldx + c);
                    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
                } else {
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t v = (c + e < a.d) ? (uint32_t)a.X[t * a.ldx + c + e] : 0u;
                        w[e >> 1] |= v << (16 * (e & 1));
                    }
                }
            }
            r[i] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
}

// Store the chunks token-major (the layout they have in memory): conflict-free 16 B writes.
GPTQ_DEV void store_stage(uint16_t* tile, int cc, int kr, const u32x4_t (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(tile + (kr + 8 * i) * HB_RS + cc * 8) = r[i];
}

// MFMA operand fragment (32 channels x 16 tokens, lane l: channel l % 32, tokens
// 8 (l / 32) .. +7) read from the token-major tile with two ds_read_b64_tr_b16.
// Within each 16-lane group the instruction returns to lane i, element e, the
// (i & 3)-th value of the 8-byte chunk addressed by lane (i >> 2) + 4 e; lane j
// therefore addresses token k0 + (j >> 2), channels m0 + 4 (j & 3) .. +3, and lane i
// receives channel m0 + i at tokens k0 .. k0 + 3.
GPTQ_DEV bf16x8_t read_frag(const uint16_t* tile, int ch0, int kk, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int m0 = ch0 + (g & 1) * 16 + 4 * (j & 3);
    const int k0 = kk + (g >> 1) * 8 + (j >> 2);
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + k0 * HB_RS + m0));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + (k0 + 4) * HB_RS + m0));
    typedef short v8i16_t __attribute__((ext_vector_type(8)));
    const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// The MFMAs of one LDS stage for one wave: 2 x 4 tiles of 32 x 32, four k16 slices.
GPTQ_DEV void mfma_stage(const uint16_t* A, const uint16_t* B, int wr, int wc, int lane, f32x16_t (&acc)[2][4]) {
#pragma unroll
    for (int kk = 0; kk < HB_BK; kk += 16) {
        bf16x8_t fa[2], fb[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = read_frag(A, wr * 64 + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = read_frag(B, wc * 128 + j * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
}

// Main loop: stage st in LDS buffer st & 1; the registers hold stage st + 1.
template <bool FULL>
GPTQ_DEV void hess_main_loop(const HessBf16Args& a, uint16_t (*lds)[2][HB_TILE], int64_t t_beg, int64_t t_end,
                             int64_t nst, int which, int cc, int kr, int lc, int wr, int wc, int lane,
                             f32x16_t (&acc)[2][4]) {
    u32x4_t r[8];
    if (nst <= 0) return;
    // a load past the last stage re-reads the last stage (in bounds, unused), so every
    // iteration issues the same loads and the waits count them exactly
    auto t0 = [&](int64_t st) { return t_beg + (st < nst ? st : nst - 1) * HB_BK; };
    load_stage<FULL>(a, t0(0), t_end, lc, kr, r);
    store_stage(&lds[0][which][0], cc, kr, r);
    load_stage<FULL>(a, t0(1), t_end, lc, kr, r);
    __syncthreads();
    int64_t st = 0;
    for (; st + 1 < nst; st += 2) {
        mfma_stage(&lds[0][0][0], &lds[0][1][0], wr, wc, lane, acc);
        store_stage(&lds[1][which][0], cc, kr, r);
        load_stage<FULL>(a, t0(st + 2), t_end, lc, kr, r);
        __syncthreads();
        mfma_stage(&lds[1][0][0], &lds[1][1][0], wr, wc, lane, acc);
        store_stage(&lds[0][which][0], cc, kr, r);
        load_stage<FULL>(a, t0(st + 3), t_end, lc, kr, r);
        __syncthreads();
    }
    if (st < nst) mfma_stage(&lds[0][0][0], &lds[0][1][0], wr, wc, lane, acc);
}

__global__ __launch_bounds__(HB_THREADS, 1) void hess_bf16_kernel(HessBf16Args a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][HB_TILE];  // 139264 B
    __shared__ int last_flag;

    // XCD-aware work mapping: workgroup L runs on XCD L % 8.  Each XCD owns a
    // contiguous range of tpx tiles and walks the splits in order, so at any time
    // all XCDs read the same token slab (shared through the Infinity Cache) and the
    // workgroups of one XCD share channel blocks through its L2.
    const int L = blockIdx.x;
    const int xcd = L & 7, k = L >> 3;
    const int s = k / a.tpx, tile = xcd * a.tpx + k % a.tpx;
    if (s >= a.S || tile >= a.T) return;
    int ti, tj;
    upper_tile(tile, a.nt, ti, tj);
    const int c0 = ti * HB_BM, c1 = tj * HB_BM;
    const int64_t t_beg = (int64_t)s * a.ks;
    const int64_t t_end = (t_beg + a.ks < a.n) ? t_beg + a.ks : a.n;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    // loader role: 256 threads per operand; 32 channel chunks (fastest) x 8 token rows
    const int which = tid >> 8;
    const int u = tid & 255;
    const int cc = u & 31, kr = u >> 5;
    const int lc = (which ? c1 : c0) + cc * 8;

    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

    const int64_t nst = (t_end > t_beg) ? (t_end - t_beg + HB_BK - 1) / HB_BK : 0;
    const bool full = (c0 + HB_BM <= a.d) && (c1 + HB_BM <= a.d) && ((t_end - t_beg) % HB_BK == 0) &&
                      ((reinterpret_cast<uintptr_t>(a.X) & 15) == 0) && ((a.ldx & 7) == 0);
    if (full) hess_main_loop<true>(a, lds, t_beg, t_end, nst, which, cc, kr, lc, wr, wc, lane, acc);
    else hess_main_loop<false>(a, lds, t_beg, t_end, nst, which, cc, kr, lc, wr, wc, lane, acc);

    // this split's partial tile (row-major 256 x 256 fp32)
    float* P = a.partials + ((int64_t)s * a.T + tile) * (HB_BM * HB_BM);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = wr * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int nn = wc * 128 + j * 32 + (lane & 31);
                P[m * HB_BM + nn] = acc[i][j][e];
            }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int old = atomicAdd(&a.counters[tile], 1);
        last_flag = (old == a.S - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();

    // last arriver: sum the partials in split order, update the upper triangle of H,
    // and mirror it into the lower triangle through an LDS-staged transpose
    float* st_lds = reinterpret_cast<float*>(&lds[0][0][0]);  // HB_SLICE x (HB_BM + 1) fp32
    constexpr int SLD = HB_BM + 1;
    for (int m0 = 0; m0 < HB_BM; m0 += HB_SLICE) {
        for (int idx = tid; idx < HB_SLICE * HB_BM; idx += HB_THREADS) {
            const int ml = idx / HB_BM, nn = idx % HB_BM, m = m0 + ml;
            const int gr = c0 + m, gc = c1 + nn;
            if (gr < a.d && gc < a.d && gr <= gc) {
                float v = 0.f;
                for (int ss = 0; ss < a.S; ++ss)
                    v += __builtin_nontemporal_load(a.partials + ((int64_t)ss * a.T + tile) * (HB_BM * HB_BM) + m * HB_BM + nn);
                const float nv = a.H[(int64_t)gr * a.d + gc] + 2.f * v;
                a.H[(int64_t)gr * a.d + gc] = nv;
                st_lds[ml * SLD + nn] = nv;
            }
        }
        __syncthreads();
        for (int idx = tid; idx < HB_SLICE * HB_BM; idx += HB_THREADS) {
            const int nn = idx / HB_SLICE, ml = idx % HB_SLICE, m = m0 + ml;
            const int gr = c0 + m, gc = c1 + nn;
            if (gr < a.d && gc < a.d && gr < gc) a.H[(int64_t)gc * a.d + gr] = st_lds[ml * SLD + nn];
        }
        __syncthreads();
    }
    if (tid == 0) a.counters[tile] = 0;
}

__global__ void fill_i32_kernel(int* p, int n, int v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

void fill_i32(int32_t* p, int n, int v, hipStream_t s) {
    fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
}

// ----------------------------------------------------------------------------
// fp32 / fp16 / unaligned path: fp32 MFMA 16x16x4, 64 x 64 tiles, one WG per tile.
constexpr int HF_BM = 64;
constexpr int HF_BK = 32;
constexpr int HF_LD = HF_BK + 1;

template <gptq_dtype DT>
__global__ __launch_bounds__(256) void hess_f32_kernel(const void* X, int64_t n, int d, int64_t ldx, float* H, int nt) {
    __shared__ float As[HF_BM * HF_LD];
    __shared__ float Bs[HF_BM * HF_LD];
    int ti, tj;
    {
        // plain row-major upper-triangle enumeration
        int idx = blockIdx.x, r = 0;
        while (idx >= nt - r) { idx -= nt - r; ++r; }
        ti = r; tj = r + idx;
    }
    const int c0 = ti * HF_BM, c1 = tj * HF_BM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{};

    for (int64_t t0 = 0; t0 < n; t0 += HF_BK) {
        for (int idx = tid; idx < HF_BM * HF_BK; idx += 256) {
            const int c = idx % HF_BM, k = idx / HF_BM;
            const int64_t t = t0 + k;
            float va = 0.f, vb = 0.f;
            if (t < n) {
                if (c0 + c < d) va = load_as_f32<DT>(X, t * ldx + c0 + c);
                if (c1 + c < d) vb = load_as_f32<DT>(X, t * ldx + c1 + c);
            }
            As[c * HF_LD + k] = va;
            Bs[c * HF_LD + k] = vb;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < HF_BK; k += 4) {
            float fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = As[(wr * 32 + i * 16 + (lane & 15)) * HF_LD + k + (lane >> 4)];
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = Bs[(wc * 32 + j * 16 + (lane & 15)) * HF_LD + k + (lane >> 4)];
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
                const int gr = c0 + wr * 32 + i * 16 + 4 * (lane >> 4) + e;
                const int gc = c1 + wc * 32 + j * 16 + (lane & 15);
                if (gr < d && gc < d && gr <= gc) {
                    const float nv = H[(int64_t)gr * d + gc] + 2.f * acc[i][j][e];
                    H[(int64_t)gr * d + gc] = nv;
                    if (gr != gc) H[(int64_t)gc * d + gr] = nv;
                }
            }
}

// ----------------------------------------------------------------------------
// Host side

static void bf16_plan(int64_t n, int64_t d, int& nt, int& T, int& S, int64_t& ks, int& tpx) {
    nt = (int)((d + HB_BM - 1) / HB_BM);
    T = nt * (nt + 1) / 2;
    tpx = (T + 7) / 8;
    const int64_t nst = (n + HB_BK - 1) / HB_BK;
    // split count: whole rounds of the 256 workgroup slots (one per CU) with a small
    // tail, while the partial tiles (S * T * 256 KB written and read back) stay a
    // small fraction of the activation traffic
    const int slots = 256;
    int best = 1;
    double best_cost = 1e300;
    for (int sp = 1; sp <= 64; ++sp) {
        if (sp > 1 && (int64_t)sp > nst) break;
        const double items = 8.0 * tpx * sp;
        const double rounds = items / slots;
        const double eff = ((double)T * sp / slots) / std::ceil(rounds);
        const double x_bytes = (double)n * d * 2.0;
        const double p_bytes = (double)sp * T * HB_BM * HB_BM * 4.0 * 2.0;
        const double cost = 1.0 / eff + 0.5 * p_bytes / (x_bytes + 1.0);
        if (cost < best_cost - 1e-9) { best_cost = cost; best = sp; }
    }
    S = best;
    ks = ((nst + S - 1) / S) * HB_BK;
}

size_t hessian_ws_bytes(int64_t n, int64_t d) {
    if (n <= 0 || d <= 0) return 0;
    int nt, T, S, tpx; int64_t ks;
    bf16_plan(n, d, nt, T, S, ks, tpx);
    const size_t cnt = ((size_t)T * sizeof(int) + 255) & ~(size_t)255;
    return cnt + (size_t)T * S * HB_BM * HB_BM * sizeof(float);
}

gptq_status hessian_launch(float* H, const void* X, gptq_dtype dt, int64_t n, int64_t d, int64_t ldx,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && ((ldx & 7) == 0);
    if (dt == GPTQ_BF16 && aligned) {
        HessBf16Args a;
        int nt, T, S, tpx; int64_t ks;
        bf16_plan(n, d, nt, T, S, ks, tpx);
        if (ws_bytes < hessian_ws_bytes(n, d) || ws == nullptr) return GPTQ_ERR_WORKSPACE;
        const size_t cnt = ((size_t)T * sizeof(int) + 255) & ~(size_t)255;
        a.X = reinterpret_cast<const uint16_t*>(X); a.n = n; a.d = (int)d; a.ldx = ldx;
        a.H = H; a.counters = reinterpret_cast<int*>(ws);
        a.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + cnt);
        a.nt = nt; a.T = T; a.S = S; a.ks = ks; a.tpx = tpx;
        fill_i32(a.counters, T, 0, stream);
        GPTQ_LAUNCH_CHECK();
        hess_bf16_kernel<<<8 * S * tpx, HB_THREADS, 0, stream>>>(a);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    const int nt = (int)((d + HF_BM - 1) / HF_BM);
    const int T = nt * (nt + 1) / 2;
    switch (dt) {
        case GPTQ_F32: hess_f32_kernel<GPTQ_F32><<<T, 256, 0, stream>>>(X, n, (int)d, ldx, H, nt); break;
        case GPTQ_F16: hess_f32_kernel<GPTQ_F16><<<T, 256, 0, stream>>>(X, n, (int)d, ldx, H, nt); break;
        case GPTQ_BF16: hess_f32_kernel<GPTQ_BF16><<<T, 256, 0, stream>>>(X, n, (int)d, ldx, H, nt); break;
        default: return GPTQ_ERR_UNSUPPORTED;
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
