// H += 2 X^T X on gfx950 matrix cores.
//
// GPTQ summary page, statement of the one-layer procedure: the layer Hessian
// H = 2 X X^T (page layout d_col x tokens; here X is tokens x d_col, so H = 2 X^T X).
//
// bf16 X: a symmetric rank-k update on v_mfma_f32_32x32x16_bf16.  Only tiles
// on or above the diagonal are computed (128 x 128 output tiles).  X is stored
// token-major (channels contiguous), i.e. the contraction index is the strided
// one, so each thread loads an 8-token x 8-channel patch with 16-byte loads and
// transposes it in registers (v_perm_b32) before writing channel-major rows to
// LDS, from where MFMA fragments are read with one 16-byte LDS read each.
// The token range is split S ways; work items are ordered split-major and the
// grid is mapped so that each XCD (workgroups are dealt round-robin to the 8
// XCDs) runs a contiguous range of work items, so the WGs sharing an XCD's L2
// walk the same token slab at the same time.  Each work item writes its fp32
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
constexpr int HB_BM = 128;           // tile edge (channels)
constexpr int HB_BK = 64;            // tokens per LDS stage
constexpr int HB_LD = HB_BK + 8;     // padded row (bf16 elements): 144 B, 16 B aligned
constexpr int HB_THREADS = 256;

struct HessBf16Args {
    const uint16_t* X; int64_t n; int d; int64_t ldx;
    float* H; float* partials; int* counters;
    int nt; int T; int S; int64_t ks;  // tokens per split (multiple of HB_BK)
    int per_xcd; int total;
};

// Load an 8-token x 8-channel patch (rows t..t+7, channels c..c+7) as 8 x 16 B.
GPTQ_DEV void load_patch(const HessBf16Args& a, int64_t t, int c, int64_t t_end, bool vec_ok, u32x4_t (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t tt = t + i;
        if (tt < t_end && vec_ok && c + 8 <= a.d) {
            r[i] = *reinterpret_cast<const u32x4_t*>(a.X + tt * a.ldx + c);
        } else {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (tt < t_end) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t v = (c + e < a.d) ? (uint32_t)a.X[tt * a.ldx + c + e] : 0u;
                    w[e >> 1] |= v << (16 * (e & 1));
                }
            }
            r[i] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
}

// Transpose the patch and store channel-major (8 rows of 8 tokens) into LDS.
GPTQ_DEV void store_patch_t(uint16_t* lds_tile, int crow, int tcol, const u32x4_t (&r)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        const int dw = c >> 1;
        u32x4_t o;
        o[0] = __builtin_amdgcn_perm(r[1][dw], r[0][dw], sel);
        o[1] = __builtin_amdgcn_perm(r[3][dw], r[2][dw], sel);
        o[2] = __builtin_amdgcn_perm(r[5][dw], r[4][dw], sel);
        o[3] = __builtin_amdgcn_perm(r[7][dw], r[6][dw], sel);
        *reinterpret_cast<u32x4_t*>(lds_tile + (crow + c) * HB_LD + tcol) = o;
    }
}

__global__ __launch_bounds__(HB_THREADS, 2) void hess_bf16_kernel(HessBf16Args a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][HB_BM * HB_LD];  // 73728 B
    __shared__ int last_flag;

    const int L = blockIdx.x;
    const int xcd = L & 7, local = L >> 3;
    const int w = xcd * a.per_xcd + local;
    if (local >= a.per_xcd || w >= a.total) return;
    const int s = w / a.T, tile = w % a.T;
    int ti, tj;
    upper_tile(tile, a.nt, ti, tj);
    const int c0 = ti * HB_BM, c1 = tj * HB_BM;
    const int64_t t_beg = (int64_t)s * a.ks;
    const int64_t t_end = (t_beg + a.ks < a.n) ? t_beg + a.ks : a.n;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    // loader role: 128 threads per operand, 16 channel groups x 8 token groups
    const int which = tid >> 7;
    const int u = tid & 127;
    const int cg = u & 15, tg = u >> 4;
    const int lc = (which ? c1 : c0) + cg * 8;
    const bool vec_ok = ((reinterpret_cast<uintptr_t>(a.X) & 15) == 0) && ((a.ldx & 7) == 0);

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    const int64_t nst = (t_end > t_beg) ? (t_end - t_beg + HB_BK - 1) / HB_BK : 0;
    u32x4_t r[8];
    if (nst > 0) {
        load_patch(a, t_beg + tg * 8, lc, t_end, vec_ok, r);
        store_patch_t(&lds[0][which][0], cg * 8, tg * 8, r);
    }
    __syncthreads();

    for (int64_t st = 0; st < nst; ++st) {
        const int buf = (int)(st & 1);
        const bool more = st + 1 < nst;
        if (more) load_patch(a, t_beg + (st + 1) * HB_BK + tg * 8, lc, t_end, vec_ok, r);

        const uint16_t* A = &lds[buf][0][0];
        const uint16_t* B = &lds[buf][1][0];
#pragma unroll
        for (int kk = 0; kk < HB_BK; kk += 16) {
            const int koff = kk + (lane >> 5) * 8;
            bf16x8_t fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wr * 64 + i * 32 + (lane & 31);
                fa[i] = *reinterpret_cast<const bf16x8_t*>(A + row * HB_LD + koff);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = wc * 64 + j * 32 + (lane & 31);
                fb[j] = *reinterpret_cast<const bf16x8_t*>(B + col * HB_LD + koff);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (more) store_patch_t(&lds[buf ^ 1][which][0], cg * 8, tg * 8, r);
        __syncthreads();
    }

    // write this split's partial tile (row-major 128 x 128 fp32)
    float* P = a.partials + (int64_t)w * (HB_BM * HB_BM);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = wr * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int nn = wc * 64 + j * 32 + (lane & 31);
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

    // last arriver: sum partials in split order, update H (upper triangle authoritative)
    float* sum = reinterpret_cast<float*>(&lds[0][0][0]);  // 128 x 129 fp32 = 66048 B
    constexpr int SLD = HB_BM + 1;
    for (int idx = tid; idx < HB_BM * HB_BM; idx += HB_THREADS) {
        const int m = idx >> 7, nn = idx & 127;
        float v = 0.f;
        for (int ss = 0; ss < a.S; ++ss)
            v += __builtin_nontemporal_load(a.partials + ((int64_t)ss * a.T + tile) * (HB_BM * HB_BM) + idx);
        const int gr = c0 + m, gc = c1 + nn;
        if (gr < a.d && gc < a.d && gr <= gc) {
            const float nv = a.H[(int64_t)gr * a.d + gc] + 2.f * v;
            a.H[(int64_t)gr * a.d + gc] = nv;
            sum[m * SLD + nn] = nv;
        }
    }
    __syncthreads();
    // mirror into the lower triangle, coalesced along the H row (index m)
    for (int idx = tid; idx < HB_BM * HB_BM; idx += HB_THREADS) {
        const int nn = idx >> 7, m = idx & 127;
        const int gr = c0 + m, gc = c1 + nn;
        if (gr < a.d && gc < a.d && gr < gc) a.H[(int64_t)gc * a.d + gr] = sum[m * SLD + nn];
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

static void bf16_plan(int64_t n, int64_t d, int& nt, int& T, int& S, int64_t& ks) {
    nt = (int)((d + HB_BM - 1) / HB_BM);
    T = nt * (nt + 1) / 2;
    const int64_t nst = (n + HB_BK - 1) / HB_BK;
    // split count: enough work items to fill 512 WG slots with a small tail,
    // bounded so that the partial tiles stay a small fraction of the X traffic
    const int slots = 512;
    int best = 1;
    double best_cost = 1e300;
    for (int s = 1; s <= 32; ++s) {
        if (s > 1 && (int64_t)s > nst) break;
        const double items = (double)T * s;
        const double rounds = items / slots;
        const double eff = rounds / std::ceil(rounds);
        // compute time ~ 1/eff; partial traffic ~ s * T tiles * 128 KB vs X traffic
        const double x_bytes = (double)n * d * 2.0;
        const double p_bytes = (double)s * T * HB_BM * HB_BM * 4.0 * 2.0;
        const double cost = 1.0 / eff + 0.5 * p_bytes / (x_bytes + 1.0);
        if (cost < best_cost - 1e-9) { best_cost = cost; best = s; }
    }
    S = best;
    ks = ((nst + S - 1) / S) * HB_BK;
}

size_t hessian_ws_bytes(int64_t n, int64_t d) {
    if (n <= 0 || d <= 0) return 0;
    int nt, T, S; int64_t ks;
    bf16_plan(n, d, nt, T, S, ks);
    const size_t cnt = ((size_t)T * sizeof(int) + 255) & ~(size_t)255;
    return cnt + (size_t)T * S * HB_BM * HB_BM * sizeof(float);
}

gptq_status hessian_launch(float* H, const void* X, gptq_dtype dt, int64_t n, int64_t d, int64_t ldx,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && ((ldx & 7) == 0);
    if (dt == GPTQ_BF16 && aligned) {
        HessBf16Args a;
        int nt, T, S; int64_t ks;
        bf16_plan(n, d, nt, T, S, ks);
        if (ws_bytes < hessian_ws_bytes(n, d) || ws == nullptr) return GPTQ_ERR_WORKSPACE;
        const size_t cnt = ((size_t)T * sizeof(int) + 255) & ~(size_t)255;
        a.X = reinterpret_cast<const uint16_t*>(X); a.n = n; a.d = (int)d; a.ldx = ldx;
        a.H = H; a.counters = reinterpret_cast<int*>(ws);
        a.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + cnt);
        a.nt = nt; a.T = T; a.S = S; a.ks = ks;
        a.total = T * S;
        a.per_xcd = (a.total + 7) / 8;
        fill_i32(a.counters, T, 0, stream);
        GPTQ_LAUNCH_CHECK();
        hess_bf16_kernel<<<a.per_xcd * 8, HB_THREADS, 0, stream>>>(a);
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
