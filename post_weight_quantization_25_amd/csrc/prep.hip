// U = upper Cholesky factor of (H + lambda I)^-1, lambda = percdamp * mean(diag H).
//
// GPTQ summary page, "Innovation 3": the Cholesky decomposition of the inverse
// Hessian is computed once in advance and its rows are read directly during the
// sweep; a small dampening term lambda I handles near-singular H.
//
// Route: with J the reversal permutation, A = J (H + lambda I) J = L L^T (lower
// Cholesky).  Then H + lambda I = (J L J)(J L J)^T with J L J upper triangular,
// and (H + lambda I)^-1 = (J L^-1 J)^T (J L^-1 J), so U = J L^-1 J: one
// factorization and one triangular inverse, (2/3) d^3 flops in all.
//
// Both are done together by a recursive 2 x 2 block algorithm in fp64:
//   [L11, X11] = cholinv(A11)
//   L21 = A21 X11^T;  A22 -= L21 L21^T
//   [L22, X22] = cholinv(A22)
//   X21 = -X22 (L21 X11)
// with X = L^-1.  The leaves (<= 64 columns) run in one workgroup in LDS; the
// block products run on v_mfma_f64_16x16x4_f64, skipping tiles that are zero
// because an operand is triangular.

#include "common.h"
#include "kernels.h"

namespace gptq {

constexpr int PNB = 64;  // leaf size

// --------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prep_lambda_kernel(const float* H, int64_t d, float percdamp,
                                                         double* lam_out, int32_t* info) {
    __shared__ double red[1024];
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    double s = 0.0;
    int b = 0;
    for (int64_t i = threadIdx.x; i < d; i += 1024) {
        const float v = H[i * d + i];
        if (!isfinite(v)) b = 1;
        s += (double)v;
    }
    if (b) atomicOr(&bad, 1);
    red[threadIdx.x] = s;
    __syncthreads();
    for (int st = 512; st > 0; st >>= 1) {
        if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *lam_out = (double)percdamp * (red[0] / (double)d);
        *info = bad ? -1 : 0;
    }
}

// A[i][j] = H[d-1-i][d-1-j] + lambda [i == j] for j <= i; X = 0.
__global__ void prep_build_kernel(const float* H, int64_t d, const double* lam, double* A, double* X) {
    const int64_t i = blockIdx.y;
    const double l = *lam;
    for (int64_t j = blockIdx.x * blockDim.x + threadIdx.x; j < d; j += (int64_t)gridDim.x * blockDim.x) {
        X[i * d + j] = 0.0;
        if (j <= i) {
            double v = (double)H[(d - 1 - i) * d + (d - 1 - j)];
            if (i == j) v += l;
            A[i * d + j] = v;
        }
    }
}

// U[i][j] = X[d-1-i][d-1-j] for j >= i, 0 below the diagonal.
__global__ void prep_output_kernel(const double* X, int64_t d, float* U) {
    const int64_t i = blockIdx.y;
    for (int64_t j = blockIdx.x * blockDim.x + threadIdx.x; j < d; j += (int64_t)gridDim.x * blockDim.x)
        U[i * d + j] = (j >= i) ? (float)X[(d - 1 - i) * d + (d - 1 - j)] : 0.0f;
}

// --------------------------------------------------------------------------
// Leaf: factor the n x n (n <= 64) block A[off.., off..] (lower part read) and
// write its inverse factor X[off.., off..] (full block, zeros above the diagonal).
// On a non-positive (or NaN) pivot j the leaf records j + 1 in *info if no earlier
// failure was recorded; prep_fix_info_kernel then adds the block offset.
__global__ __launch_bounds__(256) void prep_leaf_kernel(const double* A, double* X, int64_t d, int64_t off, int n,
                                                      int32_t* info) {
    __shared__ double a[PNB][PNB + 1];
    __shared__ double x[PNB][PNB + 1];
    __shared__ int fail;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < PNB * PNB; idx += 256) {
        const int i = idx / PNB, j = idx % PNB;
        a[i][j] = (i < n && j <= i) ? A[(off + i) * d + off + j] : 0.0;
        x[i][j] = 0.0;
    }
    if (tid == 0) fail = 0;
    __syncthreads();
    const int i = tid & 63;      // row owned in the column scaling / X row
    const int part = tid >> 6;   // 0..3: column stripe in the trailing update
    for (int j = 0; j < n; ++j) {
        const double piv = a[j][j];
        if (!(piv > 0.0)) {      // uniform across the WG
            if (tid == 0) fail = j + 1;
            break;
        }
        const double l = sqrt(piv);
        __syncthreads();
        if (part == 0) {
            if (i == j) a[j][j] = l;
            else if (i > j && i < n) a[i][j] = a[i][j] / l;
        }
        __syncthreads();
        // trailing update a[r][k] -= a[r][j] a[k][j] for j < k <= r, and X row j
        for (int idx = tid; idx < PNB * PNB; idx += 256) {
            const int r = idx >> 6, k = idx & 63;
            if (k > j && k <= r && r < n) a[r][k] -= a[r][j] * a[k][j];
        }
        // X[j][c] for c < j: -(sum_{k=c}^{j-1} L[j][k] X[k][c]) / L[j][j]; X[j][j] = 1/L[j][j]
        if (part == 1 && i <= j) {
            double v;
            if (i == j) {
                v = 1.0 / l;
            } else {
                double s = 0.0;
                for (int k = i; k < j; ++k) s += a[j][k] * x[k][i];
                v = -s / l;
            }
            x[j][i] = v;
        }
        __syncthreads();
    }
    __syncthreads();
    if (fail) {
        if (tid == 0 && *info == 0) *info = fail;  // local index; host converts
        return;
    }
    for (int idx = tid; idx < n * n; idx += 256) {
        const int r = idx / n, c = idx % n;
        X[(off + r) * d + off + c] = x[r][c];
    }
}

// Non-positive-pivot index conversion: the leaf writes its local j+1; the host
// launches this right after to make it the global order of the failing trailing
// submatrix of H + lambda I (= global pivot index + 1 in the reversed matrix).
__global__ void prep_fix_info_kernel(int32_t* info, int32_t* seen, int64_t off) {
    if (*info > 0 && *seen == 0) { *info = (int32_t)(off + *info); *seen = 1; }
}

// --------------------------------------------------------------------------
// fp64 GEMM on MFMA: C = beta C + alpha A op(B), 64 x 64 tiles, 4 waves (2 x 2 of 32 x 32).
enum : int { G_BT = 1, G_TRI_A = 2, G_TRI_B = 4, G_LOWER_C = 8 };
constexpr int GD_BM = 64, GD_BK = 16, GD_LD = GD_BK + 1;

struct GemmD {
    double* C; int64_t ldc;
    const double* A; int64_t lda;
    const double* B; int64_t ldb;
    int M, N, K;
    double alpha, beta;
    int flags;
};

__global__ __launch_bounds__(256) void gemm_f64_kernel(GemmD g) {
    __shared__ double As[GD_BM * GD_LD];
    __shared__ double Bs[GD_BM * GD_LD];
    const int mi = blockIdx.y, nj = blockIdx.x;
    const int m0 = mi * GD_BM, n0 = nj * GD_BM;
    if ((g.flags & G_LOWER_C) && n0 > m0 + GD_BM - 1) return;
    int kb = 0, ke = g.K;
    if (g.flags & G_TRI_A) ke = min(ke, m0 + GD_BM);           // A lower: A[m][k] = 0 for k > m
    if (g.flags & G_TRI_B) {
        if (g.flags & G_BT) ke = min(ke, n0 + GD_BM);           // B^T lower: Bt[n][k] = 0 for k > n
        else kb = n0;                                           // B lower: B[k][n] = 0 for k < n
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    f64x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{};

    for (int k0 = kb; k0 < ke; k0 += GD_BK) {
        for (int idx = tid; idx < GD_BM * GD_BK; idx += 256) {
            // A tile: m-major rows, k contiguous in memory
            const int m = idx / GD_BK, k = idx % GD_BK;
            const int gm = m0 + m, gk = k0 + k;
            As[m * GD_LD + k] = (gm < g.M && gk < ke) ? g.A[(int64_t)gm * g.lda + gk] : 0.0;
            double bv = 0.0;
            if (g.flags & G_BT) {
                const int gn = n0 + m;
                if (gn < g.N && gk < ke) bv = g.B[(int64_t)gn * g.ldb + gk];
                Bs[m * GD_LD + k] = bv;
            } else {
                const int kk = idx / GD_BM, n = idx % GD_BM;   // coalesced along n
                const int gn = n0 + n, gk2 = k0 + kk;
                if (gn < g.N && gk2 < ke) bv = g.B[(int64_t)gk2 * g.ldb + gn];
                Bs[n * GD_LD + kk] = bv;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GD_BK; kk += 4) {
            double fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = As[(wr * 32 + i * 16 + (lane & 15)) * GD_LD + kk + (lane >> 4)];
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = Bs[(wc * 32 + j * 16 + (lane & 15)) * GD_LD + kk + (lane >> 4)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // v_mfma_f64_16x16x4_f64 result layout: element e of lane l is row 4 e + l / 16
                const int gm = m0 + wr * 32 + i * 16 + 4 * e + (lane >> 4);
                const int gn = n0 + wc * 32 + j * 16 + (lane & 15);
                if (gm < g.M && gn < g.N) {
                    double* c = g.C + (int64_t)gm * g.ldc + gn;
                    const double v = g.alpha * acc[i][j][e];
                    *c = (g.beta == 0.0) ? v : g.beta * *c + v;
                }
            }
}

__global__ void copy_f64_kernel(double* dst, int64_t ldd, const double* src, int64_t lds, int M, int N) {
    const int64_t i = blockIdx.y;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < N; j += gridDim.x * blockDim.x)
        if (i < M) dst[i * ldd + j] = src[i * lds + j];
}

// --------------------------------------------------------------------------
// Host side
struct PrepCtx {
    double* A; double* X; double* T; int64_t d;
    int32_t* info; int32_t* seen; hipStream_t s;
};

static gptq_status gemm(PrepCtx& c, double* C, int64_t ldc, const double* A, int64_t lda, const double* B,
                        int64_t ldb, int M, int N, int K, double alpha, double beta, int flags) {
    if (M <= 0 || N <= 0) return GPTQ_OK;
    GemmD g{C, ldc, A, lda, B, ldb, M, N, K, alpha, beta, flags};
    dim3 grid((N + GD_BM - 1) / GD_BM, (M + GD_BM - 1) / GD_BM);
    gemm_f64_kernel<<<grid, 256, 0, c.s>>>(g);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

static gptq_status cholinv(PrepCtx& c, int64_t off, int64_t n) {
    const int64_t d = c.d;
    if (n <= PNB) {
        prep_leaf_kernel<<<1, 256, 0, c.s>>>(c.A, c.X, d, off, (int)n, c.info);
        GPTQ_LAUNCH_CHECK();
        prep_fix_info_kernel<<<1, 1, 0, c.s>>>(c.info, c.seen, off);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    int64_t h = ((n / 2 + PNB - 1) / PNB) * PNB;
    if (h >= n) h = n - PNB;
    const int64_t n2 = n - h;
    gptq_status st;
    if ((st = cholinv(c, off, h)) != GPTQ_OK) return st;
    double* A21 = c.A + (off + h) * d + off;
    double* A22 = c.A + (off + h) * d + off + h;
    double* X11 = c.X + off * d + off;
    double* X21 = c.X + (off + h) * d + off;
    double* X22 = c.X + (off + h) * d + off + h;
    // L21 = A21 X11^T  -> T (n2 x h)
    if ((st = gemm(c, c.T, h, A21, d, X11, d, (int)n2, (int)h, (int)h, 1.0, 0.0, G_BT | G_TRI_B)) != GPTQ_OK) return st;
    // A22 -= L21 L21^T (lower tiles)
    if ((st = gemm(c, A22, d, c.T, h, c.T, h, (int)n2, (int)n2, (int)h, -1.0, 1.0, G_BT | G_LOWER_C)) != GPTQ_OK) return st;
    // X21 <- L21 X11 (temporary, X21's own storage is untouched by the next call)
    if ((st = gemm(c, X21, d, c.T, h, X11, d, (int)n2, (int)h, (int)h, 1.0, 0.0, G_TRI_B)) != GPTQ_OK) return st;
    if ((st = cholinv(c, off + h, n2)) != GPTQ_OK) return st;
    // X21 = -X22 (L21 X11)  via T
    if ((st = gemm(c, c.T, h, X22, d, X21, d, (int)n2, (int)h, (int)n2, -1.0, 0.0, G_TRI_A)) != GPTQ_OK) return st;
    dim3 grid(((int)h + 255) / 256 < 64 ? ((int)h + 255) / 256 : 64, (unsigned)n2);
    copy_f64_kernel<<<grid, 256, 0, c.s>>>(X21, d, c.T, h, (int)n2, (int)h);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t prep_ws_bytes(int64_t d) {
    if (d <= 0) return 0;
    const size_t dd = (size_t)d * d * sizeof(double);
    const size_t t = (size_t)(d / 2 + PNB) * (d / 2 + PNB) * sizeof(double);
    return align256(dd) * 2 + align256(t) + 256;
}

gptq_status prep_launch(const float* H, float* U, int64_t d, float percdamp, void* ws, size_t ws_bytes,
                        int32_t* info, hipStream_t s) {
    if (ws == nullptr || ws_bytes < prep_ws_bytes(d)) return GPTQ_ERR_WORKSPACE;
    char* p = reinterpret_cast<char*>(ws);
    const size_t dd = align256((size_t)d * d * sizeof(double));
    PrepCtx c;
    c.A = reinterpret_cast<double*>(p);
    c.X = reinterpret_cast<double*>(p + dd);
    c.T = reinterpret_cast<double*>(p + 2 * dd);
    const size_t t = align256((size_t)(d / 2 + PNB) * (d / 2 + PNB) * sizeof(double));
    double* lam = reinterpret_cast<double*>(p + 2 * dd + t);
    c.seen = reinterpret_cast<int32_t*>(p + 2 * dd + t + 8);
    c.d = d; c.info = info; c.s = s;

    prep_lambda_kernel<<<1, 1024, 0, s>>>(H, d, percdamp, lam, info);
    GPTQ_LAUNCH_CHECK();
    fill_i32(c.seen, 1, 0, s);
    GPTQ_LAUNCH_CHECK();
    dim3 gb((unsigned)((d + 255) / 256 < 64 ? (d + 255) / 256 : 64), (unsigned)d);
    prep_build_kernel<<<gb, 256, 0, s>>>(H, d, lam, c.A, c.X);
    GPTQ_LAUNCH_CHECK();
    gptq_status st = cholinv(c, 0, d);
    if (st != GPTQ_OK) return st;
    prep_output_kernel<<<gb, 256, 0, s>>>(c.X, d, U);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
