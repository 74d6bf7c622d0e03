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
// Both in fp64: a right-looking blocked Cholesky with 64-column panels (the
// diagonal block is factored and inverted in one workgroup, the panel below it is
// multiplied by that inverse, the trailing matrix gets a rank-64 update), then
// X = L^-1 from the inverted diagonal blocks by recursive doubling over block
// pairs, X[q][p] = -X[q][q] (L[q][p] X[p][p]), each level one batched product.
// The block products run on v_mfma_f64_16x16x4_f64 and skip tiles that are zero
// because an operand is triangular.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gptq {

constexpr int PNB = 64;  // leaf size

// --------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prep_lambda_kernel(const float* H, int64_t d, float percdamp,
                                                         double* lam_out, int32_t* info, int* flag) {
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
        *flag = 0;    // no diagonal block published yet in this call
    }
}

// A[i][j] = H[d-1-i][d-1-j] + lambda [i == j] for j <= i.  Neither triangle above the
// diagonal is ever read: the diagonal 64 x 64 blocks of L and X are written whole (zeros
// above the diagonal) by the diagonal routine, the products clip their k ranges to
// those blocks and the ones below, and the output reads the lower part of X only; so X
// needs no initialization.
// VEC (d a multiple of 4, H 16-byte aligned): each thread moves four columns, one
// 16-byte load of H (the four values in reverse order) and two 16-byte stores of A.
template <bool VEC>
__global__ void prep_build_kernel(const float* H, int64_t d, const double* lam, double* A) {
    const int64_t i = blockIdx.y;
    const double l = *lam;
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VEC) {
        const float* hrow = H + (d - 1 - i) * d;
        for (int64_t j = 4 * (blockIdx.x * blockDim.x + threadIdx.x); j <= i; j += 4 * nth) {
            const f32x4_t h = *reinterpret_cast<const f32x4_t*>(hrow + (d - 4 - j));   // columns d-4-j .. d-1-j
            double v[4] = {(double)h[3], (double)h[2], (double)h[1], (double)h[0]};  // A columns j .. j+3
            if (j + 3 <= i) {
                if (i - j < 4) v[i - j] += l;
                *reinterpret_cast<double2*>(A + i * d + j) = double2{v[0], v[1]};
                *reinterpret_cast<double2*>(A + i * d + j + 2) = double2{v[2], v[3]};
            } else {
                for (int e = 0; e < 4 && j + e <= i; ++e) A[i * d + j + e] = v[e] + ((j + e == i) ? l : 0.0);
            }
        }
        return;
    }
    for (int64_t j = blockIdx.x * blockDim.x + threadIdx.x; j <= i; j += nth) {
        double v = (double)H[(d - 1 - i) * d + (d - 1 - j)];
        if (i == j) v += l;
        A[i * d + j] = v;
    }
}

// U[i][j] = X[d-1-i][d-1-j] for j >= i, 0 below the diagonal.  VEC (d a multiple of
// 4, U 16-byte aligned): each thread writes four columns with one 16-byte store (from
// two 16-byte loads of X where any of the four lies on or above the diagonal; the
// values read from X's unwritten upper part are discarded).
template <bool VEC>
__global__ void prep_output_kernel(const double* X, int64_t d, float* U) {
    const int64_t i = blockIdx.y;
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VEC) {
        const double* xrow = X + (d - 1 - i) * d;
        for (int64_t j = 4 * (blockIdx.x * blockDim.x + threadIdx.x); j < d; j += 4 * nth) {
            f32x4_t u = {0.f, 0.f, 0.f, 0.f};
            if (j + 3 >= i) {
                const double2 a = *reinterpret_cast<const double2*>(xrow + (d - 4 - j));   // X columns d-4-j, d-3-j
                const double2 b = *reinterpret_cast<const double2*>(xrow + (d - 2 - j));   // d-2-j, d-1-j
                const double v[4] = {b.y, b.x, a.y, a.x};                                  // U columns j .. j+3
#pragma unroll
                for (int e = 0; e < 4; ++e) u[e] = (j + e >= i) ? (float)v[e] : 0.f;
            }
            *reinterpret_cast<f32x4_t*>(U + i * d + j) = u;
        }
        return;
    }
    for (int64_t j = blockIdx.x * blockDim.x + threadIdx.x; j < d; j += nth)
        U[i * d + j] = (j >= i) ? (float)X[(d - 1 - i) * d + (d - 1 - j)] : 0.0f;
}

// --------------------------------------------------------------------------
// Diagonal block k (n <= 64 columns at offset k0, fully updated by the earlier
// panels): Cholesky A_kk = L_kk L_kk^T in place (lower part), one workgroup.
// The block is processed in 8-column sub-panels.  For a sub-panel, every lane of
// wave 0 factors the sub-panel's 8 x 8 top block redundantly in registers (no
// cross-lane traffic) and then solves its own row of the sub-panel against it;
// afterwards the four waves apply the rank-8 update to the rest of the block on
// v_mfma_f64_16x16x4_f64.  Then X_kk = L_kk^-1 is built in LDS (8 x 8 diagonal
// blocks by substitution, then recursive doubling).  Writes L_kk (lower) and X_kk.
// On a non-positive (or NaN) pivot j the first failure is recorded as
// info = k0 + j + 1, the order of the trailing principal submatrix of H + lambda I
// that is not positive definite.
constexpr int DLD = PNB + 1;

// LDS of the diagonal routine: the block (padded rows), its inverse, and the
// recursive-doubling temporaries (at most one 32 x 32 product, or two 16 x 16).
constexpr int DIAG_TS = 32 * 32;
constexpr int DIAG_LDS_DOUBLES = 2 * PNB * DLD + DIAG_TS;

// Inverse of the 8 x 8 lower block of L at rows / columns o .. o + 7 into xs, by
// forward substitution; lane c < 8 computes column c.
GPTQ_DEV void diag_inv8(const double* a, double* xs, int o, int c) {
    double x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        double v = (i == c) ? 1.0 : 0.0;
#pragma unroll
        for (int k = 0; k < i; ++k) v -= a[(o + i) * DLD + o + k] * x[k];
        x[i] = v / a[(o + i) * DLD + o + i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[(o + i) * DLD + o + c] = (i >= c) ? x[i] : 0.0;
}

// One 16 x 16 tile of a rank-8 update on MFMA: a[R0.., C0..] -= L[R0.., cL..cL+7]
// L[C0.., cL..cL+7]^T, stored where row and column are >= cmask.
GPTQ_DEV void diag_upd_tile(double* a, int R0, int C0, int cL, int cmask, int lane) {
    f64x4_t acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = a[(R0 + 4 * e + (lane >> 4)) * DLD + C0 + (lane & 15)];
#pragma unroll
    for (int kk = 0; kk < 8; kk += 4) {
        const double fa = -a[(R0 + (lane & 15)) * DLD + cL + kk + (lane >> 4)];
        const double fb = a[(C0 + (lane & 15)) * DLD + cL + kk + (lane >> 4)];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(fa, fb, acc, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rr = R0 + 4 * e + (lane >> 4), cc = C0 + (lane & 15);
        if (rr >= cmask && cc >= cmask) a[rr * DLD + cc] = acc[e];
    }
}

// 1 / sqrt(x) for positive x: the hardware estimate (v_rsq_f64, about 2^-24 relative)
// and one Newton step, y (3/2 - x y^2 / 2): about 2^-47.8 relative at worst over 4M
// arguments spanning 2^-40 .. 2^40 (measured); four dependent operations instead of
// the nine of the library routine, which also handles zero, infinity and NaN.
GPTQ_DEV double rsqrt_pos(double x) {
    const double y = __builtin_amdgcn_rsq(x);
    return y * fma(-0.5 * x * y, y, 1.5);
}

// The block is in a[] (lower part, identity padding past n).  All 256 threads of
// the workgroup call this.
//
// Look-ahead: the rank-8 update of round P is split into the 16-column tile strip
// holding the next sub-panel (done by all waves right after round P's factor step)
// and the tile columns right of it, which waves 2 and 3 apply while wave 0 factors
// round P + 1 (those columns are disjoint from the sub-panel being factored).  Every
// element receives the same updates in the same order as with whole-round updates.
// flag (may be null): once X_kk is stored it is published for other workgroups of
// the launch, before L_kk is stored; after a failed pivot it is published too (info
// then holds the failure).  X_kk is written with device-scope stores, which write
// through this XCD's L2, and read by the waiting workgroups with device-scope loads,
// which do not hit a stale line in theirs; every thread waits for its stores to
// complete before the barrier after which *flag = step is stored (device scope).  So
// no L2 write-back or invalidation is needed: a release fence at device scope would
// write back every dirty line of the L2, and an acquire fence would invalidate it for
// every workgroup sharing it (4% of the factorization at d = 4096 and 11008).
// v of lane l, in every lane (l a compile-time constant)
GPTQ_DEV double bcast_lane(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

GPTQ_DEV void publish_block(int* flag, int step) {
    if (flag == nullptr) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
GPTQ_DEV void store_dev(double* p, double v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
GPTQ_DEV double load_dev(const double* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

GPTQ_DEV void diag_block(double* a, double* xs, double* ts, int* fail_p, double* A, double* X, int64_t d,
                         int64_t k0, int n, int32_t* info, int* flag = nullptr, int step = 0) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int& fail_s = *fail_p;

    // eight rounds of 8 columns, unrolled (compile-time addresses and tile lists); a
    // failed pivot skips the remaining rounds
    static_for<0, PNB / 8>([&](auto P) {
        constexpr int c0 = decltype(P)::value * 8;
        if (fail_s) return;
        if (wave == 0) {
            // every lane solves its own row of the sub-panel, one column k at a time; the
            // top block's row k (lane c0 + k) supplies the pivot d_k (its own value at step
            // k) and the factor entries t[k][m] of the later steps, broadcast from that lane.
            // For the top block's rows this is the Cholesky of the 8 x 8 block with the same
            // operands in the same order; the entries right of a row's diagonal are never read
            const int r = lane;
            double x[8], rd[8], t[8][8];
            int f = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = a[r * DLD + c0 + k];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                double v = x[k];
#pragma unroll
                for (int m = 0; m < k; ++m) v = fma(-t[k][m], x[m], v);
                const double dk = bcast_lane(v, c0 + k);
                if (!(dk > 0.0) && f == 0) f = c0 + k + 1;
                rd[k] = rsqrt_pos(dk > 0.0 ? dk : 1.0);
                x[k] = v * rd[k];
#pragma unroll
                for (int i = k + 1; i < 8; ++i) t[i][k] = bcast_lane(x[k], c0 + i);
            }
            if (r >= c0) {
#pragma unroll
                for (int k = 0; k < 8; ++k) a[r * DLD + c0 + k] = x[k];
            }
            if constexpr (c0 == PNB - 8) {
                // the last sub-panel's 8 x 8 inverse, from the factor and reciprocal pivots
                // in registers (lane c < 8: column c); the earlier ones are formed by wave 1
                if (lane < 8) {
                    double y[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        double v = (i == lane) ? 1.0 : 0.0;
#pragma unroll
                        for (int k = 0; k < i; ++k) v -= t[i][k] * y[k];
                        y[i] = v * rd[i];
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) xs[(c0 + i) * DLD + c0 + lane] = (i >= lane) ? y[i] : 0.0;
                }
            }
            if (lane == 0 && f) fail_s = f;
        } else if constexpr (c0 == 0) {
            // meanwhile: the inverse starts as zero (the other three waves)
            for (int idx = tid - 64; idx < PNB * DLD; idx += 192) xs[idx] = 0.0;
        } else if (wave == 1) {
            // meanwhile: the inverse of the previous sub-panel's 8 x 8 diagonal block (its
            // divisions stay off the critical path of wave 0)
            if (lane < 8) diag_inv8(a, xs, c0 - 8, lane);
        } else {
            // meanwhile: the rest of the previous round's update, tile columns right of
            // the strip it updated (the strip holding column c0), on waves 2 and 3
            constexpr int tp = c0 >> 4;
            constexpr int nr = 3 - tp;                     // tile columns left to update
            constexpr int nrt = nr * (nr + 1) / 2;         // their lower tiles
            static_for<0, (nrt + 1) / 2>([&](auto R) {
                const int tt = (wave - 2) + 2 * decltype(R)::value;
                if (tt < nrt) {
                    int tc = tp + 1, rem = tt;
                    while (rem >= 4 - tc) { rem -= 4 - tc; ++tc; }
                    diag_upd_tile(a, (tc + rem) * 16, tc * 16, c0 - 8, c0, lane);
                }
            });
        }
        __syncthreads();
        if (fail_s) return;
        // this round's update of the strip holding the next sub-panel (columns c1 ..),
        // rows >= c1: at most four tiles, one per wave
        constexpr int c1 = c0 + 8;
        if constexpr (c1 < PNB) {
            constexpr int tn = c1 >> 4;
            if (wave < 4 - tn) diag_upd_tile(a, (tn + wave) * 16, tn * 16, c0, c1, lane);
        }
        __syncthreads();
    });
    if (fail_s) {
        if (tid == 0 && fail_s <= n && *info == 0) *info = (int32_t)(k0 + fail_s);
        publish_block(flag, step);
        return;
    }
    // X_kk = L_kk^-1: the inverses of the eight 8 x 8 diagonal blocks were formed during
    // the rounds; recursive doubling X[q][p] = -X[q][q] (L[q][p] X[p][p]) for block
    // sizes 8, 16, 32
    for (int b = 8; b < PNB; b *= 2) {
        const int np = PNB / (2 * b);
        if (b == 8) {
            // 8 x 8 products: one output element per thread
            for (int idx = tid; idx < np * 64; idx += 256) {
                const int m = idx >> 6, rr = (idx >> 3) & 7, cc = idx & 7, p0 = 16 * m, q0 = p0 + 8;
                double acc = 0.0;
#pragma unroll
                for (int k = 0; k < 8; ++k) acc += a[(q0 + rr) * DLD + p0 + k] * xs[(p0 + k) * DLD + p0 + cc];
                ts[idx] = acc;
            }
            // pair m = idx / 64 = wave: the same wave reads its T (LDS is in order per wave)
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            for (int idx = tid; idx < np * 64; idx += 256) {
                const int m = idx >> 6, rr = (idx >> 3) & 7, cc = idx & 7, p0 = 16 * m, q0 = p0 + 8;
                double acc = 0.0;
#pragma unroll
                for (int k = 0; k < 8; ++k) acc += xs[(q0 + rr) * DLD + q0 + k] * ts[m * 64 + k * 8 + cc];
                xs[(q0 + rr) * DLD + p0 + cc] = -acc;
            }
            __syncthreads();
        } else {
            // b = 16, 32: 16 x 16 output tiles on MFMA, one tile per wave at a time
            const int tpb = b / 16, ntile = np * tpb * tpb;
            for (int t = wave; t < ntile; t += 4) {           // T_m = L[q][p] X[p][p]
                const int m = t / (tpb * tpb), ti = (t / tpb) % tpb, tj = t % tpb;
                const int p0 = 2 * m * b, q0 = p0 + b;
                f64x4_t acc = f64x4_t{0.0, 0.0, 0.0, 0.0};
                for (int k = 0; k < b; k += 4) {
                    const double fa = a[(q0 + ti * 16 + (lane & 15)) * DLD + p0 + k + (lane >> 4)];
                    const double fb = xs[(p0 + k + (lane >> 4)) * DLD + p0 + tj * 16 + (lane & 15)];
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(fa, fb, acc, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ts[(m * b + ti * 16 + 4 * e + (lane >> 4)) * 32 + tj * 16 + (lane & 15)] = acc[e];
            }
            // b = 16: one tile per pair, the same wave reads it; b = 32: tiles are shared
            if (tpb == 1) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            else __syncthreads();
            for (int t = wave; t < ntile; t += 4) {           // X[q][p] = -X[q][q] T_m
                const int m = t / (tpb * tpb), ti = (t / tpb) % tpb, tj = t % tpb;
                const int p0 = 2 * m * b, q0 = p0 + b;
                f64x4_t acc = f64x4_t{0.0, 0.0, 0.0, 0.0};
                for (int k = 0; k < b; k += 4) {
                    const double fa = -xs[(q0 + ti * 16 + (lane & 15)) * DLD + q0 + k + (lane >> 4)];
                    const double fb = ts[(m * b + k + (lane >> 4)) * 32 + tj * 16 + (lane & 15)];
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(fa, fb, acc, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xs[(q0 + ti * 16 + 4 * e + (lane >> 4)) * DLD + p0 + tj * 16 + (lane & 15)] = acc[e];
            }
            __syncthreads();
        }
    }
    // X_kk first (the workgroups waiting for this block read only X_kk), published, then
    // L_kk; 16-byte stores of whole rows (32 threads per row) for a full block.  The
    // strictly upper part of L's block is written as 0 (it is never read).
    const bool vec = n == PNB && (d & 1) == 0;
    if (vec) {
        double2 vx[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = (tid >> 5) + 8 * q, c = 2 * (tid & 31);
            vx[q] = double2{xs[r * DLD + c], xs[r * DLD + c + 1]};
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = (tid >> 5) + 8 * q, c = 2 * (tid & 31);
            store_dev(X + (k0 + r) * d + k0 + c, vx[q].x);
            store_dev(X + (k0 + r) * d + k0 + c + 1, vx[q].y);
        }
    } else {
        for (int idx = tid; idx < n * n; idx += 256) {
            const int r = idx / n, c = idx % n;
            store_dev(X + (k0 + r) * d + k0 + c, xs[r * DLD + c]);
        }
    }
    publish_block(flag, step);
    if (vec) {
        double2 vl[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = (tid >> 5) + 8 * q, c = 2 * (tid & 31);
            vl[q] = double2{c <= r ? a[r * DLD + c] : 0.0, c + 1 <= r ? a[r * DLD + c + 1] : 0.0};
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = (tid >> 5) + 8 * q, c = 2 * (tid & 31);
            *reinterpret_cast<double2*>(A + (k0 + r) * d + k0 + c) = vl[q];
        }
    } else {
        for (int idx = tid; idx < n * n; idx += 256) {
            const int r = idx / n, c = idx % n;
            if (c <= r) A[(k0 + r) * d + k0 + c] = a[r * DLD + c];
        }
    }
}

// Load the lower part of diagonal block k (identity padding past n) into a[].
GPTQ_DEV void diag_load(double* a, const double* A, int64_t d, int64_t k0, int n) {
    constexpr int NV = PNB * PNB / 256;
    double v[NV];
#pragma unroll
    for (int t = 0; t < NV; ++t) {            // all loads first
        const int idx = threadIdx.x + 256 * t;
        const int i = idx >> 6, k = idx & 63;
        // unconditional load from a clamped (in-bounds) address, then the selection
        const double x = A[(k0 + (i < n ? i : n - 1)) * d + k0 + (k < n ? k : n - 1)];
        v[t] = (i < n && k <= i) ? x : ((i == k) ? 1.0 : 0.0);
    }
#pragma unroll
    for (int t = 0; t < NV; ++t) {
        const int idx = threadIdx.x + 256 * t;
        a[(idx >> 6) * DLD + (idx & 63)] = v[t];
    }
}

// Diagonal block 0 on its own (every later block is factored inside the trailing
// update of the step before it).
__global__ __launch_bounds__(256) void prep_diag_kernel(double* A, double* X, int64_t d, int64_t k0, int n,
                                                      int32_t* info) {
    __shared__ double lds[DIAG_LDS_DOUBLES];
    __shared__ int fail_s;
    if (threadIdx.x == 0) fail_s = 0;
    diag_load(lds, A, d, k0, n);
    __syncthreads();
    diag_block(lds, lds + PNB * DLD, lds + 2 * PNB * DLD, &fail_s, A, X, d, k0, n, info);
}

// Panel: L[k0+64:, k0:k0+64] = A[k0+64:, k0:k0+64] X_kk^T, in place (each workgroup
// reads its 64 rows completely before writing them).  fp64 MFMA 16x16x4.
__global__ __launch_bounds__(256) void prep_panel_kernel(double* A, const double* X, int64_t d, int64_t k0) {
    __shared__ double As[64 * DLD];
    __shared__ double Xs[64 * DLD];
    const int64_t r0 = k0 + PNB + (int64_t)blockIdx.x * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    // all loads of a thread first, then the LDS stores
    constexpr int PV = 64 * PNB / 2 / 256;      // double2 per thread and operand
    double2 va[PV], vx[PV];
#pragma unroll
    for (int v = 0; v < PV; ++v) {
        const int idx = tid + 256 * v;
        const int i = idx / (PNB / 2), k = 2 * (idx % (PNB / 2));
        va[v] = (r0 + i < d) ? *reinterpret_cast<const double2*>(A + (r0 + i) * d + k0 + k) : double2{0.0, 0.0};
        vx[v] = *reinterpret_cast<const double2*>(X + (k0 + i) * d + k0 + k);
    }
#pragma unroll
    for (int v = 0; v < PV; ++v) {
        const int idx = tid + 256 * v;
        const int i = idx / (PNB / 2), k = 2 * (idx % (PNB / 2));
        As[i * DLD + k] = va[v].x; As[i * DLD + k + 1] = va[v].y;
        Xs[i * DLD + k] = vx[v].x; Xs[i * DLD + k + 1] = vx[v].y;
    }
    __syncthreads();
    f64x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{};
#pragma unroll 4
    for (int kk = 0; kk < PNB; kk += 4) {
        double fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = As[(wr * 32 + i * 16 + (lane & 15)) * DLD + kk + (lane >> 4)];
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = Xs[(wc * 32 + j * 16 + (lane & 15)) * DLD + kk + (lane >> 4)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t gr = r0 + wr * 32 + i * 16 + 4 * e + (lane >> 4);
                const int c = wc * 32 + j * 16 + (lane & 15);
                if (gr < d) A[gr * d + k0 + c] = acc[i][j][e];
            }
}

// --------------------------------------------------------------------------
// fp64 GEMM on MFMA: C = beta C + alpha A op(B), 64 x 64 tiles, 4 waves (2 x 2 of 32 x 32).
enum : int { G_BT = 1, G_TRI_A = 2, G_TRI_B = 4, G_LOWER_C = 8, G_DIAG0 = 16, G_PANEL1 = 32 };
constexpr int GD_BM = 64, GD_BK = 32, GD_LD = GD_BK + 1;

struct GemmD {
    double* C; int64_t ldc;
    const double* A; int64_t lda;
    const double* B; int64_t ldb;
    int M, N, K;
    double alpha, beta;
    int flags;
    // batching over blockIdx.z: operand offsets advance by these element strides;
    // the last batch entry may have fewer rows (M_last) and, for G_TRI_A, fewer k (= M_last)
    int64_t sA, sB, sC; int M_last; int nbatch;
    // G_DIAG0: tile (0, 0) of C is the next diagonal block (rows / columns k1 ..
    // k1 + n1 of the factored matrix fA, inverse blocks in fX); its workgroup
    // factors it after the update instead of storing it
    double* fA; double* fX; int64_t fd, k1; int n1; int32_t* info;
    int ntm, ntn;   // tiles along M (of a full batch entry) and N
    // G_PANEL1: the tiles of block column 0 below tile (0, 0) are the next panel; their
    // workgroups multiply the updated tile by the transposed inverse of the next
    // diagonal block once the G_DIAG0 workgroup has published it (*flag >= step)
    int* flag; int step;
    int wait_polls;   // bound of that wait (0: give up at once)
    // capped grid (0: one workgroup per tile): vtiles = tiles per batch entry (tpb) x
    // entries, taken by the workgroups in turn
    int vtiles, tpb;
};

// Operand chunk of GD_BK columns of k: 64 rows (m or n) x 32 k, as 4 double2 per thread.
template <bool KMAJOR>
GPTQ_DEV void gd_load(const double* P, int64_t ld, int rows, int r0, int kc, int ke, int tid, double2 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;            // 1024 double2 slots
        double2 x = double2{0.0, 0.0};
        if constexpr (!KMAJOR) {
            // P[r][k] row-major with k contiguous: 16 double2 per row of 32 k
            const int r = idx >> 4, k = kc + 2 * (idx & 15);
            if (r0 + r < rows) {
                const double* src = P + (int64_t)(r0 + r) * ld + k;
                if (k + 1 < ke) x = *reinterpret_cast<const double2*>(src);
                else if (k < ke) x.x = src[0];
            }
        } else {
            // P[k][n] row-major with n contiguous: 32 double2 per k row of 64 n
            const int k = kc + (idx >> 5), r = 2 * (idx & 31);
            if (k < ke) {
                const double* src = P + (int64_t)k * ld + r0 + r;
                if (r0 + r + 1 < rows) x = *reinterpret_cast<const double2*>(src);
                else if (r0 + r < rows) x.x = src[0];
            }
        }
        v[i] = x;
    }
}

template <bool KMAJOR>
GPTQ_DEV void gd_store(double* S, int tid, const double2 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;
        if constexpr (!KMAJOR) {
            const int r = idx >> 4, k = 2 * (idx & 15);
            S[r * GD_LD + k] = v[i].x;
            S[r * GD_LD + k + 1] = v[i].y;
        } else {
            const int k = idx >> 5, r = 2 * (idx & 31);
            S[r * GD_LD + k] = v[i].x;
            S[(r + 1) * GD_LD + k] = v[i].y;
        }
    }
}

constexpr int GD_TILE = GD_BM * GD_LD;
constexpr int GD_LDS = (4 * GD_TILE > DIAG_LDS_DOUBLES) ? 4 * GD_TILE : DIAG_LDS_DOUBLES;

// --------------------------------------------------------------------------
// Direct global -> LDS operand ring for whole 64 x 64 tiles of C += A op(B) with the k
// range a multiple of 16: four stages of 16 k (16 KB each), filled by
// global_load_lds_dwordx4 three stages ahead; no register staging and one barrier per
// stage.  A is row-major (k contiguous), stored [64 rows][16 k] with the 16-byte chunk c
// of row r at chunk position c ^ ((r / 2) % 8); B is either the same (op = transpose,
// B given as rows n) or k-major (B[k][n], n contiguous), stored [16 k][64 n] with chunk
// c of k row k at position c ^ 8 (k % 2).  Either way the MFMA operand reads (16 rows or
// columns at 2 consecutive k per half-wave) hit distinct banks.  The MFMAs and their
// order are those of the register-staged loop (4 k per MFMA, k increasing), so the
// result is the same bit for bit.
constexpr int GX_BK = 16, GX_NST = 4, GX_DMA = 4;          // k per stage, stages, loads per wave and stage
constexpr int GX_OP = GD_BM * GX_BK;                       // doubles of one operand in a stage
constexpr int GX_ST = 2 * GX_OP;                           // doubles of a stage
constexpr int GX_VM = (GX_NST - 2) * GX_DMA;               // loads left in flight at a stage wait
static_assert(GX_NST * GX_ST <= GD_LDS && GX_NST * GX_ST <= 4 * GD_BM * GD_LD,
              "the operand ring fits in both kernels' LDS");

GPTQ_DEV int gx_swz(int r) { return (r >> 1) & 7; }        // row-major operands
GPTQ_DEV int gx_swzk(int k) { return (k & 1) << 3; }       // k-major B

struct GxCopy {
    uint32_t voff[GX_DMA];     // per-lane byte offsets (from the operand's origin at k = kb)
    const double* abase;       // A row m0 at k = kb; B row n0 at k = kb, or B row kb at column n0
    const double* bbase;
    int64_t bstage;            // doubles between B's stages
    uint32_t m0base;           // LDS byte address of the wave's share of slot 0
};

// wave w, loads 0 and 1: A rows 8 (2 w + i) .. + 7, lane l row + l / 8, chunk position
// l % 8.  Loads 2 and 3: B the same (transposed), or k-major: k rows 2 (2 w + i - 2) .. + 1,
// lane l k row + l / 32, chunk position l % 32.
template <bool BKMAJOR>
GPTQ_DEV GxCopy gx_setup(const GemmD& g, int m0, int n0, int kb, int wave, int lane, const double* ring) {
    GxCopy x;
    const int w = __builtin_amdgcn_readfirstlane(wave);
    x.abase = g.A + (int64_t)m0 * g.lda + kb;
    x.bbase = BKMAJOR ? g.B + (int64_t)kb * g.ldb + n0 : g.B + (int64_t)n0 * g.ldb + kb;
    x.bstage = BKMAJOR ? (int64_t)GX_BK * g.ldb : GX_BK;
    x.m0base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) double*)ring + (uint32_t)(w * 2048);
#pragma unroll
    for (int i = 0; i < GX_DMA; ++i) {
        if (i < 2 || !BKMAJOR) {
            const int r = 8 * (2 * w + (i & 1)) + (lane >> 3);
            const int c = (lane & 7) ^ gx_swz(r);
            const int64_t ld = (i >> 1) ? g.ldb : g.lda;
            x.voff[i] = (uint32_t)(((int64_t)r * ld + 2 * c) * 8);
        } else {
            const int k = 2 * (2 * w + (i & 1)) + (lane >> 5);
            const int c = (lane & 31) ^ gx_swzk(k);
            x.voff[i] = (uint32_t)(((int64_t)k * g.ldb + 2 * c) * 8);
        }
    }
    return x;
}

template <int SLOT>
GPTQ_DEV void gx_issue(const GxCopy& x, int st) {
    const double* a = x.abase + st * GX_BK;
    const double* b = x.bbase + st * x.bstage;
    dma16<(uint32_t)(SLOT * GX_ST * 8 + 0)>(x.voff[0], a, x.m0base);
    dma16<(uint32_t)(SLOT * GX_ST * 8 + 1024)>(x.voff[1], a, x.m0base);
    dma16<(uint32_t)(SLOT * GX_ST * 8 + GX_OP * 8)>(x.voff[2], b, x.m0base);
    dma16<(uint32_t)(SLOT * GX_ST * 8 + GX_OP * 8 + 1024)>(x.voff[3], b, x.m0base);
}

struct GxFrags { double a[4][2], b[4][2]; };   // [k step][i or j]

template <bool BKMAJOR>
GPTQ_DEV void gx_read(const double* stg, int wr, int wc, int lane, GxFrags& f) {
#pragma unroll
    for (int s = 0; s < GX_BK / 4; ++s) {
        const int k = 4 * s + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = wr * 32 + i * 16 + (lane & 15);
            f.a[s][i] = stg[r * GX_BK + 2 * ((k >> 1) ^ gx_swz(r)) + (k & 1)];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = wc * 32 + j * 16 + (lane & 15);
            if constexpr (BKMAJOR)
                f.b[s][j] = stg[GX_OP + k * GD_BM + 2 * ((r >> 1) ^ gx_swzk(k)) + (r & 1)];
            else
                f.b[s][j] = stg[GX_OP + r * GX_BK + 2 * ((k >> 1) ^ gx_swz(r)) + (k & 1)];
        }
    }
}

GPTQ_DEV void gx_mfma(const GxFrags& f, f64x4_t (&acc)[2][2]) {
#pragma unroll
    for (int s = 0; s < GX_BK / 4; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(f.a[s][i], f.b[s][j], acc[i][j], 0, 0, 0);
}

// acc += A[m0 .. + 63][kb .. ke) op(B)[kb .. ke)[n0 .. + 63] through the ring
template <bool BKMAJOR>
GPTQ_DEV void gx_tile(const GemmD& g, int m0, int n0, int kb, int ke, double* lds, f64x4_t (&acc)[2][2]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int nst = (ke - kb) / GX_BK;
    // loads of stages past the last re-load the last one (addresses stay inside the
    // operands), so that every step leaves the same number of loads in flight
    auto t0 = [&](int st) { return st < nst ? st : nst - 1; };
    const GxCopy x = gx_setup<BKMAJOR>(g, m0, n0, kb, wave, lane, lds);
    static_for<0, GX_NST - 1>([&](auto I) { gx_issue<decltype(I)::value>(x, t0(decltype(I)::value)); });
    wait_vm_lgkm0<GX_VM>();
    __syncthreads();
    gx_issue<GX_NST - 1>(x, t0(GX_NST - 1));
    GxFrags f0, f1;
    gx_read<BKMAJOR>(lds, wr, wc, lane, f0);
    for (int st = 0; st < nst; st += GX_NST) {
        static_for<0, GX_NST>([&](auto U) {
            constexpr int u = decltype(U)::value;
            if (st + u < nst) {
                // stage st + u + 1 has landed and every wave is done with slot u
                wait_vm_lgkm0<GX_VM>();
                __syncthreads();
                gx_issue<u>(x, t0(st + u + GX_NST));
                GxFrags& cur = (u & 1) ? f1 : f0;
                GxFrags& nxt = (u & 1) ? f0 : f1;
                gx_read<BKMAJOR>(lds + ((u + 1) % GX_NST) * GX_ST, wr, wc, lane, nxt);
                gx_mfma(cur, acc);
            }
        });
    }
    __builtin_amdgcn_s_waitcnt(0);   // the trailing re-loads land before the ring is reused
    __syncthreads();
}

// One output tile (bid within batch entry bz).  lds: the operand double buffers, and
// the diagonal routine's buffers in the G_DIAG0 workgroup.  FUSED: the G_DIAG0 /
// G_PANEL1 paths are compiled in.
template <bool BKMAJOR, bool FUSED>
GPTQ_DEV void gemm_f64_tile(GemmD g, const int bid, const int bz, double* lds, int& fail_s) {
    auto As = [&](int b) { return lds + b * GD_TILE; };
    auto Bs = [&](int b) { return lds + (2 + b) * GD_TILE; };
    if (bz > 0) {
        g.A += bz * g.sA; g.B += bz * g.sB; g.C += bz * g.sC;
        if (bz == g.nbatch - 1) {
            if (g.flags & G_TRI_A) g.K = g.M_last;
            g.M = g.M_last;
        }
    } else if (g.nbatch == 1 && g.M_last > 0) {
        if (g.flags & G_TRI_A) g.K = g.M_last;
        g.M = g.M_last;
    }
    // tile order of the 1-D grid: longest k ranges first where they differ (a lower-
    // triangular operand), so the long tiles do not finish last; only the lower tiles
    // of a lower-triangular C are enumerated
    int mi, nj;
    auto tri = [](int t, int& r, int& c) {   // t-th entry of a lower triangle, row-major
        r = (int)((sqrtf(8.f * t + 1.f) - 1.f) * 0.5f);
        while ((r + 1) * (r + 2) / 2 <= t) ++r;
        while (r * (r + 1) / 2 > t) --r;
        c = t - r * (r + 1) / 2;
    };
    // t-th tile of the lower trapezoid {(mi, nj): nj <= mi < ntm, nj < w}, row-major: a
    // triangle of w rows, then rows of w tiles
    auto trap = [&](int t, int w, int& r, int& c) {
        const int tt = w * (w + 1) / 2;
        if (t < tt) tri(t, r, c);
        else { r = w + (t - tt) / w; c = (t - tt) % w; }
    };
    if (g.flags & G_PANEL1) {
        // tile (0, 0) first (the next diagonal block), then the tiles right of block
        // column 0, then block column 0 (the next panel, which waits for the block): in
        // a large update those workgroups start after the block is published
        const int w = g.ntn - 1;
        const int inner = (g.ntm <= g.ntn) ? (g.ntm - 1) * g.ntm / 2 : w * (w + 1) / 2 + (g.ntm - 1 - w) * w;
        if (bid == 0) { mi = 0; nj = 0; }
        else if (bid <= inner) { trap(bid - 1, w, mi, nj); ++mi; ++nj; }
        else { mi = bid - inner; nj = 0; }
    } else if (g.flags & G_LOWER_C) {
        trap(bid, g.ntn, mi, nj);
    } else if (g.flags & G_TRI_B) {          // k >= n0 (B lower) or k < n0 + 64 (B^T lower)
        const int q = bid / g.ntm;
        nj = (g.flags & G_BT) ? g.ntn - 1 - q : q;
        mi = bid % g.ntm;
    } else if (g.flags & G_TRI_A) {          // k < m0 + 64
        mi = g.ntm - 1 - bid / g.ntn;
        nj = bid % g.ntn;
    } else {
        mi = bid / g.ntn;
        nj = bid % g.ntn;
    }
    const int m0 = mi * GD_BM, n0 = nj * GD_BM;
    const bool diag0 = FUSED && (g.flags & G_DIAG0) && mi == 0 && nj == 0 && bz == 0;
    if (m0 >= g.M) return;
    // the next diagonal block heads the factorization chain: its waves take issue
    // priority over the update tiles that share their compute unit
    if (diag0) __builtin_amdgcn_s_setprio(3);
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

    const bool full = (m0 + GD_BM <= g.M) && (n0 + GD_BM <= g.N);
    const bool panel = FUSED && (g.flags & G_PANEL1) && nj == 0 && mi > 0 && bz == 0;
    // v_mfma_f64_16x16x4_f64 result layout: element e of lane l is row 4 e + l / 16
    double* cbase = g.C + (int64_t)(m0 + wr * 32 + (lane >> 4)) * g.ldc + n0 + wc * 32 + (lane & 15);
    auto off = [&](int i, int j, int e) { return (int64_t)(i * 16 + 4 * e) * g.ldc + j * 16; };
    // C of a whole tile, loaded after the products (loading it before them measured
    // slower: it competes with the operand loads of the first chunks), except for the
    // next diagonal block, whose load latency would add to the chain
    double cold[2][2][4];
    const bool pre = full && g.beta != 0.0;
    auto load_c = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) cold[i][j][e] = cbase[off(i, j, e)];
    };
    if (pre && diag0) load_c();

#ifndef GD_DMA
#define GD_DMA 1
#endif
    // whole tiles (even row pitches, 16-byte aligned operands, k range a multiple of 16)
    // take the direct-load ring
#ifndef GD_DMA_CHAIN
#define GD_DMA_CHAIN 1
#endif
    const bool dma = GD_DMA && full && (GD_DMA_CHAIN || (!diag0 && !panel)) && ke > kb && ((ke - kb) % GX_BK) == 0 &&
                     ((g.lda | g.ldb) & 1) == 0 &&
                     ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B)) & 15) == 0;
    if (dma) gx_tile<BKMAJOR>(g, m0, n0, kb, ke, lds, acc);
    const int nch = (!dma && ke > kb) ? (ke - kb + GD_BK - 1) / GD_BK : 0;
    double2 va[4], vb[4];
    if (nch > 0) {
        gd_load<false>(g.A, g.lda, g.M, m0, kb, ke, tid, va);
        gd_load<BKMAJOR>(g.B, g.ldb, g.N, n0, kb, ke, tid, vb);
        gd_store<false>(As(0), tid, va);
        gd_store<BKMAJOR>(Bs(0), tid, vb);
        if (nch > 1) {
            gd_load<false>(g.A, g.lda, g.M, m0, kb + GD_BK, ke, tid, va);
            gd_load<BKMAJOR>(g.B, g.ldb, g.N, n0, kb + GD_BK, ke, tid, vb);
        }
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const double* as = As(c & 1);
        const double* bs = Bs(c & 1);
#pragma unroll
        for (int kk = 0; kk < GD_BK; kk += 4) {
            double fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = as[(wr * 32 + i * 16 + (lane & 15)) * GD_LD + kk + (lane >> 4)];
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = bs[(wc * 32 + j * 16 + (lane & 15)) * GD_LD + kk + (lane >> 4)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (c + 1 < nch) {
            gd_store<false>(As((c + 1) & 1), tid, va);
            gd_store<BKMAJOR>(Bs((c + 1) & 1), tid, vb);
        }
        if (c + 2 < nch) {
            gd_load<false>(g.A, g.lda, g.M, m0, kb + (c + 2) * GD_BK, ke, tid, va);
            gd_load<BKMAJOR>(g.B, g.ldb, g.N, n0, kb + (c + 2) * GD_BK, ke, tid, vb);
        }
        __syncthreads();
    }
    if (pre && !diag0) load_c();
    if constexpr (FUSED) if (diag0) {
        // updated diagonal block -> a[] (lower part; upper 0, identity padding), factor
        double* a = lds;
        if (tid == 0) fail_s = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = wr * 32 + i * 16 + 4 * e + (lane >> 4);
                    const int cc = wc * 32 + j * 16 + (lane & 15);
                    double v = (r == cc) ? 1.0 : 0.0;
                    if (r < g.n1 && cc <= r) {
                        const double c = pre ? cold[i][j][e] : g.C[(int64_t)r * g.ldc + cc];
                        v = g.beta * c + g.alpha * acc[i][j][e];
                    }
                    a[r * DLD + cc] = v;
                }
        __syncthreads();
        // the routine publishes the block's inverse to the panel workgroups (also after a
        // failed pivot, so that none waits in vain; info then holds the failure)
        diag_block(a, a + PNB * DLD, a + 2 * PNB * DLD, &fail_s, g.fA, g.fX, g.fd, g.k1, g.n1, g.info,
                   (g.flags & G_PANEL1) ? g.flag : nullptr, g.step);
        return;
    }
    if constexpr (FUSED) if (panel) {
        // updated tile (rows past M as zeros) -> LDS; the operand buffers are free after
        // the last barrier of the product loop
        double* pa = lds;
        double* px = lds + PNB * DLD;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = wr * 32 + i * 16 + 4 * e + (lane >> 4);
                    const int cc = wc * 32 + j * 16 + (lane & 15);
                    double v = 0.0;
                    if (m0 + r < g.M) {
                        const double c = pre ? cold[i][j][e] : g.C[(int64_t)(m0 + r) * g.ldc + cc];
                        v = g.beta * c + g.alpha * acc[i][j][e];
                    }
                    pa[r * DLD + cc] = v;
                }
        // wait (at most wait_polls polls of about 128 clocks) until the inverse of the next
        // diagonal block is published
        if (tid == 0) {
            for (int polls = 0;; ++polls) {
                if (polls >= g.wait_polls) {
                    atomicCAS(g.info, 0, -2);
                    break;
                }
                if (__hip_atomic_load(g.flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= g.step) break;
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
        __builtin_amdgcn_s_setprio(2);   // from here the panel is on the chain
        constexpr int PV = 64 * PNB / 2 / 256;      // double2 per thread
        double2 vx[PV];
#pragma unroll
        for (int v = 0; v < PV; ++v) {
            const int idx = tid + 256 * v;
            const int i = idx / (PNB / 2), k = 2 * (idx % (PNB / 2));
            const double* xp = g.fX + (g.k1 + i) * g.fd + g.k1 + k;   // device-scope loads (see publish_block)
            vx[v] = double2{load_dev(xp), load_dev(xp + 1)};
        }
#pragma unroll
        for (int v = 0; v < PV; ++v) {
            const int idx = tid + 256 * v;
            const int i = idx / (PNB / 2), k = 2 * (idx % (PNB / 2));
            px[i * DLD + k] = vx[v].x; px[i * DLD + k + 1] = vx[v].y;
        }
        __syncthreads();
        // L[rows][k1 : k1 + 64] = (updated tile) X_kk^T, in the panel kernel's order
        f64x4_t pacc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) pacc[i][j] = f64x4_t{};
#pragma unroll 4
        for (int kk = 0; kk < PNB; kk += 4) {
            double fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = pa[(wr * 32 + i * 16 + (lane & 15)) * DLD + kk + (lane >> 4)];
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = px[(wc * 32 + j * 16 + (lane & 15)) * DLD + kk + (lane >> 4)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    pacc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb[j], pacc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = wr * 32 + i * 16 + 4 * e + (lane >> 4);
                    if (m0 + r < g.M) cbase[off(i, j, e)] = pacc[i][j][e];
                }
        return;
    }
    // C = beta C + alpha acc: all loads of C first (above), then all stores (a load
    // after a store to the same array would otherwise wait for that store's round trip)
    if (full) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double v = g.alpha * acc[i][j][e];
                    cbase[off(i, j, e)] = pre ? g.beta * cold[i][j][e] + v : v;
                }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int gm = m0 + wr * 32 + i * 16 + 4 * e + (lane >> 4);
                    const int gn = n0 + wc * 32 + j * 16 + (lane & 15);
                    if (gm < g.M && gn < g.N) {
                        double* c = g.C + (int64_t)gm * g.ldc + gn;
                        const double v = g.alpha * acc[i][j][e];
                        *c = (g.beta == 0.0) ? v : g.beta * *c + v;
                    }
                }
    }
}

template <bool BKMAJOR>
__global__ __launch_bounds__(256) void gemm_f64_kernel(GemmD g) {
    __shared__ __align__(16) double lds[GD_LDS];
    __shared__ int fail_s;
    gemm_f64_tile<BKMAJOR, true>(g, blockIdx.x, blockIdx.z, lds, fail_s);
}

// Capped grid: workgroup w takes the tiles w, w + gridDim.x, ... (batch-major); no
// G_DIAG0 / G_PANEL1 work.
template <bool BKMAJOR>
__global__ __launch_bounds__(256) void gemm_f64_capped_kernel(GemmD g) {
    __shared__ __align__(16) double lds[4 * GD_TILE];
    __shared__ int fail_s;
    for (int vt = blockIdx.x; vt < g.vtiles; vt += gridDim.x) {
        __syncthreads();   // the previous tile's last LDS reads are done
        gemm_f64_tile<BKMAJOR, false>(g, vt % g.tpb, vt / g.tpb, lds, fail_s);
    }
}

// --------------------------------------------------------------------------
// Host side
struct PrepCtx {
    double* A; double* X; double* T; int64_t d;
    int32_t* info; int* flag; hipStream_t s;
    int32_t wait_polls;
};

static gptq_status gemm(PrepCtx& c, double* C, int64_t ldc, const double* A, int64_t lda, const double* B,
                        int64_t ldb, int M, int N, int K, double alpha, double beta, int flags,
                        int nbatch = 1, int64_t sA = 0, int64_t sB = 0, int64_t sC = 0, int M_last = 0,
                        int64_t k1 = 0, int n1 = 0, int step = 0, int max_wg = 0) {
    if (M <= 0 || N <= 0 || nbatch <= 0) return GPTQ_OK;
    const int ntm = (M + GD_BM - 1) / GD_BM, ntn = (N + GD_BM - 1) / GD_BM;
    GemmD g{C, ldc, A, lda, B, ldb, M, N, K, alpha, beta, flags, sA, sB, sC, M_last, nbatch,
            c.A, c.X, c.d, k1, n1, c.info, ntm, ntn, c.flag, step, c.wait_polls, 0, 0};
    // a lower-triangular C: the tiles on and below the diagonal of an M x N block, N <= M
    // (a trapezoid when N < M)
    if ((flags & G_LOWER_C) && N > M) return GPTQ_ERR_INVALID_ARG;
    const int ntiles = (flags & G_LOWER_C) ? ntn * (ntn + 1) / 2 + (ntm - ntn) * ntn : ntm * ntn;
    dim3 grid((unsigned)ntiles, 1, nbatch);
    if (max_wg > 0 && (int64_t)ntiles * nbatch > max_wg && !(flags & (G_DIAG0 | G_PANEL1))) {
        g.vtiles = ntiles * nbatch;
        g.tpb = ntiles;
        if (flags & G_BT) gemm_f64_capped_kernel<false><<<max_wg, 256, 0, c.s>>>(g);
        else gemm_f64_capped_kernel<true><<<max_wg, 256, 0, c.s>>>(g);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    if (flags & G_BT) gemm_f64_kernel<false><<<grid, 256, 0, c.s>>>(g);
    else gemm_f64_kernel<true><<<grid, 256, 0, c.s>>>(g);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

// X = L^-1 on the diagonal block [off, off + m) by recursive doubling of the inverted
// 64 x 64 diagonal blocks over independent block pairs, X[q][p] = -X[q][q] (L[q][p]
// X[p][p]), block sizes 64, 128, .. < m, each level two batched products; T is
// scratch for the products (at most m * m doubles).
static gptq_status trtri_block(PrepCtx& c, int64_t off, int64_t m, double* T, int max_wg = 0) {
    const int64_t d = c.d;
    gptq_status st;
    for (int64_t b = PNB; b < m; b *= 2) {
        // pairs p = off + [2 j b, (2 j + 1) b), q = off + [(2 j + 1) b, min((2 j + 2) b, m))
        const int64_t npairs = (m - b + 2 * b - 1) / (2 * b);
        const int64_t q_last = (2 * (npairs - 1) + 1) * b;
        const int qn_last = (int)std::min<int64_t>(b, m - q_last);
        const int64_t step = 2 * b * (d + 1);
        const int bb = (int)b;
        double* Ab = c.A + (off + b) * d + off;       // L[q][p] of the first pair
        double* Xp = c.X + off * d + off;             // X[p][p]
        double* Xq = c.X + (off + b) * d + off;       // X[q][p]
        // T_j = L[q][p] X[p][p]   (b x b each, X[p][p] lower triangular)
        if ((st = gemm(c, T, bb, Ab, d, Xp, d, bb, bb, bb, 1.0, 0.0, G_TRI_B,
                       (int)npairs, step, step, (int64_t)b * b, qn_last, 0, 0, 0, max_wg)) != GPTQ_OK) return st;
        // X[q][p] = -X[q][q] T_j   (X[q][q] lower triangular)
        if ((st = gemm(c, Xq, d, Xq + b, d, T, bb, bb, bb, bb, -1.0, 0.0, G_TRI_A,
                       (int)npairs, step, (int64_t)b * b, step, qn_last, 0, 0, 0, max_wg)) != GPTQ_OK) return st;
    }
    return GPTQ_OK;
}

// The auxiliary work starts once the trailing matrix is down to AUX_FORK_REST columns
// (or later, when the leading block is final only then), and its products take at
// most AUX_MAX_WG workgroups at a time, so that the factorization steps beside it
// still find free slots.
#ifndef AUX_MAX_WG
#define AUX_MAX_WG 384
#endif

// Right-looking blocked Cholesky of A (lower, reversed damped H) with the inverse of
// every 64 x 64 diagonal block of L, then X = L^-1.
// Block 0 and its panel have launches of their own; every later diagonal block and
// its panel are finished inside the trailing update of the step before (tile (0, 0)
// factors the block, the tiles below it apply its inverse), so each step of the
// chain is one launch.  From d = DEFER_MIN_D on, the trailing update is deferred to
// outer blocks of W columns (DEFER_W_SMALL below DEFER_W_MIN_D, else DEFER_W): each
// step inside an outer block updates only the rest of that block (its columns, all rows
// below), and the step of the block's last panel applies the block's W columns to the
// whole matrix after it (one product with K = W, whose tile (0, 0) and block column 0
// again form the next block and panel).  Every element receives the same products,
// grouped differently.  (At d = 4096 this measured no faster: the chain, not the matrix
// traffic, bounds the time there, and the K = W update lies on it.)
//
// The inverse is assembled by row blocks B_0, B_1, .., B_last: B_0 = [0, h) with h
// the largest 64 * 2^i below d, and each next block the largest 64 * 2^i below what
// remains, until at most INV_LAST columns are left (the last block).  With P_i =
// [0, s_i) the columns before B_i and Trest[r][P_i] = L[r][P_i] X[P_i][P_i] for the
// rows r after B_{i-1}:
//   X[B_i][P_i] = -X[B_i][B_i] Trest[B_i][P_i],
//   Trest[r][P_i] += L[r][B_i] X[B_i][P_i] and Trest[r][B_i] = L[r][B_i] X[B_i][B_i]
//   for the rows r after B_i.
// As soon as the columns of B_i are final (and for B_0 no earlier than AUX_FORK_REST
// columns before the end), its inverse X[B_i][B_i] (recursive doubling) and these
// products run on the auxiliary stream, beside the remaining (latency-bound)
// factorization steps.  After the loop only the last block's inverse and one product
// remain on the caller's stream.  (A last block of at most 512 columns measured 3%
// faster than 1024 at d = 3000 and 4096, and the same at 11008; 256 no better.)
// Deferral of the trailing update (see cholinv) from d = DEFER_MIN_D on, in outer blocks
// of DEFER_W_SMALL columns below DEFER_W_MIN_D and DEFER_W from there.  A step's update
// of the whole trailing matrix reads and writes it for 2 * 64 flops per element (8 flops
// per byte in fp64: bound by HBM once the matrix leaves the caches); deferred, the update
// after an outer block does 2 W.
#ifndef DEFER_MIN_D
#define DEFER_MIN_D 4200
#endif
#ifndef DEFER_W
#define DEFER_W 512
#endif
#ifndef DEFER_W_SMALL
#define DEFER_W_SMALL 256
#endif
#ifndef DEFER_W_MIN_D
#define DEFER_W_MIN_D 7168
#endif
#ifndef AUX_MAX_WG_DEFER
#define AUX_MAX_WG_DEFER 0
#endif
#ifndef AUX_FORK_REST
#define AUX_FORK_REST 8192
#endif
#ifndef INV_LAST
#define INV_LAST 512
#endif
static gptq_status cholinv(PrepCtx& c, const PrepAux* aux) {
    const int64_t d = c.d;
    gptq_status st;
    prep_diag_kernel<<<1, 256, 0, c.s>>>(c.A, c.X, d, 0, (int)std::min<int64_t>(PNB, d), c.info);
    GPTQ_LAUNCH_CHECK();
    if (d <= PNB) return GPTQ_OK;
    prep_panel_kernel<<<(unsigned)((d - PNB + 63) / 64), 256, 0, c.s>>>(c.A, c.X, d, 0);
    GPTQ_LAUNCH_CHECK();

    // row blocks: B_i = [bs[i], bs[i + 1]) for i < nb, the last block [bs[nb], d)
    int64_t bs[64];
    int nb = 0;
    for (int64_t s0 = 0;;) {
        const int64_t r = d - s0;
        if (r <= PNB || (nb > 0 && r <= INV_LAST)) { bs[nb] = s0; break; }
        int64_t b = PNB;
        while (2 * b < r) b *= 2;
        bs[nb++] = s0;
        s0 += b;
    }
    const int64_t h = bs[1], sl = bs[nb], nl = d - sl;
    if (h * h + (d - h) * sl + nl * nl > d * d) return GPTQ_ERR_INVALID_ARG;   // scratch bound
    // product scratch (doubles): the auxiliary levels (h * h), Trest (rows h .. d, row
    // pitch sl, columns 0 .. sl), the last block's levels (nl * nl); with m = d - h <= h:
    // h * h + m * sl + nl * nl <= h * h + m * d + m * m <= d * d
    double* Saux = c.T;
    double* Trest = c.T + h * h;
    double* Smain = Trest + (d - h) * sl;
    auto trow = [&](int64_t r) { return Trest + (r - h) * sl; };

    // Without an auxiliary stream the same work is queued on the caller's stream at the
    // same points (stream order then gives every dependency) with an uncapped grid.
    PrepCtx ca = c;
    if (aux) ca.s = aux->s;
    // (the cap keeps slots free for the latency-bound chain at moderate d; with the
    // deferred update the auxiliary products run mostly after the chain, uncapped)
    const int aux_wg = aux ? (d < DEFER_MIN_D ? AUX_MAX_WG : AUX_MAX_WG_DEFER) : 0;
    // block i's columns are final once the step that forms the panel of its last 64
    // columns has been enqueued (step bs[i + 1] / 64 - 2; before the loop when negative)
    int64_t fork_step[64];
    for (int i = 0; i < nb; ++i) {
        fork_step[i] = bs[i + 1] / PNB - 2;
        if (i == 0) fork_step[i] = std::max<int64_t>(fork_step[i], (d - AUX_FORK_REST) / PNB);
        else fork_step[i] = std::max(fork_step[i], fork_step[i - 1]);
    }
    auto fork = [&](int i) -> gptq_status {
        if (aux && (hipEventRecord(aux->fork, c.s) != hipSuccess ||
                    hipStreamWaitEvent(ca.s, aux->fork, 0) != hipSuccess))
            return GPTQ_ERR_HIP;
        const int64_t b0 = bs[i], b1 = bs[i + 1], len = b1 - b0, below = d - b1;
        gptq_status r;
        if ((r = trtri_block(ca, b0, len, Saux, aux_wg)) != GPTQ_OK) return r;
        if (i > 0) {
            // X[B_i][P_i] = -X[B_i][B_i] Trest[B_i][P_i]   (lower triangular X block)
            if ((r = gemm(ca, c.X + b0 * d, d, c.X + b0 * d + b0, d, trow(b0), sl, (int)len, (int)b0, (int)len, -1.0,
                          0.0, G_TRI_A, 1, 0, 0, 0, 0, 0, 0, 0, aux_wg)) != GPTQ_OK)
                return r;
            // Trest[after B_i][P_i] += L[after B_i][B_i] X[B_i][P_i]
            if ((r = gemm(ca, trow(b1), sl, c.A + b1 * d + b0, d, c.X + b0 * d, d, (int)below, (int)b0, (int)len, 1.0,
                          1.0, 0, 1, 0, 0, 0, 0, 0, 0, 0, aux_wg)) != GPTQ_OK)
                return r;
        }
        // Trest[after B_i][B_i] = L[after B_i][B_i] X[B_i][B_i]   (lower triangular X block)
        if ((r = gemm(ca, trow(b1) + b0, sl, c.A + b1 * d + b0, d, c.X + b0 * d + b0, d, (int)below, (int)len, (int)len,
                      1.0, 0.0, G_TRI_B, 1, 0, 0, 0, 0, 0, 0, 0, aux_wg)) != GPTQ_OK)
            return r;
        if (aux && hipEventRecord(aux->join, ca.s) != hipSuccess) return GPTQ_ERR_HIP;
        return GPTQ_OK;
    };
    int nf = 0;   // blocks handed to the auxiliary stream
    while (nf < nb && fork_step[nf] < 0)
        if ((st = fork(nf++)) != GPTQ_OK) return st;
    // deferred trailing update (large d): inside an outer block of defer_w columns each
    // step updates only the rest of the outer block (all rows below), and the step of the
    // block's last panel applies all defer_w columns to the matrix after the block at once
    const int64_t defer_w = (d < DEFER_MIN_D) ? PNB : (d < DEFER_W_MIN_D) ? DEFER_W_SMALL : DEFER_W;
    for (int64_t k0 = 0; k0 < d; k0 += PNB) {
        const int n = (int)std::min<int64_t>(PNB, d - k0);
        const int64_t rest = d - k0 - n;
        if (rest <= 0) break;
        const int64_t K0 = k0 / defer_w * defer_w;                  // the outer block [K0, oe)
        const int64_t oe = std::min<int64_t>(K0 + defer_w, d);
        // trailing update; tile (0, 0) factors diagonal block k+1, the tiles below it
        // form panel k+1
        double* A22 = c.A + (k0 + n) * d + k0 + n;
        const bool inner = k0 + n < oe;
        const int64_t kb = inner ? k0 : K0;                          // update columns kb .. k0 + n
        double* L21 = c.A + (k0 + n) * d + kb;
        const int kw = (int)(k0 + n - kb);
        const int flg = G_BT | G_LOWER_C | G_DIAG0 | G_PANEL1;
        const int n1 = (int)std::min<int64_t>(PNB, rest), step = (int)(k0 / PNB) + 1;
        // inner: the rest of the outer block; else the whole trailing matrix
        const int64_t ncols = inner ? oe - (k0 + n) : rest;
        if ((st = gemm(c, A22, d, L21, d, L21, d, (int)rest, (int)ncols, kw, -1.0, 1.0, flg, 1, 0, 0, 0, 0, k0 + n,
                       n1, step)) != GPTQ_OK)
            return st;
        while (nf < nb && fork_step[nf] == k0 / PNB)
            if ((st = fork(nf++)) != GPTQ_OK) return st;
    }
    while (nf < nb)
        if ((st = fork(nf++)) != GPTQ_OK) return st;
    // the last block's inverse, then X[last][P] = -X[last][last] Trest[last][P]
    if ((st = trtri_block(c, sl, nl, Smain)) != GPTQ_OK) return st;
    if (aux && hipStreamWaitEvent(c.s, aux->join, 0) != hipSuccess) return GPTQ_ERR_HIP;
    return gemm(c, c.X + sl * d, d, c.X + sl * d + sl, d, trow(sl), sl, (int)nl, (int)sl, (int)nl, -1.0, 0.0, G_TRI_A);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t t_bytes(int64_t d) {
    // product scratch: h * h doubles for the auxiliary levels, (d - h) * sl for Trest,
    // nl * nl for the last block's levels; at most d * d (see cholinv)
    return (size_t)d * d * sizeof(double);
}

size_t prep_ws_bytes(int64_t d) {
    if (d <= 0) return 0;
    const size_t dd = (size_t)d * d * sizeof(double);
    return align256(dd) * 2 + align256(t_bytes(d)) + 256;
}

gptq_status prep_launch(const float* H, float* U, int64_t d, float percdamp, void* ws, size_t ws_bytes,
                        int32_t* info, hipStream_t s, const PrepAux* aux) {
    if (ws == nullptr || ws_bytes < prep_ws_bytes(d)) return GPTQ_ERR_WORKSPACE;
    char* p = reinterpret_cast<char*>(ws);
    const size_t dd = align256((size_t)d * d * sizeof(double));
    PrepCtx c;
    c.A = reinterpret_cast<double*>(p);
    c.X = reinterpret_cast<double*>(p + dd);
    c.T = reinterpret_cast<double*>(p + 2 * dd);
    const size_t t = align256(t_bytes(d));
    double* lam = reinterpret_cast<double*>(p + 2 * dd + t);
    c.d = d; c.info = info; c.s = s;
    c.wait_polls = aux ? aux->wait_polls : PREP_WAIT_POLLS;
    c.flag = reinterpret_cast<int*>(lam + 1);    // inside the 256 reserved bytes

    prep_lambda_kernel<<<1, 1024, 0, s>>>(H, d, percdamp, lam, info, c.flag);
    GPTQ_LAUNCH_CHECK();
    dim3 gb((unsigned)((d + 255) / 256 < 64 ? (d + 255) / 256 : 64), (unsigned)d);
    dim3 gb4((unsigned)((d + 1023) / 1024 < 64 ? (d + 1023) / 1024 : 64), (unsigned)d);
    if ((d & 3) == 0 && (reinterpret_cast<uintptr_t>(H) & 15) == 0) prep_build_kernel<true><<<gb4, 256, 0, s>>>(H, d, lam, c.A);
    else prep_build_kernel<false><<<gb, 256, 0, s>>>(H, d, lam, c.A);
    GPTQ_LAUNCH_CHECK();
    gptq_status st;
    st = cholinv(c, aux);
    if (st != GPTQ_OK) return st;
    if ((d & 3) == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0) prep_output_kernel<true><<<gb4, 256, 0, s>>>(c.X, d, U);
    else prep_output_kernel<false><<<gb, 256, 0, s>>>(c.X, d, U);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
