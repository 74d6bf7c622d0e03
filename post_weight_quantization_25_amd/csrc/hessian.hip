// H += 2 X^T X on gfx950 matrix cores.
//
// GPTQ summary page, statement of the one-layer procedure: the layer Hessian
// H = 2 X X^T (page layout d_col x tokens; here X is tokens x d_col, so H = 2 X^T X).
//
// bf16 or fp16 X (rows 16-byte aligned): a symmetric rank-k update on
// v_mfma_f32_32x32x16_bf16 / _f16 (16-bit products are exact in fp32).  Only tiles
// on or above the diagonal are computed (256 x 256 output tiles, one workgroup of
// eight waves per CU, each wave accumulating a 64 x 128 sub-tile in 8 MFMAs).  X is stored
// token-major (channels contiguous), i.e. the contraction index is the strided
// one.  Tiles are copied to LDS as they lie in memory by direct global -> LDS
// loads (global_load_lds_dwordx4, no register staging) into a ring of four
// 32-token stages, and the MFMA operands, which need 8 consecutive tokens of one
// channel per lane, are read with the gfx950 transposing LDS read
// ds_read_b64_tr_b16; the 16-byte chunks of a row are XOR-swizzled so that these
// reads are free of bank conflicts.
// The token range is split S ways; XCDs are grouped and each group owns a compact
// run of tiles (see the work mapping in the kernel).  Each work item writes its
// fp32 partial tile; a second kernel sums the S partials of every element in split
// order and updates H, so results are bitwise reproducible.
//
// fp32 X, and 16-bit X whose rows are not 16-byte aligned: exact-product path on
// v_mfma_f32_16x16x4_f32, one WG per 64 x 64 upper tile over all tokens (no split).

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
constexpr int HB_BK = 32;            // tokens per LDS stage
constexpr int HB_NSTG = 4;           // LDS ring depth (stages in flight: 3 loading, 1 computing)
static_assert(HB_NSTG * 32 * 1024 <= 160 * 1024, "LDS ring exceeds the workgroup's LDS");
constexpr int HB_WAVES = 8;          // waves per workgroup, two per SIMD
constexpr int HB_WN = 128;           // columns per wave
constexpr int HB_WM = HB_BM * (HB_BM / HB_WN) / HB_WAVES;   // rows per wave (waves: rows x 2 columns)
constexpr int HB_THREADS = 64 * HB_WAVES;
constexpr int HB_FA = HB_WM / 32;    // 32 x 32 MFMA tiles per wave: HB_FA x HB_FB
constexpr int HB_FB = HB_WN / 32;
constexpr int HB_DMA = 32 / HB_WAVES;  // 1 KB direct-to-LDS loads per wave and stage
constexpr int HB_OPE = HB_BK * HB_BM;  // bf16 elements of one operand stage (16 KB)
constexpr int HB_STE = 2 * HB_OPE;     // bf16 elements of one stage (A then B)

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

struct HessBf16Args {
    const uint16_t* X; int64_t n; int d; int64_t ldx;
    float* H; float* partials;
    int nt; int T; int S; int64_t ks;  // tokens per split (multiple of HB_BK)
    int tpg;                           // tiles per XCD group
    int xpg;                           // XCDs per group (1, 2, 4 or 8)
};

// LDS layout of an operand stage: token rows of 256 channels (512 B, 32 chunks of
// 16 B), chunk c of row k stored at chunk position c ^ 2 f(k mod 4), f = 0, 3, 5, 6.
// A transposed fragment read touches 4 consecutive rows, 32 B per row for 16 lanes
// and 64 B per row for 32 lanes; with this swizzle the 4 rows fall on distinct banks
// both within 128 B (f mod 4 distinct) and within 256 B (f / 2 mod 4 distinct).
GPTQ_DEV int swz(int k, int c) {
    const int r = k & 3;
    const int f = 2 * r + ((r ^ (r >> 1)) & 1);
    return c ^ (f << 1);
}

// Per-wave constants of the stage copy.  Wave w issues loads HB_DMA w .. HB_DMA w +
// HB_DMA - 1 of 1 KB each; load i (of the wave) covers operand (HB_DMA w) / 16 (0: the
// c0 channel block, 1: c1), token rows kb + 2 i and kb + 2 i + 1 (kb = 2 ((HB_DMA w) mod
// 16)), lane l writing chunk position l % 32 of row kb + 2 i + l / 32, i.e. logical
// chunk swz(row, l % 32).  The per-lane byte offset of load i carries its row.
struct StageCopy {
    uint32_t voff[HB_DMA];  // per-lane byte offsets of the wave's loads
    int64_t row_elems;      // ldx
    int cbase;              // channel base of this wave's operand (wave-uniform)
    uint32_t m0base;        // LDS byte address of the wave's first block in slot 0
    bool skip;              // diagonal tile: the wave's operand is the other one, not loaded
};

GPTQ_DEV StageCopy stage_copy_setup(const HessBf16Args& a, const uint16_t* ring0, int c0, int c1, int wave,
                                    int lane) {
    StageCopy sc;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    sc.cbase = ((wave_u * HB_DMA) >> 4) ? c1 : c0;
    sc.row_elems = a.ldx;
    sc.m0base = lds_addr(ring0) + (uint32_t)(wave_u * HB_DMA) * 1024u;
    sc.skip = (c0 == c1) && ((wave_u * HB_DMA) >> 4);
    const int kb = ((wave * HB_DMA) & 15) * 2 + (lane >> 5), pc = lane & 31;
#pragma unroll
    for (int i = 0; i < HB_DMA; ++i)
        sc.voff[i] = (uint32_t)(((int64_t)(kb + 2 * i) * a.ldx + 8 * swz(kb + 2 * i, pc)) * 2);
    return sc;
}

// Direct global -> LDS copy of one stage (tokens t0 .. t0 + 31) into ring slot SLOT.
template <int SLOT>
GPTQ_DEV void issue_stage(const HessBf16Args& a, const StageCopy& sc, int64_t t0) {
    if (sc.skip) return;
    const uint16_t* sbase = a.X + t0 * sc.row_elems + sc.cbase;
    static_for<0, HB_DMA>([&](auto I) {
        constexpr int i = decltype(I)::value;
        dma16<(uint32_t)(SLOT * HB_STE * 2 + i * 1024)>(sc.voff[i], sbase, sc.m0base);
    });
}

// Register path for tiles at the matrix edge or a partial stage: zero-filled loads
// written to the same swizzled layout.
GPTQ_DEV void copy_stage_edge(const HessBf16Args& a, uint16_t* buf, int64_t t0, int64_t t_end, int c0, int c1, int tid) {
#pragma unroll
    for (int i = 0; i < 2048 / HB_THREADS; ++i) {
        const int p = tid + HB_THREADS * i;
        const int op = p >> 10, pos = p & 1023;
        const int k = pos >> 5, pc = pos & 31;
        const int c = swz(k, pc);
        const int64_t t = t0 + k;
        const int ch = (op ? c1 : c0) + 8 * c;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (t < t_end) {
            if (ch + 8 <= a.d && ((reinterpret_cast<uintptr_t>(a.X + t * a.ldx + ch) & 15) == 0)) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.X + t * a.ldx + ch);
                w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
            } else {
                for (int e = 0; e < 8; ++e) {
                    const uint32_t v = (ch + e < a.d) ? (uint32_t)a.X[t * a.ldx + ch + e] : 0u;
                    w[e >> 1] |= v << (16 * (e & 1));
                }
            }
        }
        *reinterpret_cast<u32x4_t*>(buf + p * 8) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
}

// MFMA operand fragment (32 channels x 16 tokens, lane l: channel l % 32, tokens
// 8 (l / 32) .. +7) from a token-major swizzled operand stage, with two
// ds_read_b64_tr_b16.  In each 16-lane group the instruction returns to lane i,
// element e, the (i & 3)-th value of the 8-byte chunk addressed by lane (i >> 2) + 4 e;
// lane j therefore addresses token k0 + (j >> 2), channels m0 + 4 (j & 3) .. +3, and
// lane i receives channel m0 + i at tokens k0 .. k0 + 3.
GPTQ_DEV bf16x8_t read_frag(const uint16_t* op, int ch0, int kk, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int m = ch0 + (g & 1) * 16 + 4 * (j & 3);
    const int k0 = kk + (g >> 1) * 8 + (j >> 2);
    const int c = m >> 3, half = (m >> 2) & 1;
    const int k1 = k0 + 4;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(op + k0 * HB_BM + 8 * swz(k0, c) + 4 * half));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(op + k1 * HB_BM + 8 * swz(k1, c) + 4 * half));
    typedef short v8i16_t __attribute__((ext_vector_type(8)));
    const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// One wave's operand fragments for one 16-token slice of a stage: 2 (rows) + 4
// (columns) fragments of 32 channels.
struct Frags { bf16x8_t a[HB_FA], b[HB_FB]; };

// On a diagonal tile both operands are the same channel block, loaded once (DIAG).
template <bool DIAG = false>
GPTQ_DEV void read_slice(const uint16_t* stg, int kk, int wr, int wc, int lane, Frags& f) {
#pragma unroll
    for (int i = 0; i < HB_FA; ++i) f.a[i] = read_frag(stg, wr * HB_WM + i * 32, kk, lane);
#pragma unroll
    for (int j = 0; j < HB_FB; ++j) f.b[j] = read_frag(stg + (DIAG ? 0 : HB_OPE), wc * HB_WN + j * 32, kk, lane);
}

// F16: the fragments hold fp16 bit patterns (the same 16-bit copies and reads), multiplied
// on v_mfma_f32_32x32x16_f16; products of two fp16 values are exact in fp32 too.
template <bool F16>
GPTQ_DEV void mfma_slice(const Frags& f, f32x16_t (&acc)[HB_FA][HB_FB]) {
#pragma unroll
    for (int i = 0; i < HB_FA; ++i)
#pragma unroll
        for (int j = 0; j < HB_FB; ++j) {
            if constexpr (F16)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, f.a[i]),
                                                                   __builtin_bit_cast(f16x8_t, f.b[j]), acc[i][j], 0, 0, 0);
            else
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        }
}

// Scheduling hint for one region of the pipelined loop, which holds the LDS reads of
// the next slice and the MFMAs of the current one (12 and 8 with eight waves, 16 and
// 16 with four): issue them interleaved, so that the LDS port and the matrix core work
// at the same time instead of in bursts.
GPTQ_DEV void interleave_reads_mfma() {
    constexpr int NR = 2 * (HB_FA + HB_FB), NM = HB_FA * HB_FB;   // LDS reads, MFMAs
    static_assert((NR == 12 && NM == 8) || NR == NM, "interleave pattern for this wave layout");
    if constexpr (NR == 12 && NM == 8) {
        static_for<0, 4>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        });
        static_for<0, 4>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        });
    } else {
        static_for<0, NM>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        });
    }
}

// The MFMAs of one LDS stage for one wave (both slices), used by the edge path.
template <bool F16>
GPTQ_DEV void mfma_stage(const uint16_t* stg, int wr, int wc, int lane, f32x16_t (&acc)[HB_FA][HB_FB]) {
#pragma unroll
    for (int kk = 0; kk < HB_BK; kk += 16) {
        Frags f;
        read_slice(stg, kk, wr, wc, lane, f);
        mfma_slice<F16>(f, acc);
    }
}

// s_waitcnt vmcnt(HB_VM) lgkmcnt(0): the loads of the HB_NSTG - 2 stages issued after
// the one about to be used may stay in flight; this wave's LDS reads are complete.
constexpr int HB_VM = (HB_NSTG - 2) * HB_DMA;
static_assert(HB_VM < 64, "vmcnt field");
GPTQ_DEV void wait_vm8_lgkm0() { __builtin_amdgcn_s_waitcnt((HB_VM & 15) | (0x7 << 4) | ((HB_VM >> 4) << 14)); }

// Fast path: every stage full and the tile inside the matrix.  LDS ring of HB_NSTG
// stages, DMA issued HB_NSTG - 1 stages ahead (re-loads of the last stage past the end
// keep the number of loads in flight constant, so one wait count fits every step),
// and the LDS reads software-pipelined by 16-token slices: the fragments of the
// next slice are read while the MFMAs of the current one run.  Step u:
//   read slice 1 of stage u | MFMAs of slice 0 | wait stage u+1, barrier |
//   DMA stage u+HB_NSTG into stage u's slot | read slice 0 of stage u+1 | MFMAs of slice 1.
// The reads of the next stage are issued also after the last stage (of a slot that
// stays inside the ring, results unused), so that each region is one basic block
// and the reads can be interleaved with the MFMAs.
// Whether wave w's sub-tile of a diagonal tile lies strictly below the diagonal (its
// first row after its last column).  Wave-uniform by construction.
GPTQ_DEV bool below_diagonal(int wave) {
    const int w = __builtin_amdgcn_readfirstlane(wave);
    return (w >> 1) * HB_WM > (w & 1) * HB_WN + HB_WN - 1;
}

// DIAG: a diagonal tile (c0 == c1).  One operand is loaded, and the waves whose
// sub-tile lies strictly below the diagonal (never read by the reduction) only take
// part in the loads and barriers.
template <bool DIAG, bool F16>
GPTQ_DEV void hess_loop_dma(const HessBf16Args& a, uint16_t* const (&ring)[HB_NSTG], int64_t t_beg, int64_t nst,
                            int c0, int c1, int wr, int wc, int wave, int lane, f32x16_t (&acc)[HB_FA][HB_FB]) {
    const bool work = !DIAG || !below_diagonal(wave);
    auto t0 = [&](int64_t st) { return t_beg + (st < nst ? st : nst - 1) * HB_BK; };
    const StageCopy sc = stage_copy_setup(a, ring[0], c0, c1, wave, lane);
    static_for<0, HB_NSTG - 1>([&](auto I) { issue_stage<decltype(I)::value>(a, sc, t0(decltype(I)::value)); });
    wait_vm8_lgkm0();
    __syncthreads();
    issue_stage<HB_NSTG - 1>(a, sc, t0(HB_NSTG - 1));
    Frags f0, f1;
    if (work) read_slice<DIAG>(ring[0], 0, wr, wc, lane, f0);
    for (int64_t st = 0; st < nst; st += HB_NSTG) {
        static_for<0, HB_NSTG>([&](auto U) {
            constexpr int u = decltype(U)::value;
            if (st + u < nst) {
                if (work) {
                    read_slice<DIAG>(ring[u], 16, wr, wc, lane, f1);
                    mfma_slice<F16>(f0, acc);
                    interleave_reads_mfma();
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the phases in this order
                wait_vm8_lgkm0();
                __syncthreads();
                issue_stage<u>(a, sc, t0(st + u + HB_NSTG));
                if (work) {
                    read_slice<DIAG>(ring[(u + 1) % HB_NSTG], 0, wr, wc, lane, f0);
                    mfma_slice<F16>(f1, acc);
                    interleave_reads_mfma();
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    }
    __builtin_amdgcn_s_waitcnt(0);   // drain the trailing re-loads before the LDS is reused
    __syncthreads();
}

// Edge path: register copies, two LDS stages.
template <bool F16>
GPTQ_DEV void hess_loop_edge(const HessBf16Args& a, uint16_t* const (&ring)[HB_NSTG], int64_t t_beg, int64_t t_end,
                             int64_t nst, int c0, int c1, int wr, int wc, int tid, int lane, f32x16_t (&acc)[HB_FA][HB_FB]) {
    for (int64_t st = 0; st < nst; st += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (st + u < nst) {
                copy_stage_edge(a, ring[u], t_beg + (st + u) * HB_BK, t_end, c0, c1, tid);
                __syncthreads();
                mfma_stage<F16>(ring[u], wr, wc, lane, acc);
            }
        }
    }
    __syncthreads();
}

template <bool F16>
__global__ __launch_bounds__(HB_THREADS, 1) void hess_bf16_kernel(HessBf16Args a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_ring[HB_NSTG * HB_STE];  // HB_NSTG x 32 KB
    uint16_t* ring[HB_NSTG];
    static_for<0, HB_NSTG>([&](auto I) { ring[decltype(I)::value] = lds_ring + decltype(I)::value * HB_STE; });

    // XCD-aware work mapping: workgroup L runs on XCD L % 8 (round-robin dispatch).
    // The tiles, in super-tile order, are cut into 8 / xpg runs of tpg tiles; the xpg
    // XCDs of a group share one run and take its token splits in turn, each XCD
    // walking its splits in order.  The 32 CUs of an XCD thus work on one or two
    // splits of one compact run of tiles, whose few distinct channel blocks are
    // shared through that XCD's L2.
    const int L = blockIdx.x;
    const int xcd = L & 7, k = L >> 3;
    const int grp = xcd / a.xpg, xi = xcd % a.xpg;
    const int tig = k % a.tpg;
    const int s = (k / a.tpg) * a.xpg + xi, tile = grp * a.tpg + tig;
    if (s >= a.S || tile >= a.T) return;
    int ti, tj;
    upper_tile(tile, a.nt, ti, tj);
    const int c0 = ti * HB_BM, c1 = tj * HB_BM;
    const int64_t t_beg = (int64_t)s * a.ks;
    const int64_t t_end = (t_beg + a.ks < a.n) ? t_beg + a.ks : a.n;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    f32x16_t acc[HB_FA][HB_FB];
#pragma unroll
    for (int i = 0; i < HB_FA; ++i)
#pragma unroll
        for (int j = 0; j < HB_FB; ++j) acc[i][j] = f32x16_t{};

    const int64_t nst = (t_end > t_beg) ? (t_end - t_beg + HB_BK - 1) / HB_BK : 0;
    // the DMA path: whole tiles, whole stages, 16-byte aligned rows, per-lane offsets
    // (up to 31 rows) within 32 bits
    const bool full = (c0 + HB_BM <= a.d) && (c1 + HB_BM <= a.d) && ((t_end - t_beg) % HB_BK == 0) &&
                      ((reinterpret_cast<uintptr_t>(a.X) & 15) == 0) && ((a.ldx & 7) == 0) &&
                      (a.ldx < ((int64_t)1 << 25));
    if (nst > 0) {
        if (full && c0 == c1) hess_loop_dma<true, F16>(a, ring, t_beg, nst, c0, c1, wr, wc, wave, lane, acc);
        else if (full) hess_loop_dma<false, F16>(a, ring, t_beg, nst, c0, c1, wr, wc, wave, lane, acc);
        else hess_loop_edge<F16>(a, ring, t_beg, t_end, nst, c0, c1, wr, wc, tid, lane, acc);
    }

    // this split's partial tile (row-major 256 x 256 fp32); the reduction reads no
    // element below the diagonal of a diagonal tile
    if (c0 == c1 && below_diagonal(wave)) return;
    float* P = a.partials + ((int64_t)s * a.T + tile) * (HB_BM * HB_BM);
#pragma unroll
    for (int i = 0; i < HB_FA; ++i)
#pragma unroll
        for (int j = 0; j < HB_FB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = wr * HB_WM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int nn = wc * HB_WN + j * 32 + (lane & 31);
                P[m * HB_BM + nn] = acc[i][j][e];
            }
}

// Split reduction: H += 2 * (sum of the S partial tiles, in split order), on the upper
// triangle, mirrored into the lower triangle.  One workgroup per 16 rows of a tile;
// thread t sums 4 x 4 consecutive columns with 16-byte loads (columns 4 (t % 16) +
// 64 q, row t / 16), so every partial is read once, coalesced, by the whole grid.
constexpr int HR_ROWS = 16;

__global__ __launch_bounds__(256) void hess_reduce_kernel(HessBf16Args a) {
    __shared__ float st[HR_ROWS][HB_BM + 1];
    const int tile = blockIdx.x / (HB_BM / HR_ROWS), rc = blockIdx.x % (HB_BM / HR_ROWS);
    int ti, tj;
    upper_tile(tile, a.nt, ti, tj);
    const int c0 = ti * HB_BM, c1 = tj * HB_BM;
    const int tid = threadIdx.x, ml = tid >> 4, m = rc * HR_ROWS + ml;
    const int64_t tstride = (int64_t)a.T * HB_BM * HB_BM;
    const float* P = a.partials + (int64_t)tile * (HB_BM * HB_BM) + m * HB_BM + 4 * (tid & 15);
    f32x4_t v[4] = {};
#pragma unroll 4
    for (int ss = 0; ss < a.S; ++ss) {
        f32x4_t x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            x[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(P + ss * tstride + 64 * q));
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += x[q];
    }
    const int gr = c0 + m;
    // all loads of H first, then the stores (a load after a store to the same array
    // would otherwise wait for that store's round trip)
    float h0[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int gc = c1 + 4 * (tid & 15) + 64 * q + e;
            h0[q][e] = (gr < a.d && gc < a.d && gr <= gc) ? a.H[(int64_t)gr * a.d + gc] : 0.f;
        }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int nn = 4 * (tid & 15) + 64 * q + e, gc = c1 + nn;
            if (gr < a.d && gc < a.d && gr <= gc) {
                const float nv = h0[q][e] + 2.f * v[q][e];
                a.H[(int64_t)gr * a.d + gc] = nv;
                st[ml][nn] = nv;
            }
        }
    __syncthreads();
    // mirror: thread t writes column c1 + t of the slice as row c1 + t of H, i.e. the
    // HR_ROWS consecutive entries H[c1 + t][c0 + rc HR_ROWS ..]: 16-byte stores when the
    // whole slice lies below the diagonal and inside H with aligned rows, else one by one
    const int gc = c1 + tid, g0 = c0 + rc * HR_ROWS;
    if (gc < a.d) {
        if (c0 < c1 && g0 + HR_ROWS <= a.d && (a.d & 3) == 0 && (reinterpret_cast<uintptr_t>(a.H) & 15) == 0) {
            float* dst = a.H + (int64_t)gc * a.d + g0;
#pragma unroll
            for (int r = 0; r < HR_ROWS; r += 4)
                *reinterpret_cast<f32x4_t*>(dst + r) = f32x4_t{st[r][tid], st[r + 1][tid], st[r + 2][tid], st[r + 3][tid]};
        } else {
#pragma unroll
            for (int r = 0; r < HR_ROWS; ++r) {
                const int g = g0 + r;
                if (g < a.d && g < gc) a.H[(int64_t)gc * a.d + g] = st[r][tid];
            }
        }
    }
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

struct Bf16Plan {
    int nt, T, S, tpg, xpg;
    int64_t ks;
    int grid() const { return 8 * tpg * ((S + xpg - 1) / xpg); }
};

static Bf16Plan bf16_plan(int64_t n, int64_t d) {
    Bf16Plan p;
    p.nt = (int)((d + HB_BM - 1) / HB_BM);
    p.T = p.nt * (p.nt + 1) / 2;
    // one run of tiles per XCD (8 groups); fewer, larger groups raise the L2 hit rate
    // but were not faster at d = 4096 once the split reduction ran in parallel
    const int G = 8;
    p.xpg = 8 / G;
    p.tpg = (p.T + G - 1) / G;
    const int64_t nst = (n + HB_BK - 1) / HB_BK;
    // split count: minimize the estimated time = rounds of the 32 workgroup slots of
    // an XCD (one per CU) x stages per item x time of one 32-token stage of a
    // 256 x 256 tile (about 0.75 us), plus writing and reading back the S partial
    // tiles of 256 KB each (about 4 TB/s)
    const int slots_per_xcd = 32;
    const double t_stage = 0.75e-6, bw = 4.0e12;
    int best = 1;
    double best_cost = 1e300;
    for (int sp = 1; sp <= 64; ++sp) {
        if (sp > 1 && (int64_t)sp > nst) break;
        const double items = (double)p.tpg * ((sp + p.xpg - 1) / p.xpg);   // per XCD
        const double rounds = std::ceil(items / slots_per_xcd);
        const double stages = (double)((nst + sp - 1) / sp);
        const double p_bytes = (double)sp * p.T * HB_BM * HB_BM * 4.0 * 2.0;
        const double cost = rounds * stages * t_stage + p_bytes / bw;
        if (cost < best_cost - 1e-12) { best_cost = cost; best = sp; }
    }
    p.S = best;
    p.ks = ((nst + p.S - 1) / p.S) * HB_BK;
    return p;
}

size_t hessian_ws_bytes(int64_t n, int64_t d) {
    if (n <= 0 || d <= 0) return 0;
    const Bf16Plan p = bf16_plan(n, d);
    return (size_t)p.T * p.S * HB_BM * HB_BM * sizeof(float);
}

gptq_status hessian_launch(float* H, const void* X, gptq_dtype dt, int64_t n, int64_t d, int64_t ldx,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && ((ldx & 7) == 0);
    if ((dt == GPTQ_BF16 || dt == GPTQ_F16) && aligned) {
        HessBf16Args a;
        const Bf16Plan p = bf16_plan(n, d);
        if (ws_bytes < hessian_ws_bytes(n, d) || ws == nullptr) return GPTQ_ERR_WORKSPACE;
        a.X = reinterpret_cast<const uint16_t*>(X); a.n = n; a.d = (int)d; a.ldx = ldx;
        a.H = H;
        a.partials = reinterpret_cast<float*>(ws);
        a.nt = p.nt; a.T = p.T; a.S = p.S; a.ks = p.ks; a.tpg = p.tpg; a.xpg = p.xpg;
        if (dt == GPTQ_F16) hess_bf16_kernel<true><<<p.grid(), HB_THREADS, 0, stream>>>(a);
        else hess_bf16_kernel<false><<<p.grid(), HB_THREADS, 0, stream>>>(a);
        GPTQ_LAUNCH_CHECK();
        hess_reduce_kernel<<<p.T * (HB_BM / HR_ROWS), 256, 0, stream>>>(a);
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
