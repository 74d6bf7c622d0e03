// Internal declarations shared by the quantization kernels.
#pragma once
#include "common.h"

namespace gptq {

constexpr int QB = 128;             // lazy-update block width (columns)
constexpr int QT = 256;             // threads per sweep workgroup
constexpr int SL = 16;              // lanes per row in the sweep (one DPP row)
constexpr int SROWS = QT / SL;      // rows per sweep workgroup

struct SweepArgs {
    const float* Wws; int64_t d_row, d_col;
    const float* U;
    int64_t b0; int nb;
    uint16_t* Ehi; uint16_t* Elo;   // error block of this block as bf16 hi + lo (hi = bf16(e),
    int64_t lde;                    // lo = bf16(e - hi)): d_row x 128, row stride lde
    uint8_t* codes; int64_t code_ld;
    uint16_t* scales; uint16_t* zeros; int n_groups;
    int32_t* info;
    int group;                      // 32, 64, 128 (power of two), or 0 = per-row params precomputed
    int qmin, qmax, zoff;           // grid and stored-code offset
    int sym; int packed;            // packed: two codes per byte
};

gptq_status sweep_launch(const SweepArgs& a, hipStream_t s);

}  // namespace gptq
