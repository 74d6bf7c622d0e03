// Device helpers shared by the GPTQ kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <utility>

#include "gptq.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define GPTQ_DEV __device__ __forceinline__

// bf16 / fp16 bit patterns <-> fp32 (exact widening; narrowing rounds to nearest even).
GPTQ_DEV float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

GPTQ_DEV uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

GPTQ_DEV float f16_bits_to_f32(uint16_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, b);
    return (float)h;
}

GPTQ_DEV uint16_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

template <gptq_dtype DT>
GPTQ_DEV float load_as_f32(const void* base, int64_t idx) {
    if constexpr (DT == GPTQ_F32) return reinterpret_cast<const float*>(base)[idx];
    else if constexpr (DT == GPTQ_BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
    else return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// DPP broadcast of lane `src` of each group of 4 lanes to the whole group.
template <int SRC>
GPTQ_DEV float quad_bcast(float v) {
    constexpr int ctrl = SRC | (SRC << 2) | (SRC << 4) | (SRC << 6);  // quad_perm
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xf, 0xf, false));
}

// DPP quad_perm with an arbitrary pattern.
template <int CTRL>
GPTQ_DEV float quad_perm(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
GPTQ_DEV int quad_perm_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
// quad_perm encodings: lane i of the quad reads lane sel[i].
constexpr int QP_XOR1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // [1,0,3,2]
constexpr int QP_XOR2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // [2,3,0,1]

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. N-1.
template <int I, int N, typename F>
GPTQ_DEV void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// One direct global -> LDS load (global_load_lds_dwordx4, scalar-base form): lane i
// reads 16 bytes at sbase + voff_i and they land at LDS byte address m0base + MOFF +
// 16 i (M0 is formed in the asm from one wave-uniform register and a compile-time
// offset, so no register per slot and load stays live).
// (Written as inline asm: the compiler counts the builtin's LDS write against every
// later LDS read of the array and inserts a full vmcnt(0) wait before it, which would
// leave no load in flight; the callers place the waits explicitly, and the asm has no
// register results, the data going to LDS only.)
template <uint32_t MOFF>
GPTQ_DEV void dma16(uint32_t voff, const void* sbase, uint32_t m0base) {
    // the base and M0 are wave-uniform; readfirstlane makes that visible to the
    // compiler, which must place them in scalar registers
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t mu = __builtin_amdgcn_readfirstlane(m0base);
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(bu), "s"(mu), "i"(MOFF) : "memory", "scc");
}

// s_waitcnt vmcnt(VM) lgkmcnt(0), expcnt not waited for.
template <int VM>
GPTQ_DEV void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (0x7 << 4) | ((VM >> 4) << 14));
}

GPTQ_DEV uint32_t lds_addr(const uint16_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// Launch-error helper for the host side.
#define GPTQ_LAUNCH_CHECK()                                   \
    do {                                                      \
        if (hipGetLastError() != hipSuccess) return GPTQ_ERR_HIP; \
    } while (0)

// Codes of the 3-bit stream: eight codes in three bytes, code c in stream bits 3c .. 3c+2
// (lowest bit first), stream bit i in bit i % 8 of byte i / 8.  The 24 bits of an
// 8-code group as one integer (little-endian bytes), and code e of it.
GPTQ_DEV uint32_t load_u24(const uint8_t* p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
}
GPTQ_DEV uint32_t code3(uint32_t g24, int e) { return (g24 >> (3 * e)) & 7u; }

