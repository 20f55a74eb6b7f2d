// Device helpers shared by the quantize, dequantize and decode kernels.
//
// 128-element block layout used by the quantize/dequantize kernels: eight lanes
// own one block, sixteen consecutive elements each.  Element e = 16*j + k lives
// in register k of the lane with "virtual lane" j (0..7).  Within a 16-lane DPP
// row, the physical lane of virtual lane j of block half `sel` is
//     p = (j & 3) | (sel << 2) | ((j >> 2) << 3)
// so flipping bit 0, 1, 2 of j is a physical xor 1, 2, 8 - all three are single
// DPP moves (quad_perm, quad_perm, row_ror:8).  A 64-lane wave therefore holds
// eight blocks (two per DPP row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

// DPP control words (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;   // row_ror:4
constexpr int kDppRor8 = 0x128;   // row_ror:8 (= xor 8 inside a 16-lane row)

// Every control above reads a valid lane of the same row, so bound_ctrl (zero for
// an out-of-range source) never applies; setting it lets the compiler fold the
// move into the add or max that uses it (one DPP instruction instead of two).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the eight lanes of one block (virtual-lane bits <-> xor 1, 2, 8).
__device__ __forceinline__ float block8_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppRor8>(x);
    return x;
}

// Unnormalised Walsh-Hadamard transform of the 16 in-register elements
// (element-index bits 0..3), natural Sylvester order: (a, b) -> (a + b, a - b)
// on pairs that differ in one index bit.  `from` skips already-done stages.
template <int FROM = 1>
__device__ __forceinline__ void wht16(float (&v)[16]) {
#pragma unroll
    for (int h = FROM; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (!(i & h)) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

// The three cross-lane stages (element-index bits 4, 5, 6 = virtual-lane bits 0,
// 1, 2).  Each lane forms  mine + mu * partner  with mu = -1 on the lane whose
// bit is set; that lane then holds the negated difference, so after the three
// stages lane j holds (-1)^popcount(j) times the true transform.  The caller
// folds that sign into its per-lane scale (see lane_sign()).  Products by +-1
// are exact, so every output is rounded once per stage, exactly as a plain
// add or subtract would be.
//
// Each stage is one v_fmac_f32 with a DPP source per element.  The compiler
// does not fold a DPP move into v_fmac, so the stage is written out; the
// leading s_nop 1 gives the two wait states a DPP read of a VGPR needs after a
// VALU write of it, and the trailing one covers DPP reads emitted after the
// block.  Within a stage every instruction reads only its own register.
#define TQ_FMAC_DPP16(CTRL)                                                              \
    asm volatile(                                                                        \
        "s_nop 1\n\t"                                                                     \
        "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"              \
        "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "s_nop 1"                                                                        \
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),        \
          "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),       \
          "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                              \
        : "v"(mu))

__device__ __forceinline__ void wht_cross(float (&v)[16], int j) {
    float mu = (j & 1) ? -1.f : 1.f;
    TQ_FMAC_DPP16("quad_perm:[1,0,3,2]");
    mu = (j & 2) ? -1.f : 1.f;
    TQ_FMAC_DPP16("quad_perm:[2,3,0,1]");
    mu = (j & 4) ? -1.f : 1.f;
    TQ_FMAC_DPP16("row_ror:8");
}

// floor(t) as int32 in one instruction.
__device__ __forceinline__ int cvt_floor(float t) {
    int g;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(g) : "v"(t));
    return g;
}

// (a + b, a - b) in float32 straight from the two float16 halves of w (exact).
__device__ __forceinline__ void half_pair_butterfly(uint32_t w, float &sum, float &diff) {
    asm("v_fma_mix_f32 %0, %2, 1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %1, %2, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
        : "=&v"(sum), "=v"(diff)
        : "v"(w));
}

__device__ __forceinline__ float lane_sign(int j) { return (__popc(j) & 1) ? -1.f : 1.f; }

// Virtual lane / block-in-wave of the calling lane.
struct Lane8 {
    int j;      // virtual lane 0..7 (owns elements 16j .. 16j+15)
    int vin;    // block within the wave, 0..7
};
__device__ __forceinline__ Lane8 lane8() {
    const int lane = threadIdx.x & 63;
    const int pl = lane & 15;
    Lane8 r;
    r.j = (pl & 3) | ((pl >> 3) << 2);
    r.vin = (lane >> 4) * 2 + ((pl >> 2) & 1);
    return r;
}

// Code i (compile-time) of an LSB-first bitstream held in 32-bit words.
template <int BITS, int I>
__device__ __forceinline__ uint32_t stream_code(const uint32_t *w) {
    constexpr int bit = BITS * I;
    constexpr int d = bit >> 5;
    constexpr int o = bit & 31;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    if constexpr (o + BITS <= 32) {
        return (w[d] >> o) & mask;
    } else {
        return __builtin_amdgcn_alignbit(w[d + 1], w[d], o) & mask;
    }
}

}  // namespace tq
