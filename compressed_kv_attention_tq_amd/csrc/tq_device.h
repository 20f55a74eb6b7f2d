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

// Quantize one 128-element block held in the 8-lane layout above: lane j has
// elements 16j .. 16j+15 as float16 pairs w16 and their 16 sign bits sb; bnd
// (any address space) holds the 2^BITS - 1 boundaries in ascending order.
// code[k] = the number of boundaries below y = H (s * x / |x|) / sqrt(128) for
// element 16j + k, found by binary descent (BITS steps; equal to the count for
// sorted boundaries); a zero or non-finite vector encodes y = 0.  Returns the
// norm |x| (every lane of the block).  The arithmetic of the quantize kernel.
template <int BITS, typename BndPtr>
__device__ __forceinline__ float encode_block8(const uint32_t (&w16)[8], uint32_t sb, BndPtr bnd, int j,
                                               uint32_t (&code)[16]) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    uint32_t w[8];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t m = (((sb >> (2 * k)) & 1u) << 15) | (((sb >> (2 * k + 1)) & 1u) << 31);
        w[k] = w16[k] ^ m;
        const h2_t h = __builtin_bit_cast(h2_t, w[k]);
        ss = __builtin_amdgcn_fdot2(h, h, ss, false);
    }
    ss = block8_sum(ss);
    const bool finite = ss <= 3.402823466e38f;   // false for inf and NaN
    if (!finite) {
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = 0;
    }
    const float tscale = (finite && ss > 0.f) ? lane_sign(j) * 0.088388347648318440550f * __frsqrt_rn(ss) : 0.f;
    float v[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) half_pair_butterfly(w[k], v[2 * k], v[2 * k + 1]);
    wht16<2>(v);
    wht_cross(v, j);
    float y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        y[k] = v[k] * tscale;
        code[k] = 0;
    }
#pragma unroll
    for (int lvl = BITS - 1; lvl >= 0; --lvl)
#pragma unroll
        for (int k = 0; k < 16; ++k)
            code[k] += y[k] > bnd[code[k] + (1u << lvl) - 1u] ? (1u << lvl) : 0u;
    return __fsqrt_rn(ss);
}

// Lane j's 16 codes (elements 16j .. 16j+15 of a block) as its 2 * BITS bytes of
// the block's LSB-first bitstream: lo, then (3 and 4 bits) hi.
template <int BITS>
__device__ __forceinline__ void pack_lane_codes(const uint32_t (&code)[16], uint32_t &lo, uint32_t &hi) {
    lo = 0;
    hi = 0;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 8; ++k) lo |= code[k] << (4 * k);
#pragma unroll
        for (int k = 0; k < 8; ++k) hi |= code[8 + k] << (4 * k);
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int k = 0; k < 16; ++k) lo |= code[k] << (2 * k);
    } else {  // 3 bits: 48 bits
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (3 * k + 3 <= 32) lo |= code[k] << (3 * k);
            else if (3 * k >= 32) hi |= code[k] << (3 * k - 32);
            else { lo |= code[k] << (3 * k); hi |= code[k] >> (32 - 3 * k); }
        }
    }
}

// Store those bytes into the block's row of 16 * BITS bytes, at byte 2 * BITS * j
// (3 bits: 48 bits at byte 6j as a dword and a ushort, both 2-byte aligned).
template <int BITS, typename Ptr>
__device__ __forceinline__ void store_lane_packed(Ptr row, uint32_t lo, uint32_t hi, int j) {
    if constexpr (BITS == 4) {
        *reinterpret_cast<uint2 *>(row + 8 * j) = make_uint2(lo, hi);
    } else if constexpr (BITS == 2) {
        *reinterpret_cast<uint32_t *>(row + 4 * j) = lo;
    } else {
        // (even j: dword then ushort; odd j: ushort then dword)
        auto d = row + 6 * j;
        const bool odd = j & 1;
        *reinterpret_cast<uint16_t *>(d + (odd ? 0 : 4)) = (uint16_t)(odd ? lo : hi);
        *reinterpret_cast<uint32_t *>(d + (odd ? 2 : 0)) = odd ? ((lo >> 16) | (hi << 16)) : lo;
    }
}

}  // namespace tq
