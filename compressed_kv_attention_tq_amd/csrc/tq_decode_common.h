// Helpers shared by the vector-ALU and the matrix-core decode kernels.
#pragma once

#include <float.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

enum { MODE_DENSE = 0, MODE_SCORE = 1, MODE_GATED = 2 };

// x of lane ^ (1 << B), B = 0..5, without LDS: DPP inside a 16-lane row (xor 4 is
// the half-row mirror, xor 7, followed by the quad reverse, xor 3), the row and
// half-wave swaps of gfx950 across rows.  A swap of x with itself returns
// (x of the even row or half, x of the odd one) in both lanes of a pair.
template <int B>
__device__ __forceinline__ float lane_xor(float x, int lane) {
    if constexpr (B == 0) {
        return dpp<kDppXor1>(x);
    } else if constexpr (B == 1) {
        return dpp<kDppXor2>(x);
    } else if constexpr (B == 2) {
        constexpr int kHalfMirror = 0x141, kQuadReverse = 0x1B;   // row_half_mirror, quad_perm [3,2,1,0]
        return dpp<kQuadReverse>(dpp<kHalfMirror>(x));
    } else if constexpr (B == 3) {
        return dpp<kDppRor8>(x);
    } else if constexpr (B == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float((lane & 32) ? r[0] : r[1]);
    }
}

// Max / sum over the 64 lanes (the row and half-wave swaps: own and partner value
// in either order, so the result is the same in every lane).
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    x = fmaxf(x, dpp<kDppRor4>(x));
    x = fmaxf(x, dpp<kDppRor8>(x));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppRor4>(x);
    x += dpp<kDppRor8>(x);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^(a - b) with the -inf conventions of an online softmax (0 when a is -inf).
__device__ __forceinline__ float exp2_diff(float a, float b) {
    return a == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(a - b);
}

// y = H x for one 128-vector held two elements per lane (x0 = x[lane],
// x1 = x[lane + 64]), H the unnormalised Sylvester Hadamard matrix in natural
// order: element bit 6 in registers, bits 0..5 across lanes.  On return
// x0 = y[lane], x1 = y[lane + 64].  Each stage forms partner + mu * mine with
// mu = -1 on the lane whose bit is set (the difference there, exact as a
// subtraction), the partner from lane_xor.
__device__ __forceinline__ void hadamard128(float &x0, float &x1, int lane) {
    float a0 = x0 + x1, a1 = x0 - x1;
    auto stage = [&](auto bit) __attribute__((always_inline)) {
        constexpr int B = decltype(bit)::value;
        const float mu = ((lane >> B) & 1) ? -1.f : 1.f;
        const float p0 = lane_xor<B>(a0, lane), p1 = lane_xor<B>(a1, lane);
        a0 = __builtin_fmaf(mu, a0, p0);
        a1 = __builtin_fmaf(mu, a1, p1);
    };
    stage(std::integral_constant<int, 0>{});
    stage(std::integral_constant<int, 1>{});
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 3>{});
    stage(std::integral_constant<int, 4>{});
    stage(std::integral_constant<int, 5>{});
    x0 = a0;
    x1 = a1;
}

// Keep a wave-uniform value in a VGPR (SGPRs are reserved for q'').
__device__ __forceinline__ float in_vgpr(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// One token's cache rows, loaded by the lane that scores it.  The physical page
// of a token is looked up one slice before its rows are loaded (page_of), so the
// block-table load never stalls the row loads.
// (the table index is clamped to the table and the page to the pool, so a bad
// entry or length reads another page, never outside the cache)
__device__ __forceinline__ int page_of(const int32_t *__restrict__ btab, const FastDiv &bsdiv, int t, int end,
                                       int last_entry, int max_page) {
    return t < end ? min(max(btab[min((int)fdiv((uint32_t)t, bsdiv), last_entry)], 0), max_page) : 0;
}

template <int KB, int VB, bool WITH_V>
struct TokenRows {
    uint4 k[KB];
    uint4 v[WITH_V ? VB : 1];
    float kn, vn;
    bool active;

    __device__ __forceinline__ void load(const uint8_t *__restrict__ k_codes, const float *__restrict__ k_norms,
                                         const uint8_t *__restrict__ v_codes, const float *__restrict__ v_norms,
                                         const FastDiv &bsdiv, int bs, int n_kv, int kv, int t, int end,
                                         int blk) {
        active = t < end;
        int64_t row = 0;
        if (active) {
            const uint32_t pg = fdiv((uint32_t)t, bsdiv);
            row = ((int64_t)blk * n_kv + kv) * bs + (t - (int)pg * bs);
        }
        const uint4 *kp = reinterpret_cast<const uint4 *>(k_codes + row * (16 * KB));
#pragma unroll
        for (int i = 0; i < KB; ++i) k[i] = kp[i];
        kn = active ? k_norms[row] : 0.f;
        if constexpr (WITH_V) {
            const uint4 *vp = reinterpret_cast<const uint4 *>(v_codes + row * (16 * VB));
#pragma unroll
            for (int i = 0; i < VB; ++i) v[i] = vp[i];
            vn = active ? v_norms[row] : 0.f;
        }
    }
};

}  // namespace tq
