// Helpers shared by the vector-ALU and the matrix-core decode kernels.
#pragma once

#include <float.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

enum { MODE_DENSE = 0, MODE_SCORE = 1, MODE_GATED = 2 };

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    x = fmaxf(x, dpp<kDppRor4>(x));
    x = fmaxf(x, dpp<kDppRor8>(x));
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppRor4>(x);
    x += dpp<kDppRor8>(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// 2^(a - b) with the -inf conventions of an online softmax (0 when a is -inf).
__device__ __forceinline__ float exp2_diff(float a, float b) {
    return a == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(a - b);
}

// y = H x for one 128-vector held two elements per lane (x0 = x[lane],
// x1 = x[lane + 64]), H the unnormalised Sylvester Hadamard matrix in natural
// order: element bit 6 in registers, bits 0..5 across lanes.  On return
// x0 = y[lane], x1 = y[lane + 64].
__device__ __forceinline__ void hadamard128(float &x0, float &x1, int lane) {
    float a0 = x0 + x1, a1 = x0 - x1;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(a0, m), p1 = __shfl_xor(a1, m);
        const bool hi = lane & m;
        a0 = hi ? p0 - a0 : a0 + p0;
        a1 = hi ? p1 - a1 : a1 + p1;
    }
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
__device__ __forceinline__ int page_of(const int32_t *__restrict__ btab, const FastDiv &bsdiv, int t, int end) {
    return t < end ? btab[fdiv((uint32_t)t, bsdiv)] : 0;
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
