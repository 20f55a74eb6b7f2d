// Quantize-on-append and dequantize kernels (gfx950).
//
// Per 128-element block (see tq_device.h for the 8-lanes-per-block layout):
//   load 16 float16 per lane, flip signs (s of the KV head) in the float16
//   domain, sum of squares with v_dot2_f32_f16, 8-lane DPP reduction -> norm,
//   Walsh-Hadamard transform (4 in-register stages + 3 DPP stages), scale to
//   the encode grid, encode with a small LDS table, bit-pack, store.
// When the KV heads (sub-heads of wide heads) divide 16 and no channels are kept
// the transform runs on the matrix cores instead, 16 vectors per tile
// (quant_side_mx below): same encode table and cache layout, about 45% fewer
// vector instructions.
// Sources: [TQ blog] 3.2 (signs then Hadamard, fast transform), [TQ blog] 3.3
// (Lloyd-Max codebook), [TQ+ README] quantization-types note (128-element
// blocks) and backend table (SET_ROWS quantize-on-append).
#include <float.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct LutEntry {
    float thr;      // boundary * grid inside this cell, or FLT_MAX if none
    int32_t base;   // number of boundaries entirely below the cell
};

// Encode table over cells [g, g+1) of t = y * grid, extended by a margin on both
// sides.  The host picks grid so that no two boundaries fall in one extended
// cell; then code(t) = base + (t > thr) for every t that floors to g.
__device__ void build_lut(const QuantSide &p, LutEntry *lut) {
    const int n = 2 * p.lut_half + 1;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const float g = (float)(e - p.lut_half);
        const float lo = g - 1e-3f, hi = g + 1.0f + 1e-3f;
        int base = 0;
        float thr = FLT_MAX;
        for (int b = 0; b < p.n_bnd; ++b) {
            const float bt = p.bnd[b] * p.grid;
            if (bt < lo) ++base;
            else if (bt < hi) thr = bt;
        }
        lut[e].thr = thr;
        lut[e].base = base;
    }
}

// OUTL: the side keeps p.n_out channels per head in float16 ([llama-tq] V with
// outlier-channel separation): they are zeroed before the norm and the rotation,
// and lane j stores the values of slots 2j and 2j + 1.
template <int BITS, bool OUTL>
__device__ __forceinline__ void quant_side(const QuantSide &p, const int64_t *__restrict__ slots,
                                           LutEntry *lut, int blk, int nblk) {
    const Lane8 L = lane8();
    const int j = L.j;
    const int wpb = blockDim.x >> 6;
    const int wave_id = __builtin_amdgcn_readfirstlane(blk * wpb + (int)(threadIdx.x >> 6));   // uniform
    // Groups of 8 vectors: with gpw > 0 (n_kv divides 8) the wave takes gpw
    // consecutive groups, so a block writes whole, line-aligned runs of every
    // head's code rows and no cache line of codes is shared with another block;
    // otherwise the grid stride (in blocks) is a multiple of n_kv.  Either way
    // the head of this lane's vector never changes and the token advances by a
    // constant per group.
    int first, step, n_groups;
    if (p.gpw > 0) {
        first = wave_id * p.gpw * 8;
        step = 8;
        n_groups = first < p.n_vec ? (int)min<int64_t>(p.gpw, (p.n_vec - first + 7) / 8) : 0;
    } else {
        first = wave_id * 8;
        step = nblk * wpb * 8;
        n_groups = first < p.n_vec ? (int)((p.n_vec - first + step - 1) / step) : 0;
    }
    n_groups = __builtin_amdgcn_readfirstlane(n_groups);   // uniform: the loop is scalar control flow
    const int v0 = first + L.vin;
    const int tok0 = (int)fdiv((uint32_t)v0, p.kv_div);
    const int head = v0 - tok0 * p.n_kv;
    const int tok_step = (int)fdiv((uint32_t)step, p.kv_div);
    const FastDiv bsdiv = p.bs_div;

    // Sign flips of this lane's 16 elements as float16 sign-bit masks (a float16
    // side, BITS = 16, has no signs: its rows are stored as they come).
    const uint32_t sb = BITS == 16 ? 0u : (p.signs[head * 4 + (j >> 1)] >> ((j & 1) * 16)) & 0xFFFFu;
    uint32_t smask[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        smask[k] = (((sb >> (2 * k)) & 1u) << 15) | (((sb >> (2 * k + 1)) & 1u) << 31);

    // kept channels: and-masks of this lane's float16 pairs, and its two slots' channels
    uint32_t keep[8];
    int oc0 = 0, oc1 = 0;
    if constexpr (OUTL) {
        const uint4 iw = *reinterpret_cast<const uint4 *>(p.out_idx + head * 16);
        const uint32_t words[4] = {iw.x, iw.y, iw.z, iw.w};
        uint32_t om = 0;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const uint32_t c = (words[s >> 2] >> (8 * (s & 3))) & 127u;
            if (s < p.n_out && (int)(c >> 4) == j) om |= 1u << (c & 15u);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            keep[k] = (((om >> (2 * k)) & 1u) ? 0u : 0xFFFFu) | (((om >> (2 * k + 1)) & 1u) ? 0u : 0xFFFF0000u);
        oc0 = (int)((words[j >> 1] >> (16 * (j & 1))) & 127u);
        oc1 = (int)((words[j >> 1] >> (16 * (j & 1) + 8)) & 127u);
    }

    const float kscale = lane_sign(j) * p.grid * 0.088388347648318440550f;   // grid / sqrt(128)
    const uint16_t *src = p.src + (int64_t)head * kD + j * 16;
    const uint16_t *vsrc = p.src + (int64_t)head * kD;   // the vector's first element
    const LutEntry *lut0 = lut + p.lut_half;

    // One group = 8 vectors (one per 8-lane block of the wave).  Two groups'
    // loads are in flight while one is encoded: every load is issued (past the
    // wave's groups, from its last group's rows: cached and never stored), and the
    // loop exits only at the top, so a wait never covers the group loading behind it.
    struct Group {
        uint32_t w[8];
        uint32_t o;       // OUTL: the float16 values of slots 2j, 2j + 1
        int64_t slot;
    };
    // past the wave's last group a load re-reads that group's rows (cached)
    const int tok_last = tok0 + max(n_groups - 1, 0) * tok_step;
    auto load = [&](Group &gr, int tk) __attribute__((always_inline)) {
        const int t = min(min(tk, tok_last), p.n_tokens - 1);
        const uint4 *sp = reinterpret_cast<const uint4 *>(src + (int64_t)t * p.src_stride);
        const uint4 a = sp[0], b = sp[1];
        gr.w[0] = a.x; gr.w[1] = a.y; gr.w[2] = a.z; gr.w[3] = a.w;
        gr.w[4] = b.x; gr.w[5] = b.y; gr.w[6] = b.z; gr.w[7] = b.w;
        if constexpr (OUTL) {
            const uint16_t *vp = vsrc + (int64_t)t * p.src_stride;
            gr.o = (uint32_t)vp[oc0] | ((uint32_t)vp[oc1] << 16);
        }
        gr.slot = slots[t];
    };
    auto encode = [&](const Group &gr, int g0) __attribute__((always_inline)) {
        const bool valid = g0 + L.vin < p.n_vec;
        if constexpr (BITS == 16) {
            const int64_t slot = gr.slot;
            if (valid && slot >= 0 && slot < p.cap) {
                const uint32_t blk_id = fdiv((uint32_t)slot, bsdiv);
                const uint32_t off = (uint32_t)slot - blk_id * (uint32_t)p.block_size;
                const int64_t row = ((int64_t)blk_id * p.n_kv + head) * p.block_size + off;
                uint4 *d = reinterpret_cast<uint4 *>(p.codes + row * 256 + 32 * j);
                d[0] = make_uint4(gr.w[0], gr.w[1], gr.w[2], gr.w[3]);
                d[1] = make_uint4(gr.w[4], gr.w[5], gr.w[6], gr.w[7]);
            }
            return;
        }
        uint32_t w[8];
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            w[k] = (OUTL ? gr.w[k] & keep[k] : gr.w[k]) ^ smask[k];
            const half2_t h = __builtin_bit_cast(half2_t, w[k]);
            ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        }
        ss = block8_sum(ss);
        const bool finite = ss <= FLT_MAX;   // false for inf and NaN
        if (!finite) {
#pragma unroll
            for (int k = 0; k < 8; ++k) w[k] = 0;
        }
        const float tscale = (finite && ss > 0.f) ? kscale * __frsqrt_rn(ss) : 0.f;

        // first Hadamard stage straight from the float16 pairs, then the rest
        float v[16];
#pragma unroll
        for (int k = 0; k < 8; ++k) half_pair_butterfly(w[k], v[2 * k], v[2 * k + 1]);
        wht16<2>(v);
        wht_cross(v, j);

        uint32_t code[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float t = v[k] * tscale;
            const LutEntry e = lut0[cvt_floor(t)];
            code[k] = (uint32_t)e.base + (t > e.thr ? 1u : 0u);
        }

        const int64_t slot = gr.slot;
        if (valid && slot >= 0 && slot < p.cap) {
            const uint32_t blk_id = fdiv((uint32_t)slot, bsdiv);
            const uint32_t off = (uint32_t)slot - blk_id * (uint32_t)p.block_size;
            const int64_t row = ((int64_t)blk_id * p.n_kv + head) * p.block_size + off;
            uint8_t *dst = p.codes + row * (16 * BITS);
            if constexpr (BITS == 4) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) lo |= code[k] << (4 * k);
#pragma unroll
                for (int k = 0; k < 8; ++k) hi |= code[8 + k] << (4 * k);
                *reinterpret_cast<uint2 *>(dst + 8 * j) = make_uint2(lo, hi);
            } else if constexpr (BITS == 2) {
                uint32_t x = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) x |= code[k] << (2 * k);
                *reinterpret_cast<uint32_t *>(dst + 4 * j) = x;
            } else {  // 3 bits: 48 bits at byte 6j
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    if (3 * k + 3 <= 32) lo |= code[k] << (3 * k);
                    else if (3 * k >= 32) hi |= code[k] << (3 * k - 32);
                    else { lo |= code[k] << (3 * k); hi |= code[k] >> (32 - 3 * k); }
                }
                // (even j: dword then ushort; odd j: ushort then dword, both 2-aligned)
                uint8_t *d = dst + 6 * j;
                const bool odd = j & 1;
                *reinterpret_cast<uint16_t *>(d + (odd ? 0 : 4)) = (uint16_t)(odd ? lo : hi);
                *reinterpret_cast<uint32_t *>(d + (odd ? 2 : 0)) = odd ? ((lo >> 16) | (hi << 16)) : lo;
            }
            if (j == 0) p.norms[row] = __fsqrt_rn(ss);
            if constexpr (OUTL) {   // [page][head][slot][block_size]
                uint16_t *od = p.outliers + ((int64_t)blk_id * p.n_kv + head) * p.n_out * p.block_size + off;
                if (2 * j < p.n_out) od[(2 * j) * p.block_size] = (uint16_t)(gr.o & 0xFFFFu);
                if (2 * j + 1 < p.n_out) od[(2 * j + 1) * p.block_size] = (uint16_t)(gr.o >> 16);
            }
        }
    };

    // kDepth groups in flight: each encode is followed by the load of the group
    // kDepth ahead
    constexpr int kDepth = 2;
    Group gr[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        __builtin_amdgcn_sched_barrier(0);
        load(gr[d], tok0 + d * tok_step);
    }
    // the encode table is built while the first groups load
    if constexpr (BITS != 16) {
        build_lut(p, lut);
        __syncthreads();
    }
    int tok = tok0;
    for (int i = 0; i < n_groups; i += kDepth, tok += kDepth * tok_step) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            encode(gr[d], first + (i + d) * step);   // (past the end: no lane stores)
            load(gr[d], tok + (kDepth + d) * tok_step);
        }
    }
}

// --------------------------------------------------------------------------
// The same quantizer with the Walsh-Hadamard transform on the matrix cores
// ([TQ blog] 3.2: the rotation is a +-1 diagonal followed by a Hadamard matrix;
// here the Hadamard product itself is a dense 128 x 128 contraction with exact
// +-1 operands and float32 accumulation).
//
// A wave takes tiles of 16 vectors.  Y = H X' (X' = the sign-flipped float16
// vectors, one per column) runs as 8 output tiles x 4 k-steps of
// v_mfma_f32_16x16x32_f16.  Rows and columns of H are taken in an order that
// makes the lane layouts line up with no data movement:
//   input  element c = i + 8 s + 32 g   (lane group g = lane >> 4, k-step s,
//                                        register element i = 0..7)
//   output element r = jj + 4 t + 32 g  (output tile t, accumulator jj = 0..3)
// so lane (g, n) loads the 64-byte quarter g of vector n (four 16-byte loads)
// and receives the 32 consecutive output elements of that same quarter, which it
// encodes, bit-packs and stores by itself (4·BITS bytes at byte 4·BITS·g of the
// code row).  With that order, bit by bit,
//   popcount(r & c) = (m0 i0 + m1 i1 + m2 g0 + m3 g1) + t0 i2 + (t1 s0 + t2 s1)
// (m = 4 g' + jj the A-tile row, g' the row's group), so every A tile is one of
// two base tiles (t0 = 0 / 1, differing by the sign of i2) times a scalar sign
// (-1)^popcount((t >> 1) & s): four constant operands in all.
// --------------------------------------------------------------------------
typedef _Float16 qh8_t __attribute__((ext_vector_type(8)));
typedef float qf4_t __attribute__((ext_vector_type(4)));
typedef uint32_t qu4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ qf4_t mfma_16x16x32(qu4_t a, qu4_t b, qf4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(qh8_t, a), __builtin_bit_cast(qh8_t, b), c,
                                                  0, 0, 0);
}

// A operand (lane: row m = lane & 15, k = 8 (lane >> 4) + i) of the base tile t0
// = odd, negated when neg: entries (-1)^(m0 i0 + m1 i1 + m2 g0 + m3 g1 + odd i2) as
// float16 +-1.
__device__ __forceinline__ qu4_t hadamard_operand(int lane, int odd, int neg) {
    const int m = lane & 15, g = lane >> 4;
    const int row = (__popc((m >> 2) & g) + neg) & 1;
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 2 * d + h;
            const int sg = (row + __popc((m & 3) & (i & 3)) + odd * (i >> 2)) & 1;
            word |= (sg ? 0xBC00u : 0x3C00u) << (16 * h);
        }
        w[d] = word;
    }
    return qu4_t{w[0], w[1], w[2], w[3]};
}

// Requires n_kv | 16 (the host sets p.gpw > 0 for such a side): a tile of 16
// consecutive vectors then holds whole tokens, so the KV head of each lane's vector
// is fixed for the wave.
template <int BITS>
__device__ __forceinline__ void quant_side_mx(const QuantSide &p, const int64_t *__restrict__ slots, LutEntry *lut,
                                              int blk) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int wpb = blockDim.x >> 6;
    const int wave_id = __builtin_amdgcn_readfirstlane(blk * wpb + (int)(threadIdx.x >> 6));
    const int first = wave_id * p.gpw * 8;   // a multiple of 32 vectors
    int n_tiles = first < p.n_vec ? (int)min<int64_t>(p.gpw / 2, (p.n_vec - first + 15) / 16) : 0;
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
    const int v0 = first + n;
    const int tok0 = (int)fdiv((uint32_t)v0, p.kv_div);
    const int head = v0 - tok0 * p.n_kv;
    const int tok_step = (int)fdiv(16u, p.kv_div);
    const FastDiv bsdiv = p.bs_div;

    // sign flips of the lane's 32 elements (one sign word): float16 sign-bit masks
    // of its 16 float16 pairs, pair d of k-step s = elements 32g + 8s + 2d, +1
    const uint32_t sb = p.signs[head * 4 + g];
    uint32_t smask[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int d = 0; d < 4; ++d)
            smask[s][d] = (((sb >> (8 * s + 2 * d)) & 1u) << 15) | (((sb >> (8 * s + 2 * d + 1)) & 1u) << 31);
    const qu4_t hop[2][2] = {{hadamard_operand(lane, 0, 0), hadamard_operand(lane, 0, 1)},
                             {hadamard_operand(lane, 1, 0), hadamard_operand(lane, 1, 1)}};

    const float kscale = p.grid * 0.088388347648318440550f;   // grid / sqrt(128)
    const uint16_t *src = p.src + (int64_t)head * kD + 32 * g;
    const LutEntry *lut0 = lut + p.lut_half;

    struct Tile {
        qu4_t x[4];
        int64_t slot;
    };
    const int tok_last = tok0 + max(n_tiles - 1, 0) * tok_step;
    auto load = [&](Tile &tl, int tk) __attribute__((always_inline)) {
        const int t = min(min(tk, tok_last), p.n_tokens - 1);
        const qu4_t *sp = reinterpret_cast<const qu4_t *>(src + (int64_t)t * p.src_stride);
#pragma unroll
        for (int s = 0; s < 4; ++s) tl.x[s] = sp[s];
        tl.slot = slots[t];
    };
    auto encode = [&](const Tile &tl, int vt) __attribute__((always_inline)) {
        qu4_t xs[4];
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                xs[s][d] = tl.x[s][d] ^ smask[s][d];
                const half2_t h = __builtin_bit_cast(half2_t, (uint32_t)xs[s][d]);
                ss = __builtin_amdgcn_fdot2(h, h, ss, false);
            }
        }
        // the four quarters of vector n sit in lanes n, n + 16, n + 32, n + 48
        {
            const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
            ss = __uint_as_float(a[0]) + __uint_as_float(a[1]);
            const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
            ss = __uint_as_float(b[0]) + __uint_as_float(b[1]);
        }
        const bool finite = ss <= FLT_MAX;   // false for inf and NaN
        if (__builtin_amdgcn_ballot_w64(!finite)) {   // (rare: a scalar branch around it)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (!finite) xs[s] = qu4_t{0u, 0u, 0u, 0u};
        }
        const float tscale = (finite && ss > 0.f) ? kscale * __frsqrt_rn(ss) : 0.f;

        uint32_t pk[BITS];
#pragma unroll
        for (int w = 0; w < BITS; ++w) pk[w] = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            // (the k-steps start at s = t >> 1, so no two tiles share a partial sum:
            // shared partials would keep more accumulators live at once)
            qf4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int s = ((t >> 1) + k) & 3;
                acc = mfma_16x16x32(hop[t & 1][__popc((t >> 1) & s) & 1], xs[s], acc);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float tv = acc[jj] * tscale;
                const LutEntry e = lut0[cvt_floor(tv)];
                const uint32_t code = (uint32_t)e.base + (tv > e.thr ? 1u : 0u);
                const int bit = BITS * (4 * t + jj);   // compile-time
                const int wd = bit >> 5, off = bit & 31;
                pk[wd] |= code << off;
                if (off + BITS > 32) pk[wd + 1] |= code >> (32 - off);
            }
            // pack each tile's codes now: left to the store, the compiler sinks every
            // table entry and scaled value into it and holds all 32 at once
#pragma unroll
            for (int w = 0; w < BITS; ++w) asm volatile("" : "+v"(pk[w]));
        }

        const int64_t slot = tl.slot;
        if (vt + n < p.n_vec && slot >= 0 && slot < p.cap) {
            const uint32_t blk_id = fdiv((uint32_t)slot, bsdiv);
            const uint32_t off = (uint32_t)slot - blk_id * (uint32_t)p.block_size;
            const int64_t row = ((int64_t)blk_id * p.n_kv + head) * p.block_size + off;
            uint8_t *dst = p.codes + row * (16 * BITS) + 4 * BITS * g;
            if constexpr (BITS == 4) {
                *reinterpret_cast<uint4 *>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            } else if constexpr (BITS == 2) {
                *reinterpret_cast<uint2 *>(dst) = make_uint2(pk[0], pk[1]);
            } else {   // 12 bytes at byte 12 g (4-byte aligned)
                uint32_t *d = reinterpret_cast<uint32_t *>(dst);
                d[0] = pk[0];
                d[1] = pk[1];
                d[2] = pk[2];
            }
            if (g == 0) p.norms[row] = __fsqrt_rn(ss);
        }
    };

    // One tile in flight: a tile's loads are issued when the previous tile has been
    // encoded.  Every wave of the call is resident at once (4 per SIMD), so the
    // memory system sees the first tiles of all waves before any second tile, and
    // the waves whose first data lands early compute while the rest still load
    // (measured 2-5% faster than issuing both tiles' loads at the start).
    Tile tl;
    load(tl, tok0);
    build_lut(p, lut);
    __syncthreads();
    for (int i = 0; i < n_tiles; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        encode(tl, first + i * 16);
        if (i + 1 < n_tiles) load(tl, tok0 + (i + 1) * tok_step);
    }
}

__global__ __launch_bounds__(256) void tq_quantize_kernel(QuantArgs a) {
    __shared__ LutEntry lut[kLutMax];   // built inside quant_side, once its first loads are out
    const bool second = (int)blockIdx.x >= a.blocks_k;
    const QuantSide &p = second ? a.side[1] : a.side[0];
    const int blk = second ? (int)blockIdx.x - a.blocks_k : (int)blockIdx.x;
    const int nblk = second ? (int)gridDim.x - a.blocks_k : a.blocks_k;
    if (p.n_out == 0 && p.gpw > 0 && p.bits != 16) {   // n_kv | 16: tiles of 16 vectors on the matrix cores
        switch (p.bits) {
            case 2: quant_side_mx<2>(p, a.slots, lut, blk); break;
            case 3: quant_side_mx<3>(p, a.slots, lut, blk); break;
            default: quant_side_mx<4>(p, a.slots, lut, blk); break;
        }
        return;
    }
    if (p.n_out > 0) {   // kept channels (compressed sides only)
        switch (p.bits) {
            case 2: quant_side<2, true>(p, a.slots, lut, blk, nblk); break;
            case 3: quant_side<3, true>(p, a.slots, lut, blk, nblk); break;
            default: quant_side<4, true>(p, a.slots, lut, blk, nblk); break;
        }
        return;
    }
    switch (p.bits) {
        case 2: quant_side<2, false>(p, a.slots, lut, blk, nblk); break;
        case 3: quant_side<3, false>(p, a.slots, lut, blk, nblk); break;
        case 16: quant_side<16, false>(p, a.slots, lut, blk, nblk); break;   // float16 side
        default: quant_side<4, false>(p, a.slots, lut, blk, nblk); break;
    }
}

// --------------------------------------------------------------------------
// Dequantize: x_hat = n * s * (H c[code]) / sqrt(128), same lane layout.
// --------------------------------------------------------------------------
// A float16 side: the rows as stored (float16 or widened to float32).
__global__ __launch_bounds__(256) void tq_dequantize_fp16_kernel(DequantArgs a) {
    const Lane8 L = lane8();
    const int j = L.j;
    const int wpb = blockDim.x >> 6;
    const int wave_id = blockIdx.x * wpb + (int)(threadIdx.x >> 6);
    const int step = gridDim.x * wpb * 8;
    for (int g0 = wave_id * 8; g0 < a.n_vec; g0 += step) {
        const int vid = g0 + L.vin;
        if (vid >= a.n_vec) continue;
        const int tok = (int)fdiv((uint32_t)vid, a.kv_div);
        const int head = vid - tok * a.n_kv;
        // (a slot outside the cache reads as a row of zeros)
        const int64_t sl = a.slots[tok];
        uint4 x0 = make_uint4(0u, 0u, 0u, 0u), x1 = x0;
        if (sl >= 0 && sl < a.cap) {
            const uint32_t slot = (uint32_t)sl;
            const uint32_t blk_id = fdiv(slot, a.bs_div);
            const uint32_t off = slot - blk_id * (uint32_t)a.block_size;
            const int64_t row = ((int64_t)blk_id * a.n_kv + head) * a.block_size + off;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.codes + row * 256 + 32 * j);
            x0 = src[0];
            x1 = src[1];
        }
        const int64_t dbase = ((int64_t)tok * a.n_kv + head) * kD + 16 * j;
        if (a.dst_fp16) {
            uint4 *d = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.dst) + dbase);
            d[0] = x0;
            d[1] = x1;
        } else {
            const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            float o[16];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const half2_t h = __builtin_bit_cast(half2_t, w[k]);
                o[2 * k] = (float)h.x;
                o[2 * k + 1] = (float)h.y;
            }
            float4 *d = reinterpret_cast<float4 *>(static_cast<float *>(a.dst) + dbase);
            d[0] = make_float4(o[0], o[1], o[2], o[3]);
            d[1] = make_float4(o[4], o[5], o[6], o[7]);
            d[2] = make_float4(o[8], o[9], o[10], o[11]);
            d[3] = make_float4(o[12], o[13], o[14], o[15]);
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void tq_dequantize_kernel(DequantArgs a) {
    __shared__ float ctab[TQ_MAX_LEVELS];
    if (threadIdx.x < TQ_MAX_LEVELS) ctab[threadIdx.x] = a.cent[threadIdx.x];
    __syncthreads();
    const Lane8 L = lane8();
    const int j = L.j;
    const int wpb = blockDim.x >> 6;
    const int wave_id = blockIdx.x * wpb + (int)(threadIdx.x >> 6);
    const int step = gridDim.x * wpb * 8;
    const float lsign = lane_sign(j) * 0.088388347648318440550f;
    const FastDiv kvdiv = a.kv_div;
    const FastDiv bsdiv = a.bs_div;
    for (int g0 = wave_id * 8; g0 < a.n_vec; g0 += step) {
        const int vid = g0 + L.vin;
        const bool valid = vid < a.n_vec;
        const int tok = valid ? (int)fdiv((uint32_t)vid, kvdiv) : 0;
        const int head = valid ? vid - tok * a.n_kv : 0;
        int64_t row = 0;
        uint32_t w[2] = {0, 0};
        float n = 0.f;
        // (a slot outside the cache reads as a row of zeros: norm 0, no kept values)
        const int64_t sl = valid ? a.slots[tok] : -1;
        const bool in_cache = sl >= 0 && sl < a.cap;
        if (in_cache) {
            const uint32_t slot = (uint32_t)sl;
            const uint32_t blk_id = fdiv(slot, bsdiv);
            const uint32_t off = slot - blk_id * (uint32_t)a.block_size;
            row = ((int64_t)blk_id * a.n_kv + head) * a.block_size + off;
            const uint8_t *src = a.codes + row * (16 * BITS) + 2 * BITS * j;
            if constexpr (BITS == 4) {
                const uint2 x = *reinterpret_cast<const uint2 *>(src);
                w[0] = x.x; w[1] = x.y;
            } else if constexpr (BITS == 2) {
                w[0] = *reinterpret_cast<const uint32_t *>(src);
            } else {
                if ((j & 1) == 0) {
                    w[0] = *reinterpret_cast<const uint32_t *>(src);
                    w[1] = *reinterpret_cast<const uint16_t *>(src + 4);
                } else {
                    const uint32_t lo = *reinterpret_cast<const uint16_t *>(src);
                    const uint32_t hi = *reinterpret_cast<const uint32_t *>(src + 2);
                    w[0] = lo | (hi << 16);
                    w[1] = hi >> 16;
                }
            }
            n = a.norms[row];
        }
        float v[16];
        v[0] = ctab[stream_code<BITS, 0>(w)];   v[1] = ctab[stream_code<BITS, 1>(w)];
        v[2] = ctab[stream_code<BITS, 2>(w)];   v[3] = ctab[stream_code<BITS, 3>(w)];
        v[4] = ctab[stream_code<BITS, 4>(w)];   v[5] = ctab[stream_code<BITS, 5>(w)];
        v[6] = ctab[stream_code<BITS, 6>(w)];   v[7] = ctab[stream_code<BITS, 7>(w)];
        v[8] = ctab[stream_code<BITS, 8>(w)];   v[9] = ctab[stream_code<BITS, 9>(w)];
        v[10] = ctab[stream_code<BITS, 10>(w)]; v[11] = ctab[stream_code<BITS, 11>(w)];
        v[12] = ctab[stream_code<BITS, 12>(w)]; v[13] = ctab[stream_code<BITS, 13>(w)];
        v[14] = ctab[stream_code<BITS, 14>(w)]; v[15] = ctab[stream_code<BITS, 15>(w)];
        wht16<1>(v);
        wht_cross(v, j);
        if (valid) {
            const uint32_t sw = a.signs[head * 4 + (j >> 1)] >> ((j & 1) * 16);
            const float sc = n * lsign;
            float o[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) o[k] = ((sw >> k) & 1u) ? -v[k] * sc : v[k] * sc;
            const int64_t dbase = ((int64_t)tok * a.n_kv + head) * kD + 16 * j;
            if (a.dst_fp16) {
                uint32_t h[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    half2_t x;
                    x.x = (_Float16)o[2 * k];
                    x.y = (_Float16)o[2 * k + 1];
                    h[k] = __builtin_bit_cast(uint32_t, x);
                }
                uint4 *d = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.dst) + dbase);
                d[0] = make_uint4(h[0], h[1], h[2], h[3]);
                d[1] = make_uint4(h[4], h[5], h[6], h[7]);
            } else {
                float4 *d = reinterpret_cast<float4 *>(static_cast<float *>(a.dst) + dbase);
                d[0] = make_float4(o[0], o[1], o[2], o[3]);
                d[1] = make_float4(o[4], o[5], o[6], o[7]);
                d[2] = make_float4(o[8], o[9], o[10], o[11]);
                d[3] = make_float4(o[12], o[13], o[14], o[15]);
            }
            // kept channels: their stored values over the reconstruction (this thread
            // wrote those elements above, so its later stores land last)
            const int64_t prow = a.n_out > 0 ? row / a.block_size : 0, poff = row - prow * a.block_size;
            for (int s = 0; in_cache && s < a.n_out; ++s) {
                const int c = a.out_idx[head * 16 + s] & 127;
                if ((c >> 4) != j) continue;
                const uint16_t hv = a.outliers[(prow * a.n_out + s) * a.block_size + poff];
                const int64_t di = ((int64_t)tok * a.n_kv + head) * kD + c;
                if (a.dst_fp16) static_cast<uint16_t *>(a.dst)[di] = hv;
                else static_cast<float *>(a.dst)[di] = (float)__builtin_bit_cast(_Float16, hv);
            }
        }
    }
}

hipError_t launch_quantize(const QuantArgs &a, int blocks_total, hipStream_t s) {
    hipLaunchKernelGGL(tq_quantize_kernel, dim3(blocks_total), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, int bits, hipStream_t s) {
    const int64_t waves = (a.n_vec + 7) / 8;
    int blocks = (int)((waves + 3) / 4);
    if (blocks > 65535) blocks = 65535;
    if (blocks < 1) blocks = 1;
    switch (bits) {
        case 2: hipLaunchKernelGGL(tq_dequantize_kernel<2>, dim3(blocks), dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL(tq_dequantize_kernel<3>, dim3(blocks), dim3(256), 0, s, a); break;
        case 16: hipLaunchKernelGGL(tq_dequantize_fp16_kernel, dim3(blocks), dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL(tq_dequantize_kernel<4>, dim3(blocks), dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace tq
