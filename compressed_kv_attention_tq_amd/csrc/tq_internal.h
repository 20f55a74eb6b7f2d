// Internal interface between the C-ABI host layer (tq_api.cpp) and the HIP
// kernels (tq_quant.hip, tq_decode.hip).  Kernel arguments are plain structs
// passed by value; nothing here allocates.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

// n / d for 32-bit n by one multiply-high and shift: m = ceil(2^(31 + l) / d),
// l = ceil(log2 d), q = umulhi(n, m) >> (l - 1).  Exact for n, d < 2^31: the
// rounding of m adds less than 1/d to n / d.  d = 1 uses m = 0, s = 0 and adds n
// back (one = all ones), so the device code has no branch.  The magic numbers
// are formed on the host and travel in the kernel arguments.
struct FastDiv {
    uint32_t m, s, one;
};
inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    if (d <= 1) {
        f.m = 0;
        f.s = 0;
        f.one = 0xFFFFFFFFu;
        return f;
    }
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    f.m = (uint32_t)(((1ull << (31 + l)) + d - 1) / d);
    f.s = l - 1;
    f.one = 0;
    return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    return (__umulhi(n, f.m) + (n & f.one)) >> f.s;
}

constexpr int kD = 128;            // elements per block
constexpr int kWaves = 8;          // decode: waves per pass block
constexpr int kBlock = 64 * kWaves;// decode: threads per pass block
constexpr int kSlice = 64;         // decode: tokens a wave scores at once (one per lane);
                                   //         also the sparse-V gating tile
constexpr int kChunkUnit = kBlock; // decode: chunks are multiples of this many tokens
constexpr int kMW = 4;             // decode, matrix-core path: waves per block
constexpr int kMBlock = 64 * kMW;  //   threads per block; chunks are multiples of kMBlock tokens
constexpr int kLutMax = 256;       // quantize: max entries of the encode lookup table
constexpr int kMaxListChunks = 1024;   // decode: chunks per sequence a work list covers
constexpr int64_t kMaxListItems = 4 << 20;   //   and (chunk, unit) items
constexpr int kListParts = 16;     // decode: work-list partitions, one item counter each
constexpr int kCtrlLine = 64;      //   words between counters (one 256-byte line each)
constexpr int kCtrlCount = 2 * kListParts * kCtrlLine;   //   word holding the item count
constexpr int kCtrlWords = kCtrlCount + 64;   // control words before the sorted units
constexpr int kListDouble = 1 << 30;   // decode: work-list flag of an item of two chunks

// One side of a quantize launch.
struct QuantSide {
    const uint16_t *src;      // float16 bits [n_tokens][n_kv][128], token stride src_stride
    uint8_t *codes;
    float *norms;
    const uint32_t *signs;    // [n_kv][4]
    int64_t src_stride;       // elements between tokens
    int64_t n_vec;            // n_tokens * n_kv
    int32_t n_tokens;
    int64_t cap;              // slots of the cache (n_blocks * block_size): larger slots are skipped
    int32_t gpw;              // groups of 8 vectors per wave (consecutive), or 0: grid stride
                              // (> 0 only where each lane's head stays fixed: n_kv | 8, or
                              // n_kv | 16 on a side for the matrix-core transform)
    int32_t n_kv;
    int32_t block_size;
    int32_t bits;
    FastDiv bs_div;           // division by block_size
    FastDiv kv_div;           // division by n_kv
    int32_t lut_half;         // table index = floor(t) + lut_half
    float grid;               // t = y * grid (cells of width 1/grid in y)
    int32_t n_bnd;            // 2^bits - 1
    float bnd[TQ_MAX_LEVELS - 1];
    // kept channels (0: none): uint8 [n_kv][16] channel lists, float16 values
    // [n_blocks][n_kv][n_out][block_size]
    int32_t n_out;
    const uint8_t *out_idx;
    uint16_t *outliers;
};

struct QuantArgs {
    QuantSide side[2];        // [0] = K, [1] = V (a side with n_vec == 0 is skipped)
    const int64_t *slots;
    int32_t blocks_k;         // blocks [0, blocks_k) do side 0, the rest side 1
};

struct DequantArgs {
    const uint8_t *codes;
    const float *norms;
    const uint32_t *signs;
    const int64_t *slots;
    void *dst;
    int64_t n_vec;
    int64_t cap;              // slots of the cache: a slot outside [0, cap) reads as zeros
    int32_t n_kv;
    int32_t block_size;
    int32_t dst_fp16;
    FastDiv kv_div, bs_div;   // division by n_kv, block_size
    float cent[TQ_MAX_LEVELS];
    int32_t n_out;            // kept channels (0: none), as in QuantSide
    const uint8_t *out_idx;
    const uint16_t *outliers;
};

// Decode attention.
struct DecodeArgs {
    const uint8_t *k_codes;
    const float *k_norms;
    const uint8_t *v_codes;
    const float *v_norms;
    const uint32_t *k_signs;
    const uint32_t *v_signs;
    const uint16_t *q;        // float16 [S][n_qtok][H_q][128 nb]
    const int32_t *seq_lens;
    const int32_t *block_table;
    float *out;
    // workspace sections
    float *qrot;              // [S][n_kv][128][RP]   rotated, scaled queries
    float *part_ml;           // [S][n_kv][n_chunks][RP][nb][2]  (max, sum) per chunk, log2 domain
    float *part_acc;          // [S][n_kv][n_chunks][RP][acc_w] rotated-domain V accumulators
                              // ([nb][128], then 16 kept-channel sums)
    float *tilemax;           // [S][n_kv][n_tiles][RP]  (sparse only)
    float *stats;             // [S][n_kv][RP][2]  global (max, sum) (sparse only)
    int32_t n_seqs, n_qtok, n_q_heads, n_kv, group, rows, rows_pad;
    int32_t max_blocks, block_size;
    int32_t max_page;         // largest physical page of the smaller cache (n_blocks - 1)
    int32_t chunk;            // tokens per chunk (multiple of kChunkUnit)
    int32_t n_chunks;         // chunks per sequence capacity
    int32_t n_tiles;          // tiles per sequence capacity
    float qscale;             // softmax_scale * log2(e) / sqrt(128)
    FastDiv bs_div, chunk_div, units_div, kv_div, grp_div, qh_div, qt_div;
                              // by block_size, chunk, n_seqs * n_kv, n_kv, group, n_q_heads, n_qtok
    float tau;
    int32_t k_bits, v_bits;
    int32_t nb, nb_log2;      // 128-element blocks per head (1, 2, 4; matrix-core path only)
    int32_t n_out;            // V channels kept in float16 (0: none; matrix-core path, nb = 1)
    const uint8_t *v_out_idx; // uint8 [n_kv][16] kept channels of each head
    const uint16_t *v_outliers;   // float16 [n_blocks][n_kv][n_out][block_size] kept values
    int32_t acc_w;            // floats per row of a chunk partial: 128 nb, + 16 with kept channels
    // fused append (matrix-core pass, nb = 1, no kept channels): the float16 K / V rows
    // of the new tokens, [n_seqs * n_qtok][n_kv][128] with new_stride elements between
    // tokens; token j of sequence b goes to position seq_len - n_qtok + j
    int32_t append;
    const uint16_t *k_new, *v_new;
    int64_t new_stride;
    uint8_t *k_codes_w, *v_codes_w;   // the caches written by the append (same memory)
    float *k_norms_w, *v_norms_w;
    float kbnd[TQ_MAX_LEVELS - 1], vbnd[TQ_MAX_LEVELS - 1];   // boundaries, unused entries +inf
    int32_t mfma;             // 1: matrix-core pass kernels, 0: vector-ALU kernels
    unsigned long long *v_rows_read;   // null, or a device counter: the gated pass adds the V
                                       // code rows it reads (one atomic per wave that read any)
    int32_t contig;           // matrix-core path: every 64-token slice lies in one page
    // Persistent matrix-core passes: a control block and work list in the workspace
    // (null: no list).  ctrl[(pass * kListParts + p) * kCtrlLine]: the item counter
    // of partition p of the first pass (dense or scoring, pass 0) or the gated pass
    // (1); ctrl[kCtrlCount]: items in the list; from word kCtrlWords: the units
    // sorted by decreasing chunk count, then the list of (chunk, unit) items,
    // c * n_seqs * n_kv + unit, chunk-major.  Partition p holds the items
    // t = p, p + kListParts, ...
    uint32_t *ctrl;
    int32_t persist;          // per launch: 1 = blocks take items from the list
    int32_t pass_slot;        // per launch: the ctrl counter this pass takes items from
    int32_t pair;             // work list: pairs of chunks form one item (then the single
                              // last chunks of odd-count units), the library's chunk halved
    int32_t merge_step;       // merge: chunk slots between partials (2 after a paired list)
    int32_t gate_pairs;       // sparse, one block per item: the gated pass takes pairs of the
                              // scoring pass's chunks (chunks sized for three scoring blocks per CU)
    float kc[TQ_MAX_LEVELS];
    float vc[TQ_MAX_LEVELS];
};

// Centroid-pair tables of the matrix-core decode pass, formed on the host:
// entry e = (c[e mod 2^b] | c[e div 2^b] << 16) as fp16 bits (codes of two
// consecutive positions, or of two tokens at one position).
struct PairTables {
    uint32_t k[1 << (2 * 4)];
    uint32_t v[1 << (2 * 4)];
};

__host__ __device__ inline uint32_t half2_bits(float lo, float hi) {
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Launchers (return hipSuccess or the launch error).
hipError_t launch_quantize(const QuantArgs &a, int blocks_total, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs &a, int bits, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, const PairTables &pt, hipStream_t s, hipEvent_t ev_before = nullptr,
                         hipEvent_t ev_after = nullptr);

}  // namespace tq
