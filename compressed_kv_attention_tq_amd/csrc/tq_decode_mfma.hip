// Decode attention over the compressed cache on the gfx950 matrix cores.
//
// Computes what the vector-ALU kernels compute (scores against K codes in the
// Hadamard domain without dequantizing K, online softmax in the log2 domain, V
// accumulated in the rotated domain and inverse-rotated once per row;
// [llama-tq] rotated-domain Q.K, [TQ+ README] sparse V, [TQ+ article] skipped V
// is zero), with the two contractions of each 64-token slice as 16x16x32 fp16
// MFMAs.  All query rows of one KV head (GQA group x query tokens, at most 16)
// share the slice's codes, so per slice:
//   scores  S[token][col] = sum_pos cK[token][pos] * Q[pos][col]     (K: 16 MFMAs)
//   values  A[pos][col]  += sum_tok cV[pos][tok] * P[tok][col]       (V: 16 MFMAs)
// Centroids are fp16-exact, so the code operands are exact.  The fp32 operands
// (q'' and the softmax weights) are split into fp16 hi + lo parts (w = hi + lo to
// ~2^-20 relative): with at most 8 rows the hi parts sit in columns 0-7 and the
// lo parts in columns 8-15 of one MFMA and the two column halves are summed
// afterwards; with 9-16 rows each part gets its own MFMA.
//
// Lane roles (lane l, g = l / 16, n = l % 16; checked on the hardware):
//   A operand: row m = n, k = 8g + e (e = 0..7, fp16 pairs per dword)
//   B operand: k = 8g + e, column n;   D: row 4g + e (e = 0..3), column n.
// K: A row = token 16tm + n of tile tm, k = position 32g + 8ks + e, so each lane
//    reads 4*KB contiguous code bytes of one token per tile and expands byte
//    pairs of codes with an LDS table of fp16 centroid pairs.
// V: k = token 32ks + 16(e/4) + 4g + (e%4), which is exactly the set of tokens
//    whose scores lane (g, n) holds in the K output (tiles 2ks, 2ks+1), so the
//    softmax weights feed the V MFMA's B operand without any data movement.
//    A row m = n is position 8n + j of tile j, so each lane reads the 8-position
//    unit n of 16 tokens and pairs two tokens' codes per table lookup.
//
// A block (4 waves) owns one chunk of one (sequence, KV head); each wave walks
// its own 64-token slices with private softmax state, loading the next slice's
// codes while it computes, and the block's partial goes to the workspace for the
// merge kernel.
//
// Heads of NB = head_dim / 128 > 1 blocks ([TQ+ README] types note: every format
// works on 128-element blocks) are stored as NB sub-heads, block i of head j
// being sub-head NB j + i with its own norms and sign words.  Wave w then takes
// block w % NB of the slices of its group w / NB: the NB waves of a group load
// the same tokens' codes of different blocks, each adds its block's partial scores
// (q''_i . c_i times the block's norm) to an LDS exchange, and all of them read
// back the sum in the same order, so they hold bitwise equal scores and softmax
// state; each keeps the V accumulator of its own block.  Register use is that
// of one block; the block's waves meet at two LDS barriers per slice.
//
// Fused append (a.append, dense and scoring passes, 128-wide heads, compressed K,
// V without kept channels): the new tokens of a (sequence, KV head) are its last n_qtok
// positions.  The wave that computes the slice holding a new position quantizes
// its K and V rows (the arithmetic of the quantize kernel), stores them to the
// cache for later launches and keeps a copy in LDS, which replaces their rows in
// that slice: within this launch those rows are never read back from memory, so
// no ordering of the stores against the slice loads is needed, and no other wave
// waits for the work.
//
// OV: the V side keeps n_out <= 16 channels per head in float16 ([llama-tq] V with
// outlier-channel separation).  They add one value MFMA per 32 tokens whose A
// rows are the kept channels (A[slot][token] = the stored float16 value, exact)
// and whose B operand is the softmax weight without the V norm; the 16 sums per
// row travel after the 128 rotated-domain sums and the merge writes them over
// their channels.
#include <map>
#include <mutex>
#include <utility>

#include "tq_decode_common.h"

namespace tq {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef int32_t i4_t __attribute__((ext_vector_type(4)));

constexpr int kQS = 132;   // padded row stride (floats) of the q'' / merge buffer

#ifndef TQ_DECODE_SLOTS
#define TQ_DECODE_SLOTS 2
#endif

__device__ __forceinline__ f4_t mfma_f16(u4_t a, u4_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ float half_lo(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16));
}

// One half of the fp16 split w = hi + lo of an fp32 pair: the hi pair when
// lo_sel == 0, the lo pair when lo_sel == 1.  hi is w truncated to fp16, so
// w - hi is exact in fp32 and lo holds it to fp16 precision.
__device__ __forceinline__ uint32_t split_pair(float w0, float w1, float lo_sel) {
    const uint32_t h = pk_rtz(w0, w1);
    return pk_rtz(__builtin_fmaf(-lo_sel, half_lo(h), w0), __builtin_fmaf(-lo_sel, half_hi(h), w1));
}

// Reductions over the four lane groups g (lanes n, n+16, n+32, n+48 hold one
// column): swap rows of 16 lanes, then halves of the wave.
__device__ __forceinline__ float xg_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xg_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// NW contiguous dwords (16, 12 or 8 bytes) of code bytes.
template <int NW>
__device__ __forceinline__ void load_words(const uint8_t *p, uint32_t (&w)[NW]) {
    if constexpr (NW == 4) {
        const uint4 t = *reinterpret_cast<const uint4 *>(p);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (NW == 3) {
        struct alignas(4) U3 { uint32_t x, y, z; };
        const U3 t = *reinterpret_cast<const U3 *>(p);
        w[0] = t.x; w[1] = t.y; w[2] = t.z;
    } else {
        const uint2 t = *reinterpret_cast<const uint2 *>(p);
        w[0] = t.x; w[1] = t.y;
    }
}

// A operand of the score MFMA for k-step ks from the lane's 32 positions of one
// token (positions 32g + 8ks .. +7): 4 lookups of a code pair -> fp16 pair.
// Centroid-pair tables are replicated 32 times, entry-major, and lane l reads
// copy l % 32, so the lanes of a half-wave never meet in an LDS bank whatever
// their indices.  Row e of the table area is RB bytes: copies 0..31 of K entry e,
// then (RB = 256, when the pass has V tables) copies 0..31 of V entry e.  With
// 256-byte rows, a pair index that fills a byte of a code word becomes its
// address in one byte permute: (index << 8) | lane_off.
template <int B>
constexpr int tab_copies() { return 32; }

// dword at byte offset `off` of the table area
__device__ __forceinline__ uint32_t tab_at(const uint32_t *tab, uint32_t off) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(tab) + off);
}

// table offset of a pair index: the FB-bit field at bit `sh` of u (its byte k
// when FB = 8, RB = 256 and sh = 8 k)
template <int FB, int RB>
__device__ __forceinline__ uint32_t tab_off(uint32_t u, int sh, uint32_t lane_off) {
    if constexpr (FB == 8 && RB == 256) {
        // v_perm_b32 bytes: 0 <- byte 0 of lane_off, 1 <- byte sh/8 of u, 2, 3 <- 0
        return __builtin_amdgcn_perm(u, lane_off, 0x0C0C0000u | ((4u + (uint32_t)(sh >> 3)) << 8));
    } else {
        // the field moved to bit RS by one shift, then masked and merged with the copy
        // offset in one v_and_or_b32 (left to itself the compiler spends a shift, an
        // and and an add)
        constexpr int RS = RB == 256 ? 8 : 7;
        const uint32_t moved = sh >= RS ? (u >> (sh - RS)) : (u << (RS - sh));
        uint32_t r;
        asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(moved), "s"(((1u << FB) - 1u) << RS), "v"(lane_off));
        return r;
    }
}

template <int KB, int RB>
__device__ __forceinline__ u4_t k_frag(const uint32_t (&w)[KB], int ks, const uint32_t *tab, uint32_t lane_off) {
    constexpr int FB = 2 * KB;
    uint32_t u;
    if constexpr (KB == 4) {
        u = w[ks];
    } else if constexpr (KB == 3) {
        u = ks == 0 ? w[0]
            : ks == 1 ? __builtin_amdgcn_alignbit(w[1], w[0], 24)
            : ks == 2 ? __builtin_amdgcn_alignbit(w[2], w[1], 16)
                      : (w[2] >> 8);
    } else {
        u = (ks & 1) ? (w[ks >> 1] >> 16) : w[ks >> 1];
    }
    u4_t f;
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = tab_at(tab, tab_off<FB, RB>(u, FB * k, lane_off));
    return f;
}

// Raw word of the 8-position unit n of one V row: one dword (4-bit), one ushort
// (2-bit).  3-bit units (bits [24n, 24n + 24)) come four to three dwords: lane
// n = 4a + b of a quad loads dword 3a + min(b, 2), and vunit_bits takes the
// low part of units 1 and 2 from the quad neighbour below.
template <int VB>
struct VUnit {
    uint32_t d;
};

template <int VB>
__device__ __forceinline__ void load_vunit(const uint8_t *row, int widx, VUnit<VB> &u) {
    if constexpr (VB == 2) u.d = reinterpret_cast<const uint16_t *>(row)[widx];
    else u.d = reinterpret_cast<const uint32_t *>(row)[widx];
}

// The unit's bits at bit 0 (bits above the unit are garbage); called by all lanes.
template <int VB>
__device__ __forceinline__ uint32_t vunit_bits(const VUnit<VB> &u, int o) {
    if constexpr (VB == 3) {
        constexpr int kQuadPerm0013 = 0xD0;   // quad_perm [0, 0, 1, 3]
        const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)u.d, kQuadPerm0013, 0xF, 0xF, false);
        return __builtin_amdgcn_alignbit(u.d, lo, o);
    } else {
        return u.d;
    }
}

// Pair the codes of tokens (2k, 2k+1) position by position: field f of x[k]
// holds position 2f of both tokens, field f of y[k] position 2f+1 (the even
// token in the low VB bits).  Bits above the unit are never read.
template <int VB>
__device__ __forceinline__ void v_pairs(const uint32_t (&u)[8], uint32_t (&x)[4], uint32_t (&y)[4]) {
    constexpr uint32_t M = VB == 4 ? 0x0F0F0F0Fu : VB == 3 ? 0x001C71C7u : 0x00003333u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[k] = (u[2 * k] & M) | ((u[2 * k + 1] << VB) & ~M);
        y[k] = ((u[2 * k] >> VB) & M) | (u[2 * k + 1] & ~M);
    }
}

// A operand of the value MFMA for position tile j (position 8n + j of 8 tokens);
// `tab` points at the V half of the 256-byte table rows.
template <int VB>
__device__ __forceinline__ u4_t v_frag(const uint32_t (&x)[4], const uint32_t (&y)[4], int j, const uint32_t *tab,
                                       uint32_t lane_off) {
    constexpr int FB = 2 * VB;
    const int sh = FB * (j >> 1);
    u4_t f;
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = tab_at(tab, tab_off<FB, 256>((j & 1) ? y[k] : x[k], sh, lane_off));
    return f;
}

// --------------------------------------------------------------------------
// The pass kernel.  MODE_DENSE: attention partials (max, sum, V accumulator) per
// chunk.  MODE_SCORE: per-chunk (max, sum) and per-slice maxima only.
// MODE_GATED: from the scoring partials, the global (max, sum) per row; then
// re-score the candidate slices and accumulate V where p = 2^(s - M) / L >= tau.
// PK: at most 8 rows (hi / lo parts packed in one MFMA's columns).
// CONTIG: block_size is a multiple of 64, so a slice lies in one page.
// --------------------------------------------------------------------------
// Waves per SIMD the register allocation aims for (without spilling): the dense
// pass holds two slices' loads and fits two; so does the gated pass, which keeps
// two candidate slices in flight; the scoring pass with at most 8 rows fits three.
template <bool PK, int VB, int MODE>
constexpr int mfma_waves_per_eu() { return (PK && MODE == MODE_SCORE) ? 3 : 2; }

// Barrier of the block's waves that orders their LDS accesses only: the global
// loads in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One (chunk, unit) item of a pass: item = c * n_seqs * n_kv + unit, covering `span`
// chunks from chunk c (a persistent pass's double items: span 2; their partial is
// written to chunk c's slot, and chunk c + 1's (max, sum) slot gets the empty pair,
// which the gated pass's statistics read; the merge of a paired list reads the even
// chunk slots only, so the second slot's accumulator is not written).
// PRIO: raise the wave's issue priority while it is behind (one-item-per-block
// scoring passes, which hold three blocks per CU).
template <int KB, int VB, bool PK, int MODE, bool CONTIG, int NB, bool OV, bool PRIO = false>
__device__ __forceinline__ void decode_item(
    const int item, const int span, const int tid, const DecodeArgs &a, const PairTables &pt, const uint8_t *__restrict__ k_codes,
    const float *__restrict__ k_norms, const uint8_t *__restrict__ v_codes, const float *__restrict__ v_norms,
    const uint16_t *__restrict__ qin, const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    float *__restrict__ part_ml, float *__restrict__ part_acc, float *__restrict__ tilemax) {
    constexpr bool DENSE = MODE == MODE_DENSE, SCORE = MODE == MODE_SCORE, GATED = MODE == MODE_GATED;
    constexpr bool WV = !SCORE;
    // KF: the K side is plain float16 (KB = 16): its rows are the score MFMA's A
    // operand as loaded, with no pair table, norm, signs or rotation of q
    constexpr bool KF = KB == 16;
    constexpr int NKT = KF ? 1 : 1 << (2 * KB), NVT = 1 << (2 * VB);
    constexpr int KROW = 16 * KB, VROW = 16 * VB;   // bytes per code row (K float16: 256)
    constexpr int KW = KF ? 16 : KB;                // K words per lane and 16-token tile
    constexpr int NQB = PK ? 4 : 8;                 // q'' B fragments
    constexpr int NPB = PK ? 2 : 4;                 // weight B fragments
    constexpr int NG = kMW / NB;                    // wave groups: slices the block has in flight
    // slices a wave's ring holds (loads in flight while one is computed)
    constexpr int NSLOT = (KF || OV || TQ_DECODE_SLOTS < 3) ? 2 : 3;
    static_assert(!OV || (NB == 1 && MODE != MODE_SCORE), "kept V channels: 128-wide heads, passes with V");
    constexpr int RW = NB * kD + (OV ? 16 : 0);     // floats per row of a chunk partial
    constexpr int WRW = kD + (OV ? 16 : 0);         // floats per row of one wave's (block's) sums
    constexpr int WRP = WRW + 4;                    // the same, padded (merge of 9-16 rows)
    constexpr int NS = PK ? 32 : 64;                // exchange slots per tile and wave (lanes
                                                    // holding distinct score columns)
    // the replicated K and V pair tables while slices are processed; afterwards the
    // waves' partials ([wave][row][128] for at most 8 rows, one [row][kQS]
    // accumulator otherwise)
    constexpr int KCOP = tab_copies<KB>(), VCOP = tab_copies<VB>();
    static_assert(KCOP == 32 && VCOP == 32, "32 copies of an entry fill half of a 256-byte row");
    constexpr int RB = WV ? 256 : 128;   // bytes per table row
    constexpr int kTabWords = (WV ? (NKT > NVT ? NKT : NVT) : NKT) * (RB / 4);   // (KF: the V halves only)
    // (NB > 1: q'' of every block, [block][row][kQS], passes through the area before
    // the tables are written)
    constexpr int kMerge = PK ? kMW * 8 * WRW : kMW * 16 * WRP;
    constexpr int kQArea = NB > 1 ? NB * 16 * kQS : 0;
    constexpr int kArea0 = kTabWords > kMerge ? kTabWords : kMerge;
    constexpr int kArea = kArea0 > kQArea ? kArea0 : kQArea;
    __shared__ __attribute__((aligned(16))) uint32_t area[kArea];
    uint32_t *const ktab = area;
    uint32_t *const vtab = area + 32;   // V half of each row (RB = 256)
    float *const mbuf = reinterpret_cast<float *>(area);
    __shared__ __attribute__((aligned(16))) float buf[NB == 1 ? 16 * kQS : 4];   // q'' during set-up
    // NB > 1: partial scores, [wave][tile][slot][4]
    __shared__ __attribute__((aligned(16))) float xch[NB == 1 ? 4 : kMW * 4 * NS * 4];
    __shared__ __attribute__((aligned(16))) float nrm[kMW][2][64];     // per wave: K, V norms of the slice
    __shared__ float wst[kMW][16][2];
    __shared__ float red[kMW];
    __shared__ float gstat[16][2];
    __shared__ __attribute__((aligned(16))) int32_t rowtab[CONTIG ? 1 : kMW][64];
    // fused append: the new tokens' code rows ([token][K row], [token][V row], then
    // K and V norms; row = position - the chunk's first new position, 16 at most),
    // each written and read by the wave that computes its slice
    constexpr bool kApp = !GATED && NB == 1 && !OV && !KF;
    // (then the K and V boundaries of the waves that encode, 16 + 16 floats each)
    __shared__ __attribute__((aligned(16))) uint8_t apbuf[kApp ? 16 * (KROW + VROW) + 32 * 4 + kMW * 32 * 4 : 16];
    float *const apn = reinterpret_cast<float *>(apbuf + (kApp ? 16 * (KROW + VROW) : 0));
    float *const abnd = apn + 32;   // [wave][K 16, V 16]

    __builtin_assume(tid >= 0 && tid < kMBlock);
    const int lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = wave % NB, grp = wave / NB;   // head block and group of this wave
    const int c = (int)fdiv((uint32_t)item, a.units_div);
    const int unit = item - c * a.n_seqs * a.n_kv;
    const int b = (int)fdiv((uint32_t)unit, a.kv_div);
    const int kv = unit - b * a.n_kv;
    const int R = a.rows, rp = a.rows_pad;
    const int start = c * a.chunk;
    const int bs = a.block_size;
    const int n_sub = a.n_kv * NB, kvs = kv * NB + blk;   // cache sub-heads; this wave's
    const FastDiv bsdiv = a.bs_div;
    const int32_t *__restrict__ btab = block_table + (int64_t)b * a.max_blocks;
    constexpr int kStride = NG * 64;
    const int first = start + grp * 64;

    // Small loads go out first.  Vector loads complete in issue order, so loads
    // issued after the slice codes could only be used once those had arrived:
    // the pair-table entries this thread replicates, this wave's query rows and
    // the K sign bits.
    constexpr int KIT = (NKT * 4 + kMBlock - 1) / kMBlock, VIT = (NVT * 4 + kMBlock - 1) / kMBlock;
    uint32_t kent[KIT], vent[WV ? VIT : 1];
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
        const int i = it * kMBlock + tid;
        kent[it] = !KF && i < NKT * 4 ? pt.k[i >> 2] : 0u;
    }
    if constexpr (WV) {
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int i = it * kMBlock + tid;
            vent[it] = i < NVT * 4 ? pt.v[i >> 2] : 0u;
        }
    }
    // (unconditional, from a row clamped into range: a load under a branch has its
    // conversion folded into the branch, which then waits for the load)
    // (the rows of this wave's block: rows grp, grp + NG, ...)
    constexpr int kRowsPerWave = 16 / NG;
    uint32_t qh0[kRowsPerWave], qh1[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        const int r = min(grp + NG * i, a.rows - 1);
        const int jq = (int)fdiv((uint32_t)r, a.grp_div), h = kv * a.group + (r - jq * a.group);
        const uint16_t *qp = qin + (((int64_t)b * a.n_qtok + jq) * a.n_q_heads + h) * (NB * kD) + blk * kD;
        qh0[i] = qp[lane];
        qh1[i] = qp[lane + 64];
    }
    const uint32_t ksg0 = KF ? 0u : a.k_signs[kvs * 4 + (lane >> 5)];
    const uint32_t ksg1 = KF ? 0u : a.k_signs[kvs * 4 + 2 + (lane >> 5)];
    // the sequence length, through the vector path as well: a scalar load would
    // either hold up the loads above (scalar loads are waited for together) or,
    // issued later, queue behind the slice loads
    int len_v;
    {
        int bi = b;
        asm volatile("" : "+v"(bi));
        len_v = seq_lens[bi];
    }

    // Page-table entries of the wave's first two slices (CONTIG: the slice's page;
    // else the page of the lane's token), through the vector path too.  Indices
    // are clamped to the table; entries past the sequence are never used.
    const int last_entry = a.max_blocks - 1;
    int vb0 = 0, vb1 = 0;
    if constexpr (!GATED) {
        int i0 = min((int)fdiv((uint32_t)(first + (CONTIG ? 0 : lane)), bsdiv), last_entry);
        int i1 = min((int)fdiv((uint32_t)(first + kStride + (CONTIG ? 0 : lane)), bsdiv), last_entry);
        asm volatile("" : "+v"(i0), "+v"(i1));
        vb0 = btab[i0];
        vb1 = btab[i1];
    }
    // Gated pass: the first round's candidate inputs (each step's tile maxima and, on
    // contiguous pages, its page-table entry; lane i = step i of the wave) and the
    // scoring pass's chunk (max, sum) pairs (lane = chunk, for at most 64 chunks) go
    // out with the small loads, before the length is known: indices are bounded by
    // the chunk and the workspace instead, and what lies past the sequence is dropped
    // later (steps at or past the end, chunks past the sequence's own).
    typedef float f2v __attribute__((ext_vector_type(2)));
    constexpr int kRW = 16 / kMW;   // rows a wave reduces
    f4_t tmx0[4] = {};
    int cpage0 = 0;
    f2v mlv[kRW] = {};
    const int64_t part_u = (int64_t)unit * a.n_chunks;
    if constexpr (GATED) {
        const int cend = min(start + span * a.chunk, a.n_chunks * a.chunk);   // (tile index < n_tiles)
        const int bic = min(first + lane * kStride, cend - 1);
        const f4_t *tp = reinterpret_cast<const f4_t *>(tilemax + ((int64_t)unit * a.n_tiles + (bic >> 6)) * rp);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            if (4 * r4 < rp) tmx0[r4] = tp[r4];
        if constexpr (CONTIG) {
            int pi = min((int)fdiv((uint32_t)bic, bsdiv), last_entry);
            asm volatile("" : "+v"(pi));
            cpage0 = btab[pi];
        }
        if (a.n_chunks <= 64) {
            const float *ml = part_ml + part_u * rp * NB * 2;
            const int cc = min(lane, a.n_chunks - 1);
#pragma unroll
            for (int i = 0; i < kRW; ++i) {
                const int rr = min(wave + kMW * i, R - 1);
                mlv[i] = *reinterpret_cast<const f2v *>(&ml[(cc * rp + rr) * NB * 2]);
            }
        }
    }
    int len = 0, end = 0;
    const int64_t part = (int64_t)unit * a.n_chunks + c;
    const int64_t tile0 = (int64_t)unit * a.n_tiles;

    // word of a V row this lane loads, and (3-bit) the unit's offset in it
    int vwi = n, vo = 0;
    if constexpr (VB == 3) {
        vwi = 3 * (n >> 2) + min(n & 3, 2);
        vo = (24 * n) & 31;
    }

    // ---- one slice's loads: code words per lane, one K and one V norm per lane
    // (token = lane).  The dense and scoring passes keep two slots, so the next
    // slice's loads are in flight while a slice is computed.
    struct Slot {
        uint32_t kw[4][KW];
        VUnit<VB> vw[2][8];
        uint32_t ow[OV ? 2 : 1][OV ? 4 : 1];   // OV: kept values, float16 pairs (A operand)
        float knl, vnl;
    };
    // OV: this lane's kept channel slot (row n of the A operand; lanes n >= n_out
    // load a valid slot and use 0)
    const int oslot = OV ? min(n, a.n_out - 1) : 0;
    const bool olive = OV && n < a.n_out;
    Slot sa, sb, sc;   // (sc: with three slots in the ring)
    int myrow = 0;   // row of token base + lane (general page layout)

    // (page ids are clamped to the pool: a bad table entry reads another page, never
    // outside the cache)
    auto row0_of = [&](int base, int page) __attribute__((always_inline)) -> int64_t {
        const int pg = (int)fdiv((uint32_t)base, bsdiv);
        return ((int64_t)min(max(page, 0), a.max_page) * n_sub + kvs) * bs + (base - pg * bs);
    };
    // general layout: the row of every token of the slice into the wave's table
    auto fill_rows = [&](int base, int blk_lane) __attribute__((always_inline)) {
        const int t = base + lane;
        myrow = 0;
        if (t < end) {
            const int pg = (int)fdiv((uint32_t)t, bsdiv);
            myrow = (min(max(blk_lane, 0), a.max_page) * n_sub + kvs) * bs + (t - pg * bs);
        }
        rowtab[CONTIG ? 0 : wave][lane] = myrow;
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's row table is written
        __builtin_amdgcn_wave_barrier();
    };
    // this lane's K words of one token for one 16-token tile: 4 KB code bytes, or
    // (K float16) the 64 bytes of positions 32g .. 32g+31
    auto load_kwords = [&](const uint8_t *p, uint32_t (&w)[KW]) __attribute__((always_inline)) {
        if constexpr (KF) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 t = reinterpret_cast<const uint4 *>(p)[i];
                w[4 * i] = t.x;
                w[4 * i + 1] = t.y;
                w[4 * i + 2] = t.z;
                w[4 * i + 3] = t.w;
            }
        } else {
            load_words<KB>(p, w);
        }
    };
    auto load_k = [&](Slot &sl, int64_t row0) __attribute__((always_inline)) {
        if constexpr (CONTIG) {
            const uint8_t *p = k_codes + (row0 + n) * KROW + g * (4 * KW);
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) load_kwords(p + tm * 16 * KROW, sl.kw[tm]);
            sl.knl = KF ? 1.f : k_norms[row0 + lane];
        } else {
            const int32_t *rt = rowtab[wave];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
                load_kwords(k_codes + (int64_t)rt[16 * tm + n] * KROW + g * (4 * KW), sl.kw[tm]);
            sl.knl = KF ? 1.f : k_norms[myrow];
        }
    };
    // V units of the slice's tokens; token (tile tm, e) of lane group g is loaded
    // only where keep(tm, e) holds (every token for the dense pass)
    // (OV: the kept value of slot oslot of the same tokens, into the A pairs)
    const uint16_t *__restrict__ v_kept = OV ? a.v_outliers : nullptr;
    // Kept values are [page][head][slot][block_size]: the element of a cache row
    // (page-row pr = row / bs, offset) is (pr n_out + slot) bs + offset.  Token
    // 16 tm + 4 g + e is k index 4 (tm & 1) + e of operand half tm >> 1.
    // Contiguous pages: the lane's 4 tokens of a tile are one 8-byte load.
    auto load_kept_run = [&](Slot &sl, int64_t row0, auto keep) __attribute__((always_inline)) {
        if constexpr (OV) {
            const int pr = (int)fdiv((uint32_t)row0, bsdiv);
            const int off = (int)row0 - pr * bs;
            const uint16_t *op = v_kept + ((int64_t)pr * a.n_out + oslot) * bs + off + 4 * g;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                uint2 t = make_uint2(0u, 0u);
                if (keep(tm, 0) || keep(tm, 1) || keep(tm, 2) || keep(tm, 3))
                    t = *reinterpret_cast<const uint2 *>(op + 16 * tm);
                if (!keep(tm, 0)) t.x &= 0xFFFF0000u;
                if (!keep(tm, 1)) t.x &= 0x0000FFFFu;
                if (!keep(tm, 2)) t.y &= 0xFFFF0000u;
                if (!keep(tm, 3)) t.y &= 0x0000FFFFu;
                sl.ow[tm >> 1][2 * (tm & 1)] = t.x;
                sl.ow[tm >> 1][2 * (tm & 1) + 1] = t.y;
            }
        }
    };
    // other pages: one float16 load per token, into its half of the pair
    auto load_kept_one = [&](Slot &sl, int tm, int e, int row, bool k) __attribute__((always_inline)) {
        if constexpr (OV) {
            const int ee = 4 * (tm & 1) + e;
            uint32_t &w = sl.ow[tm >> 1][ee >> 1];
            const int pr = (int)fdiv((uint32_t)row, bsdiv);
            const int64_t at = ((int64_t)pr * a.n_out + oslot) * bs + (row - pr * bs);
            const uint32_t h = k ? (uint32_t)v_kept[at] : 0u;
            w = (ee & 1) ? (w | (h << 16)) : h;
        }
    };
    auto load_v = [&](Slot &sl, int64_t row0, auto keep) __attribute__((always_inline)) {
        if constexpr (CONTIG) {
            const uint8_t *p = v_codes + (row0 + 4 * g) * VROW;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    VUnit<VB> &u = sl.vw[tm >> 1][4 * (tm & 1) + e];
                    if (keep(tm, e)) load_vunit<VB>(p + (16 * tm + e) * VROW, vwi, u);
                    else u = VUnit<VB>{};
                }
            load_kept_run(sl, row0, keep);
            sl.vnl = v_norms[row0 + lane];
        } else {
            const int32_t *rt = rowtab[wave];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const i4_t rr = *reinterpret_cast<const i4_t *>(rt + 16 * tm + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    VUnit<VB> &u = sl.vw[tm >> 1][4 * (tm & 1) + e];
                    if (keep(tm, e)) load_vunit<VB>(v_codes + (int64_t)rr[e] * VROW, vwi, u);
                    else u = VUnit<VB>{};
                    load_kept_one(sl, tm, e, rr[e], keep(tm, e));
                }
            }
            sl.vnl = v_norms[myrow];
        }
    };
    auto all_tokens = [](int, int) { return true; };

    // (a length past the page table's capacity is clamped to it)
    len = min(__builtin_amdgcn_readfirstlane(len_v), a.max_blocks * bs);
    if (start >= len) {
        // the small loads are consumed on this path too, so they stay ahead of
        // the length test instead of being moved below it
        uint32_t x = ksg0 ^ ksg1 ^ (uint32_t)len_v ^ (uint32_t)vb0 ^ (uint32_t)vb1;
        if constexpr (GATED) {
            x ^= (uint32_t)cpage0;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                x ^= __float_as_uint(tmx0[r4][0] + tmx0[r4][1] + tmx0[r4][2] + tmx0[r4][3]);
#pragma unroll
            for (int i = 0; i < kRW; ++i) x ^= __float_as_uint(mlv[i].x + mlv[i].y);
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) x ^= qh0[i] ^ qh1[i];
#pragma unroll
        for (int it = 0; it < KIT; ++it) x ^= kent[it];
        if constexpr (WV) {
#pragma unroll
            for (int it = 0; it < VIT; ++it) x ^= vent[it];
        }
        asm volatile("" ::"v"(x));
        return;
    }
    end = min(start + span * a.chunk, len);

    // ---- fused append: the new positions this wave computes, [own_pa, own_pa + n_own)
    // (they lie in at most two slices of the chunk, each computed by one wave), and
    // the float16 rows of its first 8 vectors (K rows of its new tokens, then their V
    // rows; lanes past the last vector repeat it, unstored) with their pages, issued
    // before the first slice so that waiting for them never waits for slice data
    constexpr bool APP = kApp;   // (not K float16: already at the register limit)
    const int p0 = len - a.n_qtok;
    int own_pa = 0, n_own = 0;
    const int app0 = max(p0, start);   // the chunk's first new position: apbuf row = position - app0
    if constexpr (APP) {
        if (a.append) {
            const int pa = app0;
            if (pa < end) {
                const int s0 = (pa - start) >> 6, s1 = (end - 1 - start) >> 6;
                if (s0 % NG == grp) {
                    own_pa = pa;
                    n_own = min(end, start + 64 * (s0 + 1)) - pa;
                } else if (s1 != s0 && s1 % NG == grp) {
                    own_pa = start + 64 * s1;
                    n_own = end - own_pa;
                }
            }
        }
    }
    const Lane8 l8 = lane8();
    struct AppVec {
        int pos, side;
        bool live;
    };
    auto app_vec = [&](int pass) __attribute__((always_inline)) -> AppVec {
        const int nv = 2 * n_own, vi = pass * 8 + l8.vin, vc = min(vi, nv - 1);
        const int side = vc >= n_own ? 1 : 0;
        return AppVec{own_pa + (side ? vc - n_own : vc), side, vi < nv};
    };
    uint32_t aw[8];
    int apage = 0;
    // (the two row pointers are held in scalar registers, so the per-lane choice
    // between them is a register select, not a load of the selected argument)
    typedef const __attribute__((address_space(1))) uint16_t g_u16;
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u4v g_u4;
    typedef const __attribute__((address_space(1))) uint32_t g_u32;
    g_u16 *k_new = (g_u16 *)a.k_new, *v_new = (g_u16 *)a.v_new;
    g_u32 *k_sg = (g_u32 *)a.k_signs, *v_sg = (g_u32 *)a.v_signs;
    asm volatile("" : "+s"(k_new), "+s"(v_new), "+s"(k_sg), "+s"(v_sg));
    uint32_t asg = 0;   // the vector's sign word (its side, this lane's 16 elements)
    auto app_load = [&](const AppVec &av) __attribute__((always_inline)) {
        asg = (av.side ? v_sg : k_sg)[kvs * 4 + (l8.j >> 1)];
        g_u16 *srcp = (av.side ? v_new : k_new) +
                      ((int64_t)b * a.n_qtok + (av.pos - p0)) * a.new_stride + kv * kD + 16 * l8.j;
        const u4v x0 = reinterpret_cast<g_u4 *>(srcp)[0], x1 = reinterpret_cast<g_u4 *>(srcp)[1];
        aw[0] = x0.x; aw[1] = x0.y; aw[2] = x0.z; aw[3] = x0.w;
        aw[4] = x1.x; aw[5] = x1.y; aw[6] = x1.z; aw[7] = x1.w;
        apage = btab[min((int)fdiv((uint32_t)av.pos, bsdiv), last_entry)];
    };
    // the first 8 vectors go out with the first slice's loads: after its page is
    // read (so the wait for the page never covers them) and before its data
    auto app_first = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if (APP && n_own > 0) app_load(app_vec(0));   // wave-uniform
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (GATED) app_first();

    // ---- the first slice's loads (r0_prev: its first row; blk_next: page of the
    // second slice)
    int64_t r0_prev = 0;
    int blk_next = 0;
    if constexpr (!GATED) {
        if constexpr (CONTIG) {
            const int blk0 = __builtin_amdgcn_readfirstlane(vb0);
            const int pg = (int)fdiv((uint32_t)first, bsdiv);
            r0_prev = ((int64_t)min(max(blk0, 0), a.max_page) * n_sub + kvs) * bs + (first - pg * bs);   // (row0_of)
            app_first();
            load_k(sa, r0_prev);   // (its V units go out after the set-up, below)
            blk_next = vb1;
        } else {
            fill_rows(first, first + lane < end ? vb0 : 0);
            app_first();
            load_k(sa, 0);
            if constexpr (DENSE) load_v(sa, 0, all_tokens);
            blk_next = first + kStride + lane < end ? vb1 : 0;
        }
    }

    // replicate the pair tables: 4 threads per entry (i = 4 e + quarter), 8 copies each
    auto fill_entry = [&](uint32_t *tab, uint32_t v, int i) __attribute__((always_inline)) {
        u4_t *d = reinterpret_cast<u4_t *>(tab + (i >> 2) * (RB / 4) + (i & 3) * 8);
        d[0] = u4_t{v, v, v, v};
        d[1] = u4_t{v, v, v, v};
    };
    auto fill_tables = [&]() __attribute__((always_inline)) {
        if constexpr (!KF) {
#pragma unroll
            for (int it = 0; it < KIT; ++it)
                if (it * kMBlock + tid < NKT * 4) fill_entry(ktab, kent[it], it * kMBlock + tid);
        }
        if constexpr (WV) {
#pragma unroll
            for (int it = 0; it < VIT; ++it)
                if (it * kMBlock + tid < NVT * 4) fill_entry(vtab, vent[it], it * kMBlock + tid);
        }
    };
    if constexpr (NB == 1) fill_tables();   // (NB > 1: once q'' has left the area)
    const uint32_t lane_off = (uint32_t)(lane & 31) << 2;

    // ---- q'' = qscale * H (s_K * q) of this KV head's rows (K float16: qscale * q) for
    // this wave's block, into qbuf
    float *const qbuf = NB == 1 ? buf : reinterpret_cast<float *>(area) + blk * 16 * kQS;
    {
        float qm = 0.f;
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = grp + NG * i;
            if (r >= R) break;
            float x0 = (float)__builtin_bit_cast(_Float16, (uint16_t)qh0[i]);
            float x1 = (float)__builtin_bit_cast(_Float16, (uint16_t)qh1[i]);
            if ((ksg0 >> (lane & 31)) & 1u) x0 = -x0;
            if ((ksg1 >> (lane & 31)) & 1u) x1 = -x1;
            if constexpr (!KF) hadamard128(x0, x1, lane);   // (K float16: q is not rotated)
            x0 *= a.qscale;
            x1 *= a.qscale;
            qbuf[r * kQS + lane] = x0;
            qbuf[r * kQS + lane + 64] = x1;
            qm = fmaxf(qm, fmaxf(fabsf(x0), fabsf(x1)));
        }
        qm = wave_max(qm);
        if (lane == 0) red[wave] = qm;
    }
    // sparse: global (max, sum) of each row from the scoring pass's chunk partials
    // (part_ml is [chunk][row][block][2]; the blocks' entries are equal, block 0's is
    // read).  With at most 64 chunks (one per lane) every row's pairs were loaded
    // with the small loads, so the statistics cost no round trip of their own; the
    // sums are the same either way.
    if constexpr (GATED) {
        const int nc = min((int)fdiv((uint32_t)(len + a.chunk - 1), a.chunk_div), a.n_chunks);
        const float *ml = part_ml + part_u * rp * NB * 2;
        if (a.n_chunks <= 64) {
#pragma unroll
            for (int i = 0; i < kRW; ++i) {
                const int r = wave + kMW * i;
                if (r < R) {
                    const float M = wave_max(lane < nc ? mlv[i].x : -INFINITY);
                    const float L = wave_sum(lane < nc ? mlv[i].y * exp2_diff(mlv[i].x, M) : 0.f);
                    if (lane == 0) {
                        gstat[r][0] = M;
                        gstat[r][1] = L;
                    }
                }
            }
        } else for (int r = wave; r < R; r += kMW) {
            float m = -INFINITY;
            for (int cc = lane; cc < nc; cc += 64) m = fmaxf(m, ml[(cc * rp + r) * NB * 2]);
            const float M = wave_max(m);
            float l = 0.f;
            for (int cc = lane; cc < nc; cc += 64)
                l += ml[(cc * rp + r) * NB * 2 + 1] * exp2_diff(ml[(cc * rp + r) * NB * 2], M);
            const float L = wave_sum(l);
            if (lane == 0) {
                gstat[r][0] = M;
                gstat[r][1] = L;
            }
        }
    }
    __syncthreads();

    // q'' is scaled by a power of two so its largest element is in [2^13, 2^14)
    // (fp16 range and precision for both parts); scores are scaled back by kscale.
    float qmax = red[blk];
#pragma unroll
    for (int g2 = 1; g2 < NG; ++g2) qmax = fmaxf(qmax, red[blk + NB * g2]);
    const int qex = qmax > 0.f ? max((int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127, -100) : 0;
    const float sq = __builtin_ldexpf(1.f, 13 - qex), kscale = __builtin_ldexpf(1.f, qex - 13);

    const int col_row = PK ? (n & 7) : n;             // query row of this lane's column
    const float losel = (PK && n >= 8) ? 1.f : 0.f;   // column holds lo parts
    u4_t qb[NQB];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // (read for every lane: the buffer holds 16 rows; rows past R are dropped)
            const float *qr = &qbuf[col_row * kQS + 32 * g + 8 * ks + 2 * k];
            const float r0 = qr[0], r1 = qr[1];
            const float q0 = col_row < R ? r0 * sq : 0.f, q1 = col_row < R ? r1 * sq : 0.f;
            if constexpr (PK) {
                qb[ks][k] = split_pair(q0, q1, losel);
            } else {
                qb[ks][k] = pk_rtz(q0, q1);
                qb[4 + ks][k] = split_pair(q0, q1, 1.f);
            }
        }
    if constexpr (NB > 1) {
        __syncthreads();   // every wave has its q'' fragments: the area takes the tables
        fill_tables();
        __syncthreads();
    }
    const bool row_ok = col_row < R;
    // last position each row sees in this chunk (row r sees t <= len - n_qtok + r / G)
    const int lim = row_ok ? min(end - 1, len - a.n_qtok + (int)fdiv((uint32_t)col_row, a.grp_div)) : -1;
    const int lim_all = min(end - 1, len - a.n_qtok);   // seen by every row

    // sparse: keep iff s >= sthr (p >= tau); weights 2^(s - mlog) = p
    float sthr = INFINITY, mlog = 0.f;
    if constexpr (GATED) {
        if (row_ok) {
            const float M = gstat[col_row][0], L = gstat[col_row][1];
            if (L > 0.f && M > -INFINITY) {
                mlog = M + log2f(L);
                sthr = mlog + log2f(a.tau);
            }
        }
    }

    // ---- the second slice's loads, once the set-up above is done: the first
    // slice's went out before it (on contiguous pages its K words only; its V units
    // follow here), both would fill the memory pipeline and hold the set-up up.  Every issue loads, whether or not its slice lies below the end: one past the
    // end re-reads the rows of the last slice issued (cached, and never used), so
    // the loads of both slots are the same instructions on every path and each
    // wait covers only the slot it needs, never the one in flight behind it.
    // blk_next: page of the next slice (CONTIG, the same in every lane), or of the
    // lane's token of it; page-table reads are clamped to the table.
    auto page_clamped = [&](int t) __attribute__((always_inline)) -> int {
        const int pg = btab[min((int)fdiv((uint32_t)t, bsdiv), last_entry)];
        return t < end ? pg : 0;
    };
    auto issue = [&](Slot &sl, int base) __attribute__((always_inline)) {
        int64_t r0 = 0;
        if constexpr (CONTIG) {
            r0 = base < end ? row0_of(base, __builtin_amdgcn_readfirstlane(blk_next)) : r0_prev;
            r0_prev = r0;
            int i = min((int)fdiv((uint32_t)(base + kStride), bsdiv), last_entry);
            asm volatile("" : "+v"(i));
            blk_next = btab[i];
        } else {
            fill_rows(base, blk_next);
            blk_next = page_clamped(base + kStride + lane);
        }
        load_k(sl, r0);
        if constexpr (DENSE) load_v(sl, r0, all_tokens);
    };
    if constexpr (!GATED) {
        // contiguous pages: the first slice's V units now (its K words went out before
        // the set-up: fewer loads ahead of the set-up's own instructions, which wait
        // behind them when the memory pipeline is full)
        if constexpr (CONTIG && DENSE) {
            __builtin_amdgcn_sched_barrier(0);
            load_v(sa, r0_prev, all_tokens);
        }
        // slot b's loads strictly after slot a's, so waiting for a never waits for b
        __builtin_amdgcn_sched_barrier(0);
        issue(sb, first + kStride);
        if constexpr (NSLOT == 3) {
            __builtin_amdgcn_sched_barrier(0);
            issue(sc, first + 2 * kStride);
        }
    }

    // ---- fused append (the waves that compute new positions): encode the rows, store
    // them to the cache and into apbuf for the patch of their slices; after the
    // set-up, while the first slice's data is on its way (V: the pass's own width;
    // the scoring pass, built for one V width, stores with a.v_bits)
    if constexpr (APP) {
        if (n_own > 0) {   // wave-uniform
            // the boundaries into the wave's LDS row (lane i < 15: K boundary i; 16 + i: V)
            {
                float bk = 0.f, bv = 0.f;
#pragma unroll
                for (int i = 0; i < TQ_MAX_LEVELS - 1; ++i) {
                    bk = (lane & 15) == i ? a.kbnd[i] : bk;
                    bv = (lane & 15) == i ? a.vbnd[i] : bv;
                }
                if (lane < 32) abnd[wave * 32 + lane] = lane < 16 ? bk : bv;
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
                __builtin_amdgcn_wave_barrier();
            }
            const float *bk = abnd + wave * 32, *bv = bk + 16;
            // one pass: the 8 vectors whose rows are in aw (pass 0's were loaded with the
            // first slice; a later pass loads its own, then waits for them)
            auto encode_pass = [&](const AppVec &av) __attribute__((always_inline)) {
                const int pg = (int)fdiv((uint32_t)av.pos, bsdiv);
                const int64_t arow = ((int64_t)apage * n_sub + kvs) * bs + (av.pos - pg * bs);
                const int tk = av.pos - app0;
                const uint32_t sb = (asg >> ((l8.j & 1) * 16)) & 0xFFFFu;
                uint32_t code[16], lo, hi;
                // (the cache rows are written only for a page inside the pool; the
                // copy for this launch's attention always)
                const bool in_pool = (unsigned)apage <= (unsigned)a.max_page;
                if (!av.side) {
                    const float nm = encode_block8<KB>(aw, sb, bk, l8.j, code);
                    pack_lane_codes<KB>(code, lo, hi);
                    if (av.live) {
                        if (in_pool) store_lane_packed<KB>(a.k_codes_w + arow * KROW, lo, hi, l8.j);
                        store_lane_packed<KB>(apbuf + tk * KROW, lo, hi, l8.j);
                        if (l8.j == 0) {
                            if (in_pool) a.k_norms_w[arow] = nm;
                            apn[tk] = nm;
                        }
                    }
                } else {
                    const int vb = DENSE ? VB : a.v_bits;
                    float nm;
                    if (vb == 4) {
                        nm = encode_block8<4>(aw, sb, bv, l8.j, code);
                        pack_lane_codes<4>(code, lo, hi);
                    } else if (vb == 3) {
                        nm = encode_block8<3>(aw, sb, bv, l8.j, code);
                        pack_lane_codes<3>(code, lo, hi);
                    } else {
                        nm = encode_block8<2>(aw, sb, bv, l8.j, code);
                        pack_lane_codes<2>(code, lo, hi);
                    }
                    if (av.live) {
                        uint8_t *vrow = a.v_codes_w + arow * (16 * vb);
                        if (in_pool) {
                            if (vb == 4) store_lane_packed<4>(vrow, lo, hi, l8.j);
                            else if (vb == 3) store_lane_packed<3>(vrow, lo, hi, l8.j);
                            else store_lane_packed<2>(vrow, lo, hi, l8.j);
                        }
                        if constexpr (DENSE) store_lane_packed<VB>(apbuf + 16 * KROW + tk * VROW, lo, hi, l8.j);
                        if (l8.j == 0) {
                            if (in_pool) a.v_norms_w[arow] = nm;
                            apn[16 + tk] = nm;
                        }
                    }
                }
            };
            encode_pass(app_vec(0));
            for (int pass = 1; pass * 8 < 2 * n_own; ++pass) {
                const AppVec av = app_vec(pass);
                app_load(av);
                encode_pass(av);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's copies are in LDS
            __builtin_amdgcn_wave_barrier();
        }
    }

    // ---- score MFMAs of the loaded slice.  The 16 table lookups of tile tm + 1 are
    // issued before the MFMAs of tile tm (the scheduling barriers keep that order),
    // so the LDS round trip of one tile is covered by the previous tile's MFMAs
    // instead of being waited for in front of every MFMA.
    auto score_mfma = [&](const Slot &sl, f4_t (&S)[4]) {
        if constexpr (KF) {
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                S[tm] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const u4_t af = u4_t{sl.kw[tm][4 * ks], sl.kw[tm][4 * ks + 1], sl.kw[tm][4 * ks + 2],
                                         sl.kw[tm][4 * ks + 3]};
                    S[tm] = mfma_f16(af, qb[ks], S[tm]);
                    if constexpr (!PK) S[tm] = mfma_f16(af, qb[4 + ks], S[tm]);
                }
            }
        } else {
            u4_t fa[4], fb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) fa[ks] = k_frag<KB, RB>(sl.kw[0], ks, ktab, lane_off);
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                __builtin_amdgcn_sched_barrier(0);
                if (tm < 3) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) fb[ks] = k_frag<KB, RB>(sl.kw[tm + 1], ks, ktab, lane_off);
                }
                __builtin_amdgcn_sched_barrier(0);
                S[tm] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    S[tm] = mfma_f16(fa[ks], qb[ks], S[tm]);
                    if constexpr (!PK) S[tm] = mfma_f16(fa[ks], qb[4 + ks], S[tm]);
                }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) fa[ks] = fb[ks];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // the slice's norms to the wave's LDS rows (V norms past the chunk's end are
    // not data and become 0); returns the V exponent E: max V norm < 2^E, so the
    // weights e * vn * 2^-E stay below 1
    float *my_kn = nrm[wave][0], *my_vn = nrm[wave][1];
    // The slice's norms into the wave's LDS rows: K before the score MFMAs, V (and
    // the exponent E_s of its largest) before the weights, so the scores never wait
    // for the V loads, which go out after the K loads.
    auto stage_knorms = [&](const Slot &sl) __attribute__((always_inline)) {
        my_kn[lane] = sl.knl * kscale;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    };
    auto stage_vnorms = [&](const Slot &sl, int base) __attribute__((always_inline)) -> float {
        if constexpr (!WV) return 0.f;
        const float v = base + lane < end ? sl.vnl : 0.f;
        my_vn[lane] = v;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const float vm = wave_max(v);
        const int ex = vm > 0.f ? (int)((__float_as_uint(vm) >> 23) & 0xFF) - 126 : -40;
        return (float)min(max(ex, -40), 40);
    };
    auto stage_norms = [&](const Slot &sl, int base) __attribute__((always_inline)) -> float {
        stage_knorms(sl);
        return stage_vnorms(sl, base);
    };
    // NB > 1: replace each partial score by the sum of the group's partials, blocks
    // in ascending order (called by every wave of the block, the same number of
    // times: it holds the block's barriers).  The first barrier keeps the previous
    // exchange's reads ahead of this one's writes.  Lane (g, n) holds the scores of
    // tokens 16 tm + 4 g + e for column n; with PK, columns n and n + 8 are equal
    // and lanes n < 8 write.
    const int xslot = PK ? 8 * g + (n & 7) : lane;
    auto exchange = [&](float (&s)[4][4]) __attribute__((always_inline)) {
        lds_barrier();
        if (!PK || n < 8) {
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
                *reinterpret_cast<f4_t *>(&xch[((wave * 4 + tm) * NS + xslot) * 4]) =
                    f4_t{s[tm][0], s[tm][1], s[tm][2], s[tm][3]};
        }
        lds_barrier();
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            f4_t t = *reinterpret_cast<const f4_t *>(&xch[(((grp * NB) * 4 + tm) * NS + xslot) * 4]);
#pragma unroll
            for (int j = 1; j < NB; ++j)
                t += *reinterpret_cast<const f4_t *>(&xch[(((grp * NB + j) * 4 + tm) * NS + xslot) * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[tm][e] = t[e];
        }
    };
    // scores in the log2 domain, -inf where the row does not see the token
    // (full: every row sees every token of the slice)
    auto scores = [&](const f4_t (&S)[4], int base, bool full, float (&s)[4][4]) {
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const f4_t kn = *reinterpret_cast<const f4_t *>(my_kn + 16 * tm + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = S[tm][e];
                if constexpr (PK) x += dpp<kDppRor8>(x);
                s[tm][e] = x * kn[e];
            }
        }
        if constexpr (NB > 1) exchange(s);
        if (!full) {
            const int dl = lim - base - 4 * g;   // element (tm, e) visible iff 16 tm + e <= dl
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * tm + e > dl) s[tm][e] = -INFINITY;
        }
    };
    // value MFMAs of the loaded slice with weights w (score layout)
    f4_t acc[WV ? 8 : 1];
#pragma unroll
    for (int j = 0; j < (WV ? 8 : 1); ++j) acc[j] = f4_t{0.f, 0.f, 0.f, 0.f};
    f4_t acc_o = f4_t{0.f, 0.f, 0.f, 0.f};   // OV: kept channel sums, D rows = slots
    // OV: wo, the weights of the kept values (score layout, no V norm)
    // (base: the slice; kept values of tokens past the chunk's end are not data and
    // become 0, as a zero weight would not cancel a non-finite value)
    auto kept_mfma = [&](const Slot &sl, const float (&wo)[4][4], int base) __attribute__((always_inline)) {
        if constexpr (OV) {
            uint32_t ow[2][4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int k = 0; k < 4; ++k) ow[ks][k] = sl.ow[ks][k];
            if (base + 64 > end) {
                const int dl = end - base - 4 * g;   // token 16 tm + 4 g + e is data iff 16 tm + e < dl
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int tm = 2 * ks + (k >> 1), e0 = 2 * (k & 1);
                        if (16 * tm + e0 >= dl) ow[ks][k] &= 0xFFFF0000u;
                        if (16 * tm + e0 + 1 >= dl) ow[ks][k] &= 0x0000FFFFu;
                    }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u4_t pb[2];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int tm = 2 * ks + (k >> 1), e0 = 2 * (k & 1);
                    if constexpr (PK) {
                        pb[0][k] = split_pair(wo[tm][e0], wo[tm][e0 + 1], losel);
                    } else {
                        pb[0][k] = pk_rtz(wo[tm][e0], wo[tm][e0 + 1]);
                        pb[1][k] = split_pair(wo[tm][e0], wo[tm][e0 + 1], 1.f);
                    }
                }
                const u4_t af = olive ? u4_t{ow[ks][0], ow[ks][1], ow[ks][2], ow[ks][3]} : u4_t{0u, 0u, 0u, 0u};
                acc_o = mfma_f16(af, pb[0], acc_o);
                if constexpr (!PK) acc_o = mfma_f16(af, pb[1], acc_o);
            }
        }
    };
    auto value_mfma = [&](const Slot &sl, const float (&w)[4][4]) {
        u4_t pb[NPB];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int tm = 2 * ks + (k >> 1), e0 = 2 * (k & 1);
                if constexpr (PK) {
                    pb[ks][k] = split_pair(w[tm][e0], w[tm][e0 + 1], losel);
                } else {
                    pb[ks][k] = pk_rtz(w[tm][e0], w[tm][e0 + 1]);
                    pb[2 + ks][k] = split_pair(w[tm][e0], w[tm][e0 + 1], 1.f);
                }
            }
        // four groups of four position tiles (ks, j0 .. j0 + 3); the lookups of the
        // next group go out before the MFMAs of the current one, as for the scores
        uint32_t x[2][4], y[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint32_t u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = vunit_bits<VB>(sl.vw[ks][e], vo);
            v_pairs<VB>(u, x[ks], y[ks]);
        }
        u4_t fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = v_frag<VB>(x[0], y[0], i, vtab, lane_off);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int ks = gi >> 1, j0 = 4 * (gi & 1);
            __builtin_amdgcn_sched_barrier(0);
            if (gi < 3) {
                const int ksn = (gi + 1) >> 1, jn = 4 * ((gi + 1) & 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) fb[i] = v_frag<VB>(x[ksn], y[ksn], jn + i, vtab, lane_off);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[j0 + i] = mfma_f16(fa[i], pb[ks], acc[j0 + i]);
                if constexpr (!PK) acc[j0 + i] = mfma_f16(fa[i], pb[2 + ks], acc[j0 + i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = fb[i];
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    float m_raw = -INFINITY, m_state = -INFINITY, l_run = 0.f, E_run = -INFINITY;
    uint32_t v_rows = 0;   // gated: V code rows this wave reads

    if constexpr (!GATED) {
        // ---------------- dense / scoring pass: a two-slot ring, the next slice's
        // loads in flight while a slice is computed
        // fused append: a slice holding this wave's new tokens takes their rows from
        // apbuf (K words: token base + 16 tm + n; V units: token base + 16 tm + 4 g + e;
        // norms: token base + lane)
        auto patch = [&](Slot &sl, int base) __attribute__((always_inline)) {
            if constexpr (APP) {
                if (n_own == 0 || base + 64 <= own_pa || base >= own_pa + n_own) return;   // uniform
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    const int to = base + 16 * tm + n - own_pa, tk = to + own_pa - app0;
                    if ((unsigned)to < (unsigned)n_own) {
                        const uint32_t *r = reinterpret_cast<const uint32_t *>(apbuf + tk * KROW + 4 * KW * g);
#pragma unroll
                        for (int i = 0; i < KW; ++i) sl.kw[tm][i] = r[i];
                    }
                }
                const int tlo = base + lane - own_pa, tl = tlo + own_pa - app0;
                if ((unsigned)tlo < (unsigned)n_own) sl.knl = apn[tl];
                if constexpr (DENSE) {
#pragma unroll
                    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int to = base + 16 * tm + 4 * g + e - own_pa, tk = to + own_pa - app0;
                            if ((unsigned)to < (unsigned)n_own)
                                load_vunit<VB>(apbuf + 16 * KROW + tk * VROW, vwi, sl.vw[tm >> 1][4 * (tm & 1) + e]);
                        }
                    if ((unsigned)tlo < (unsigned)n_own) sl.vnl = apn[16 + tl];
                }
            }
        };
        auto compute = [&](Slot &sl, int base) __attribute__((always_inline)) {
            patch(sl, base);
            stage_knorms(sl);
            f4_t S[4];
            score_mfma(sl, S);
            const bool full = base + 63 <= lim_all;
            float s[4][4];
            scores(S, base, full, s);
            float wm = -INFINITY;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int e = 0; e < 4; ++e) wm = fmaxf(wm, s[tm][e]);
            wm = xg_max(wm);
            if constexpr (SCORE) {
                if (g == 0 && row_ok && (!PK || n < 8) && blk == 0)
                    tilemax[(tile0 + (base >> 6)) * rp + col_row] = wm;
            }
            const float E_s = stage_vnorms(sl, base);
            const float m_new = fmaxf(m_raw, wm);
            const float E_new = DENSE ? fmaxf(E_run, E_s) : 0.f;
            const float mu = (m_new == -INFINITY ? 0.f : m_new) + E_new;
            const float alpha = exp2_diff(m_state, mu);
            // OV: kept sums are relative to 2^m (weights 2^(s - m) = ex 2^E, exact)
            const float alpha_o = OV ? exp2_diff(m_raw, m_new) : 1.f;
            const float eE = OV ? __builtin_ldexpf(1.f, (int)E_new) : 0.f;
            float lsum = 0.f, w[4][4], wo[4][4];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const f4_t vn = DENSE ? *reinterpret_cast<const f4_t *>(my_vn + 16 * tm + 4 * g) : f4_t{};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ex = __builtin_amdgcn_exp2f(s[tm][e] - mu);
                    lsum += ex;
                    if constexpr (DENSE) w[tm][e] = ex * vn[e];
                    if constexpr (OV) wo[tm][e] = ex * eE;
                }
            }
            lsum = xg_sum(lsum);
            l_run = l_run * alpha + lsum;
            m_raw = m_new;
            m_state = m_new == -INFINITY ? -INFINITY : mu;
            E_run = E_new;
            if constexpr (DENSE) {
                if (base != first && __ballot(alpha != 1.f)) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
                }
                value_mfma(sl, w);
                if constexpr (OV) {
                    acc_o *= alpha_o;
                    kept_mfma(sl, wo, base);
                }
            }
        };
        // one exit, at the top: a branch inside the loop would merge paths with
        // different loads outstanding, and every wait after it would then cover both
        // slots; skipping a compute (which issues no loads) does not
        // (the scheduling barriers keep each compute below the loads issued
        // before it in the source, which it must not wait for).
        // NB > 1: the steps are the block's (b0 from the chunk start, the same in
        // every wave, as the exchange's barriers need), each group's slice `lead`
        // tokens in; a slice past the end has every score masked and changes nothing.
        const int lead = first - start;
        // PRIO: the SIMD's arbiter favours its oldest wave, so of the blocks sharing a
        // CU the first one dispatched would finish well before the last, which then
        // runs with the SIMDs half idle.  Each wave's priority falls from 3 to 0 as it
        // passes each quarter of its steps, so the waves that are behind issue first
        // and the blocks end together.
        const int pq1 = first + (end - first) / 4, pq2 = first + (end - first) / 2,
                  pq3 = first + 3 * ((end - first) / 4);
        for (int b0 = NB == 1 ? first : start; b0 < end; b0 += NSLOT * kStride) {
            const int base = NB == 1 ? b0 : b0 + lead;
            if constexpr (PRIO) {
                if (b0 < pq1) __builtin_amdgcn_s_setprio(3);
                else if (b0 < pq2) __builtin_amdgcn_s_setprio(2);
                else if (b0 < pq3) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
            __builtin_amdgcn_sched_barrier(0);
            compute(sa, base);   // the other slots hold the next slices (in flight)
            issue(sa, base + NSLOT * kStride);
            __builtin_amdgcn_sched_barrier(0);
            if (b0 + kStride < end) compute(sb, base + kStride);
            issue(sb, base + (NSLOT + 1) * kStride);
            if constexpr (NSLOT == 3) {
                __builtin_amdgcn_sched_barrier(0);
                if (b0 + 2 * kStride < end) compute(sc, base + 2 * kStride);
                issue(sc, base + 5 * kStride);
            }
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    } else {
        // ---------------- gated pass: candidate slices only (a group's decision is
        // the same in its NB waves; NB > 1: every wave takes part in each step's
        // exchange, as in the dense loop)
        // The candidate test of 64 steps at a time: lane i loads the tile maxima of
        // every row for step i of the round and compares them with the rows'
        // thresholds (the same values and compare as sthr), so the loop waits for
        // one round trip per 64 slices instead of one per slice.
        // (lane r < 16 forms row r's threshold, the same expression as sthr, and every
        // row's is read from its lane: one LDS read and one logarithm per lane instead
        // of a dependent read and logarithm per row)
        float sthr_r[16];
        {
            const int rl = lane & 15;
            const float Mr = gstat[rl][0], Lr = gstat[rl][1];   // (rows >= R: not used)
            const float thr = (rl < R && Lr > 0.f && Mr > -INFINITY) ? (Mr + log2f(Lr)) + log2f(a.tau) : INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sthr_r[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(thr), r));
        }
        // (contiguous pages: the same round loads each step's page-table entry, so a
        // candidate slice's codes go out without another round trip)
        const int lead = first - start;
        uint64_t cmask = 0;
        int cpage = 0;
        // the candidate test of the 64 steps from `step` (lane i: step + i)
        auto round_mask = [&](int step, int base) __attribute__((always_inline)) {
            const int bi = base + lane * kStride;
            f4_t t[4] = {tmx0[0], tmx0[1], tmx0[2], tmx0[3]};
            if (step == 0) {
                cpage = cpage0;
            } else {
                const int bic = min(bi, end - 1);
                if constexpr (CONTIG) {
                    int pi = min((int)fdiv((uint32_t)bic, bsdiv), last_entry);
                    asm volatile("" : "+v"(pi));
                    cpage = btab[pi];
                }
                const f4_t *tp = reinterpret_cast<const f4_t *>(tilemax + (tile0 + (bic >> 6)) * rp);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    if (4 * r4 < rp) t[r4] = tp[r4];
            }
            bool c = false;
            if (bi < end) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    if (4 * r4 < rp) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) c = c || (4 * r4 + k < R && t[r4][k] >= sthr_r[4 * r4 + k]);
                    }
                }
            }
            cmask = __ballot(c);
        };
        // the V accumulation of a scored candidate slice (scores s): tokens kept by at
        // least one row; weights p = 2^(s - mlog) where kept, else 0
        auto gated_values = [&](Slot &sl, const float (&s)[4][4], float E_s, int base, int64_t r0, bool v_loaded)
            __attribute__((always_inline)) -> void {
            bool kept[4][4];
            uint64_t any = 0;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint64_t bal = __ballot(s[tm][e] >= sthr);
                    any |= bal;
                    kept[tm][e] = ((bal >> (16 * g)) & 0xFFFFull) != 0ull;
                }
            if (!any) return;
            if (a.v_rows_read) {   // the V rows the rule needs (token groups g with a kept row)
                uint32_t cnt = 0;
#pragma unroll
                for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint64_t bal = __ballot(kept[tm][e] && n == 0);
                        cnt += (uint32_t)__popcll(bal);
                    }
                v_rows += cnt;
            }
            if (!v_loaded) load_v(sl, r0, [&](int tm, int e) { return kept[tm][e]; });
            const float E_new = fmaxf(E_run, E_s);
            if (E_run != -INFINITY && E_new != E_run) {
                const float f = __builtin_amdgcn_exp2f(E_run - E_new);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] *= f;
            }
            E_run = E_new;
            const float mu = mlog + E_new;
            const float eE = OV ? __builtin_ldexpf(1.f, (int)E_new) : 0.f;
            float w[4][4], wo[4][4];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const f4_t vn = *reinterpret_cast<const f4_t *>(my_vn + 16 * tm + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ex = s[tm][e] >= sthr ? __builtin_amdgcn_exp2f(s[tm][e] - mu) : 0.f;
                    w[tm][e] = ex * vn[e];
                    if constexpr (OV) wo[tm][e] = ex * eE;   // = p, the final weight
                }
            }
            value_mfma(sl, w);
            kept_mfma(sl, wo, base);
        };
        if constexpr (NB == 1 && CONTIG && !KF && !OV) {
            // (float16 K and kept V channels keep one slot: their slots are too large
            // for two in the registers)
            // One 64-step round at a time.  Each wave tests its own steps; the masks
            // and the steps' page entries meet in LDS, and the block's candidate slices,
            // in (wave, step) order, are dealt to the waves in turn, so no wave has more
            // than one candidate more than another wherever the kept positions lie.
            // A wave's share goes two at a time: each candidate's K words, norms and
            // every V unit go out together, and the next candidate's go out before the
            // current one is computed (when there is none, the loads repeat a slice
            // already read: the same instructions on every path, so each wait covers
            // only the slot it needs).  Every wave takes part in every round (the
            // block's rounds), and the exchange alternates between two buffers, so a
            // round's writes never meet the previous round's reads.
            __shared__ uint64_t cmask_s[2][kMW];
            __shared__ int cpage_s[2][kMW][64];
            // this wave's share, per owner wave: bit i = the owner's step i
            uint64_t my0 = 0, my1 = 0, my2 = 0, my3 = 0;
            static_assert(kMW == 4, "four owner masks");
            // next candidate of the share as owner * 64 + step, or -1
            auto pop = [&]() __attribute__((always_inline)) -> int {
                int k = -1;
                if (my0) { k = __builtin_ctzll(my0); my0 &= my0 - 1; }
                else if (my1) { k = 64 + __builtin_ctzll(my1); my1 &= my1 - 1; }
                else if (my2) { k = 128 + __builtin_ctzll(my2); my2 &= my2 - 1; }
                else if (my3) { k = 192 + __builtin_ctzll(my3); my3 &= my3 - 1; }
                return k;
            };
            for (int rs = 0; start + rs * kStride < end; rs += 64) {
                const int rbase = first + rs * kStride;
                const int par = (rs >> 6) & 1;
                round_mask(rs, rbase);
                if (lane == 0) cmask_s[par][wave] = cmask;
                cpage_s[par][wave][lane] = cpage;
                lds_barrier();
                {
                    // candidate (owner o, step i) has rank (candidates of owners < o) +
                    // (the owner's candidates below step i); this wave takes the ranks
                    // equal to its index modulo kMW
                    const uint64_t m0 = cmask_s[par][0], m1 = cmask_s[par][1];
                    const uint64_t m2 = cmask_s[par][2], m3 = cmask_s[par][3];
                    auto below = [&](uint64_t m) __attribute__((always_inline)) -> int {
                        return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    };
                    const int b1 = __popcll(m0), b2 = b1 + __popcll(m1), b3 = b2 + __popcll(m2);
                    my0 = __ballot(((m0 >> lane) & 1ull) && ((below(m0)) & (kMW - 1)) == wave);
                    my1 = __ballot(((m1 >> lane) & 1ull) && ((b1 + below(m1)) & (kMW - 1)) == wave);
                    my2 = __ballot(((m2 >> lane) & 1ull) && ((b2 + below(m2)) & (kMW - 1)) == wave);
                    my3 = __ballot(((m3 >> lane) & 1ull) && ((b3 + below(m3)) & (kMW - 1)) == wave);
                }
                int kA = pop(), kB = pop();
                if (kA < 0) continue;   // (wave-uniform)
                // first token of candidate k's slice: the owner's steps start 64 owner
                // tokens into the chunk
                auto cbase = [&](int k) __attribute__((always_inline)) -> int {
                    return start + (k >> 6) * 64 + (rs + (k & 63)) * kStride;
                };
                auto issue_c = [&](Slot &sl, int k) __attribute__((always_inline)) -> int64_t {
                    const int64_t r0 = row0_of(cbase(k), cpage_s[par][k >> 6][k & 63]);
                    load_k(sl, r0);
                    sl.vnl = v_norms[r0 + lane];
                    load_v(sl, r0, all_tokens);
                    return r0;
                };
                auto compute_c = [&](Slot &sl, int k, int64_t r0) __attribute__((always_inline)) {
                    const int base = cbase(k);
                    const float E_s = stage_norms(sl, base);
                    f4_t S[4];
                    score_mfma(sl, S);
                    float s[4][4];
                    scores(S, base, base + 63 <= lim_all, s);
                    gated_values(sl, s, E_s, base, r0, true);
                };
                int64_t rA = issue_c(sa, kA);
                __builtin_amdgcn_sched_barrier(0);
                int64_t rB = issue_c(sb, kB >= 0 ? kB : kA);
                for (;;) {
                    __builtin_amdgcn_sched_barrier(0);
                    compute_c(sa, kA, rA);
                    const int nA = pop();
                    rA = issue_c(sa, nA >= 0 ? nA : kA);
                    __builtin_amdgcn_sched_barrier(0);
                    if (kB < 0) break;
                    compute_c(sb, kB, rB);
                    const int nB = pop();
                    rB = issue_c(sb, nB >= 0 ? nB : kB);
                    kA = nA;
                    kB = nB;
                    if (kA < 0) break;
                }
            }
        } else {
            int step = 0;
            for (int b0 = NB == 1 ? first : start; b0 < end; b0 += kStride, ++step) {
                const int base = NB == 1 ? b0 : b0 + lead;
                if ((step & 63) == 0) round_mask(step, base);
                const bool cand = ((cmask >> (step & 63)) & 1ull) != 0ull;
                if constexpr (NB == 1) {
                    if (!cand) continue;
                }
                int64_t r0 = 0;
                float E_s = 0.f;
                f4_t S[4] = {};
                if (cand) {
                    if constexpr (CONTIG) r0 = row0_of(base, __builtin_amdgcn_readlane(cpage, step & 63));
                    else fill_rows(base, page_of(btab, bsdiv, base + lane, end, a.max_blocks - 1, a.max_page));
                    load_k(sa, r0);
                    if constexpr (CONTIG) sa.vnl = v_norms[r0 + lane];
                    else sa.vnl = v_norms[myrow];
                    E_s = stage_norms(sa, base);
                    score_mfma(sa, S);
                }
                const bool full = base + 63 <= lim_all;
                float s[4][4];
                scores(S, base, full, s);
                if constexpr (NB > 1) {
                    if (!cand) continue;
                }
                gated_values(sa, s, E_s, base, r0, false);
            }
        }
    }

    if constexpr (GATED) {
        if (a.v_rows_read && lane == 0 && v_rows > 0) atomicAdd(a.v_rows_read, (unsigned long long)v_rows);
    }
    // ---------------- merge the waves' partials into the chunk's partial
    if constexpr (WV && PK) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] += dpp<kDppRor8>(acc[j][e]);
        if constexpr (OV) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc_o[e] += dpp<kDppRor8>(acc_o[e]);
        }
    }
    if constexpr (!GATED) {
        if (g == 0) {
            wst[wave][n][0] = m_state;
            wst[wave][n][1] = l_run;
        }
    }
    __syncthreads();   // also: every wave is done with the pair tables
    const bool writer = row_ok && (!PK || n < 8);
    float scale = 1.f, scale_o = 1.f;   // (OV gated: the kept sums are final)
    // (over the waves of this wave's block: one per group)
    if constexpr (!GATED) {
        float M = -INFINITY;
#pragma unroll
        for (int g2 = 0; g2 < NG; ++g2) M = fmaxf(M, wst[blk + NB * g2][n][0]);
        scale = exp2_diff(m_state, M);
        if constexpr (OV) scale_o = exp2_diff(m_raw, M);
        if (grp == 0 && g == 0 && writer) {
            float L = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < NG; ++g2) L += wst[blk + NB * g2][n][1] * exp2_diff(wst[blk + NB * g2][n][0], M);
            part_ml[((part * rp + col_row) * NB + blk) * 2] = M;
            part_ml[((part * rp + col_row) * NB + blk) * 2 + 1] = L;
            if (span > 1) {   // (uniform)
                part_ml[(((part + 1) * rp + col_row) * NB + blk) * 2] = -INFINITY;
                part_ml[(((part + 1) * rp + col_row) * NB + blk) * 2 + 1] = 0.f;
            }
        }
    } else {
        scale = E_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(E_run);
    }
    // part_acc rows are [block][128] (NB blocks), then (OV) the 16 kept-channel sums
    if constexpr (WV && PK) {
        if (writer) {
            float *d = &mbuf[(wave * 8 + col_row) * WRW];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) d[8 * (4 * g + e) + j] = acc[j][e] * scale;
            if constexpr (OV) {
#pragma unroll
                for (int e = 0; e < 4; ++e) d[kD + 4 * g + e] = acc_o[e] * scale_o;
            }
        }
        __syncthreads();
        for (int i = tid; i < R * RW; i += kMBlock) {
            const int row = i / RW, pos = i - row * RW;
            const int bb = NB == 1 ? 0 : pos / kD, e = pos - bb * kD;
            float x = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < NG; ++g2) x += mbuf[((bb + NB * g2) * 8 + row) * WRW + e];
            part_acc[(part * rp + row) * RW + pos] = x;
        }
    } else if constexpr (WV) {
        // every wave's scaled sums to its own rows ([wave][row][WRP]), one barrier,
        // then each element is the sum over the block's groups
        if (writer) {
            float *d = &mbuf[(wave * 16 + col_row) * WRP];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) d[8 * (4 * g + e) + j] = acc[j][e] * scale;
            if constexpr (OV) {
#pragma unroll
                for (int e = 0; e < 4; ++e) d[kD + 4 * g + e] = acc_o[e] * scale_o;
            }
        }
        __syncthreads();
        for (int i = tid; i < R * RW; i += kMBlock) {
            const int row = i / RW, pos = i - row * RW;
            const int bb = NB == 1 ? 0 : pos / kD, e = pos - bb * kD;
            float x = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < NG; ++g2) x += mbuf[((g2 * NB + bb) * 16 + row) * WRP + e];
            part_acc[(part * rp + row) * RW + pos] = x;
        }
    }
}

// The pass kernel.  Items are numbered chunk-major (c * units + unit).  The
// hardware deals consecutive blocks to the XCDs in turn, so with one item per block
// every XCD gets an equal share of each chunk index (with ragged lengths the later
// chunks of a sequence are short or empty; a unit-major order would leave the XCDs
// that receive the first chunks with most of the work), and the full chunks start
// first.  With more items than the GPU holds blocks at once the launch is
// persistent: each block takes items from the work list (non-empty items only,
// chunk-major) through an atomic counter until the list is exhausted, so no block
// slot waits on the dispatcher and the short last chunks fill the end.
// PER: the persistent form (one-block-per-item launches use the form without the
// loop, whose registers stay those of one item).
template <int KB, int VB, bool PK, int MODE, bool CONTIG, int NB, bool OV, bool PER>
__global__ __launch_bounds__(kMBlock) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_eu<PK, VB, MODE>(), 8)))
void tq_decode_mfma_kernel(
    DecodeArgs a, PairTables pt, const uint8_t *__restrict__ k_codes, const float *__restrict__ k_norms,
    const uint8_t *__restrict__ v_codes, const float *__restrict__ v_norms, const uint16_t *__restrict__ qin,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens, float *__restrict__ part_ml,
    float *__restrict__ part_acc, float *__restrict__ tilemax) {
    if constexpr (!PER) {
        // (a gated pass over pairs of the scoring pass's chunks: block = pair * units + unit)
        int item = (int)blockIdx.x, span = 1;
        if constexpr (MODE == MODE_GATED) {
            if (a.gate_pairs) {
                const int pr = (int)fdiv(blockIdx.x, a.units_div);
                item = item + pr * a.n_seqs * a.n_kv;   // (2 pr) * units + unit
                span = 2;
            }
        }
        decode_item<KB, VB, PK, MODE, CONTIG, NB, OV, MODE == MODE_SCORE>(
            item, span, (int)threadIdx.x, a, pt, k_codes, k_norms, v_codes, v_norms, qin, block_table, seq_lens,
            part_ml, part_acc, tilemax);
    } else {
        __shared__ int qitem[2];   // the item the block takes next (two rounds alternate)
        for (int it = 0;; ++it) {
            // (the barrier also ends the previous item's use of the LDS)
            // Blocks of partition p = block mod kListParts take the partition's items
            // t = p, p + kListParts, ... in order: the first round's are the blocks'
            // own indices, later ones come from the partition's counter, so the blocks
            // that finish together spread their atomics over kListParts lines instead
            // of queueing on one.
            if (threadIdx.x == 0) {
                const uint32_t part = blockIdx.x % kListParts;
                uint32_t t = blockIdx.x;
                if (it > 0) {
                    const uint32_t first_round = (gridDim.x - part + kListParts - 1) / kListParts;
                    const uint32_t k = atomicAdd(a.ctrl + (a.pass_slot * kListParts + part) * kCtrlLine, 1u);
                    t = (first_round + k) * kListParts + part;
                }
                qitem[it & 1] = t < a.ctrl[kCtrlCount] ? (int)a.ctrl[kCtrlWords + a.n_seqs * a.n_kv + t] : -1;
            }
            __syncthreads();
            const int entry = __builtin_amdgcn_readfirstlane(qitem[it & 1]);   // (block-uniform)
            if (entry < 0) break;
            const int item = entry & (kListDouble - 1), span = (entry & kListDouble) ? 2 : 1;
            // The thread index passes through an empty asm each round, so nothing
            // derived from it is hoisted out of the loop and held in registers across
            // items (the pass is at its register limit).
            int tid = (int)threadIdx.x;
            asm volatile("" : "+v"(tid));
            decode_item<KB, VB, PK, MODE, CONTIG, NB, OV>(item, span, tid, a, pt, k_codes, k_norms, v_codes, v_norms, qin,
                                                         block_table, seq_lens, part_ml, part_acc, tilemax);
        }
    }
}

// --------------------------------------------------------------------------
// Dispatch, one translation unit per K bit width and blocks per head
// (TQ_DECODE_KB = 2, 3, 4, 16; TQ_DECODE_NB = 1, 2, 4).
// --------------------------------------------------------------------------
// ev0 / ev1 (may be null): recorded at the start and the end of the kernel's
// execution (hipExtLaunchKernelGGL), for timing.
// Blocks of `kern` the current device holds at once (its CUs x the blocks one CU
// holds), looked up once per kernel and device; 0 if the runtime cannot say.
static int resident_blocks(const void *kern) {
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, kern);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kMBlock, 0) != hipSuccess)
        return 0;
    return cache[key] = cus * per_cu;
}

// a.persist on entry: the work list is built for this call; the launch is then
// persistent if the items outnumber the blocks the GPU holds at once (one-block
// heads without kept V channels, K compressed: the shapes long and batched decode
// takes).
// Returns whether the launch is persistent.
template <int KB, int VB, bool PK, bool CONTIG, int NB>
static bool launch_mfma_mode(const DecodeArgs &a, const PairTables &pt, int mode, hipStream_t s, hipEvent_t ev0,
                             hipEvent_t ev1) {
    const int64_t items = (int64_t)a.n_seqs * a.n_kv * a.n_chunks;
    DecodeArgs b = a;
    b.pass_slot = mode == MODE_GATED ? 1 : 0;
    b.persist = 0;
    auto launch = [&](auto kern, int64_t grid) {
        hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMBlock), 0, s, ev0, ev1, 0, b, pt, b.k_codes,
                              b.k_norms, b.v_codes, b.v_norms, b.q, b.block_table, b.seq_lens, b.part_ml, b.part_acc,
                              b.tilemax);
    };
    // one block per item, or (a persistent form given) as many as the GPU holds
    auto go = [&](auto kern, auto kern_persistent) {
        if (mode == MODE_GATED && a.gate_pairs) {   // pairs of chunks, one block each
            launch(kern, (int64_t)a.n_seqs * a.n_kv * ((a.n_chunks + 1) / 2));
            return;
        }
        if constexpr (!std::is_same_v<decltype(kern_persistent), std::nullptr_t>) {
            if (a.persist) {
                const int cap = resident_blocks(reinterpret_cast<const void *>(kern_persistent));
                if (cap >= kListParts && items > cap) {   // (every partition has a block)
                    b.persist = 1;
                    launch(kern_persistent, cap);
                    return;
                }
            }
        }
        launch(kern, items);
    };
    constexpr bool kPer = NB == 1 && KB != 16;
    // (kept V channels: 128-wide heads only, checked on the host)
    const bool ov = NB == 1 && a.n_out > 0;
    if (mode == MODE_DENSE) {
        if (ov) {
            go(tq_decode_mfma_kernel<KB, VB, PK, MODE_DENSE, CONTIG, NB, NB == 1, false>, nullptr);
        } else if constexpr (kPer) {
            go(tq_decode_mfma_kernel<KB, VB, PK, MODE_DENSE, CONTIG, NB, false, false>,
               tq_decode_mfma_kernel<KB, VB, PK, MODE_DENSE, CONTIG, NB, false, true>);
        } else {
            go(tq_decode_mfma_kernel<KB, VB, PK, MODE_DENSE, CONTIG, NB, false, false>, nullptr);
        }
    } else if (mode == MODE_SCORE) {
        if constexpr (kPer)
            go(tq_decode_mfma_kernel<KB, 2, PK, MODE_SCORE, CONTIG, NB, false, false>,
               tq_decode_mfma_kernel<KB, 2, PK, MODE_SCORE, CONTIG, NB, false, true>);
        else
            go(tq_decode_mfma_kernel<KB, 2, PK, MODE_SCORE, CONTIG, NB, false, false>, nullptr);
    } else {
        if (ov) {
            go(tq_decode_mfma_kernel<KB, VB, PK, MODE_GATED, CONTIG, NB, NB == 1, false>, nullptr);
        } else if constexpr (kPer) {
            go(tq_decode_mfma_kernel<KB, VB, PK, MODE_GATED, CONTIG, NB, false, false>,
               tq_decode_mfma_kernel<KB, VB, PK, MODE_GATED, CONTIG, NB, false, true>);
        } else {
            go(tq_decode_mfma_kernel<KB, VB, PK, MODE_GATED, CONTIG, NB, false, false>, nullptr);
        }
    }
    return b.persist != 0;
}

template <int KB, int VB, int NB>
static bool launch_mfma_vb(const DecodeArgs &a, const PairTables &pt, int mode, hipStream_t s, hipEvent_t ev0,
                           hipEvent_t ev1) {
    const bool pk = a.rows <= 8;
    if (a.contig) {
        if (pk) return launch_mfma_mode<KB, VB, true, true, NB>(a, pt, mode, s, ev0, ev1);
        return launch_mfma_mode<KB, VB, false, true, NB>(a, pt, mode, s, ev0, ev1);
    }
    if (pk) return launch_mfma_mode<KB, VB, true, false, NB>(a, pt, mode, s, ev0, ev1);
    return launch_mfma_mode<KB, VB, false, false, NB>(a, pt, mode, s, ev0, ev1);
}

#ifndef TQ_DECODE_NB
#define TQ_DECODE_NB 1
#endif
#define TQ_CAT4(a, b, c, d) a##b##c##d
#define TQ_NAME(a, b, c, d) TQ_CAT4(a, b, c, d)
bool TQ_NAME(launch_mfma_kb, TQ_DECODE_KB, _nb, TQ_DECODE_NB)(const DecodeArgs &a, const PairTables &pt, int mode,
                                                             hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    switch (a.v_bits) {
        case 2: return launch_mfma_vb<TQ_DECODE_KB, 2, TQ_DECODE_NB>(a, pt, mode, s, ev0, ev1);
        case 3: return launch_mfma_vb<TQ_DECODE_KB, 3, TQ_DECODE_NB>(a, pt, mode, s, ev0, ev1);
        default: return launch_mfma_vb<TQ_DECODE_KB, 4, TQ_DECODE_NB>(a, pt, mode, s, ev0, ev1);
    }
}

}  // namespace tq
