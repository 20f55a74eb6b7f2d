// Decode attention over the compressed cache (gfx950, vector ALU only).
//
//   qrot   : per (seq, KV head) rotate the G*n_qtok query rows once,
//            q'' = scale * log2(e) * H (s_K * q) / sqrt(128)            ([llama-tq])
//   pass   : per (seq, KV head, chunk): score every token against its K codes in
//            the Hadamard domain (lane per token, q'' from scalar loads, centroid
//            from an LDS table; K is never dequantized), online softmax in the
//            log2 domain, and either
//              DENSE - accumulate V in the rotated domain: acc += e * n_V * c[code]
//              SCORE - keep only per-chunk (max, sum) and per-64-token tile maxima
//              GATED - with the global (max, sum) known, skip tiles whose bound is
//                      below tau, re-score the rest, and accumulate V only where
//                      p = 2^(s - M) / L >= tau                 ([TQ+ README]
//                      sparse V; [TQ+ article] skipped V treated as zero)
//   stats  : global (max, sum) per row from the SCORE partials
//   merge  : merge chunk partials (log-sum-exp for DENSE, plain sum for GATED),
//            inverse-rotate once: o = s_V * H acc / sqrt(128)
#include <float.h>

#include <atomic>
#include <utility>

#include "tq_decode_common.h"

namespace tq {

#ifndef TQ_DECODE_KB
// --------------------------------------------------------------------------
// q rotation: one wave per row, two elements per lane.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tq_qrot_kernel(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int r = threadIdx.x >> 6;                     // row within (seq, kv)
    const int b = (int)fdiv(blockIdx.x, a.kv_div), kv = blockIdx.x - b * a.n_kv;
    float x0 = 0.f, x1 = 0.f;
    if (r < a.rows) {
        const int jq = (int)fdiv((uint32_t)r, a.grp_div), h = kv * a.group + (r - jq * a.group);
        const uint16_t *q = a.q + (((int64_t)b * a.n_qtok + jq) * a.n_q_heads + h) * kD;
        const uint32_t *sg = a.k_signs + kv * 4;
        x0 = (float)__builtin_bit_cast(_Float16, q[lane]);
        x1 = (float)__builtin_bit_cast(_Float16, q[lane + 64]);
        if ((sg[lane >> 5] >> (lane & 31)) & 1u) x0 = -x0;
        if ((sg[2 + (lane >> 5)] >> (lane & 31)) & 1u) x1 = -x1;
    }
    hadamard128(x0, x1, lane);
    const float a0 = x0, a1 = x1;
    float *dst = a.qrot + ((int64_t)b * a.n_kv + kv) * kD * a.rows_pad;
    dst[lane * a.rows_pad + r] = a0 * a.qscale;
    dst[(lane + 64) * a.rows_pad + r] = a1 * a.qscale;
}

#endif  // !TQ_DECODE_KB

// --------------------------------------------------------------------------
// K scoring of one token per lane.
//
// q'' of the (seq, KV head) is wave-uniform, so it is read with scalar loads
// into SGPRs and used as the SGPR operand of v_fmac.  It is addressed through
// the constant address space (it is read-only for the whole kernel), the base
// pointer is laundered once per sub-chunk so the loads are not hoisted out of
// the token loop, and the 128 positions are walked in groups of P: the loads of
// group g+1 are issued before the FMAs of group g, with scheduling barriers
// between groups so at most two groups of q'' are live in SGPRs.
// --------------------------------------------------------------------------
typedef const __attribute__((address_space(4))) float *cfloat_p;

template <typename T>
__device__ __forceinline__ T launder_sgpr(T p) {
    asm volatile("" : "+s"(p));
    return p;
}

// Positions per q'' group: 32 scalar values per buffer (two buffers live).
template <int RP>
constexpr int score_group() { return RP <= 1 ? 32 : RP <= 2 ? 16 : RP <= 4 ? 8 : RP <= 8 ? 4 : 2; }

// Pull every 64-byte line of q'' into the scalar cache with one round trip, so
// the grouped scalar loads of the scoring loop hit.  16 lines per batch; the
// empty asm consumes the values so the loads are issued and waited here.
template <int RP>
__device__ __forceinline__ void warm_q(cfloat_p qp) {
    constexpr int kLines = kD * RP / 16;          // 16 floats per line
#pragma unroll
    for (int l0 = 0; l0 < kLines; l0 += 16) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = (l0 + j < kLines) ? qp[(l0 + j) * 16] : 0.f;
        asm volatile("" ::"s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]), "s"(v[6]),
                     "s"(v[7]), "s"(v[8]), "s"(v[9]), "s"(v[10]), "s"(v[11]), "s"(v[12]), "s"(v[13]),
                     "s"(v[14]), "s"(v[15]));
    }
}

template <int KB, int RP, int I>
__device__ __forceinline__ void score_pos(const uint32_t *w, const float *q, const float *ktab,
                                          float (&acc)[RP]) {
    const float cv = ktab[stream_code<KB, I>(w)];
#pragma unroll
    for (int r = 0; r < RP; ++r) acc[r] = __builtin_fmaf(q[r], cv, acc[r]);
}

template <int KB, int RP, int P, int G, int... Ps>
__device__ __forceinline__ void score_grp(const uint32_t *w, const float *q, const float *ktab,
                                          float (&acc)[RP], std::integer_sequence<int, Ps...>) {
    (score_pos<KB, RP, G * P + Ps>(w, q + Ps * RP, ktab, acc), ...);
}

template <int RP, int P>
__device__ __forceinline__ void load_q(cfloat_p qp, int g, float (&q)[P * RP]) {
#pragma unroll
    for (int k = 0; k < P * RP; ++k) q[k] = qp[g * P * RP + k];
}

template <int KB, int RP, int P, int G>
__device__ __forceinline__ void score_step_g(const uint32_t *w, cfloat_p qp, float (&qa)[P * RP],
                                             float (&qb)[P * RP], const float *ktab, float (&acc)[RP]) {
    constexpr int NG = kD / P;
    // qa holds group G; prefetch G+1 into qb, then compute G
    if constexpr (G + 1 < NG) load_q<RP, P>(qp, G + 1, qb);
    __builtin_amdgcn_sched_barrier(0);
    score_grp<KB, RP, P, G>(w, qa, ktab, acc, std::make_integer_sequence<int, P>{});
    // the empty volatile asm orders the group's FMAs before the next barrier
#pragma unroll
    for (int r = 0; r < RP; ++r) asm volatile("" : "+v"(acc[r]));
    __builtin_amdgcn_sched_barrier(0);
}

template <int KB, int RP, int P, int... Gs>
__device__ __forceinline__ void score_groups(const uint32_t *w, cfloat_p qp, const float *ktab,
                                             float (&acc)[RP], std::integer_sequence<int, Gs...>) {
    float qa[P * RP], qb[P * RP];
    load_q<RP, P>(qp, 0, qa);
    // alternate the two buffers: even groups compute from qa, odd from qb
    ((Gs % 2 == 0 ? score_step_g<KB, RP, P, Gs>(w, qp, qa, qb, ktab, acc)
                  : score_step_g<KB, RP, P, Gs>(w, qp, qb, qa, ktab, acc)), ...);
}

// V phase layout: LPT lanes per token, each owning PPL consecutive positions.
template <int RP>
constexpr int v_lanes_per_token() { return RP >= 8 ? 32 : 16; }

// Code bits of lane li (positions PPL*li .. PPL*li+PPL-1) of one token's V row
// (global or LDS; the row is 4-byte aligned and 16*VB bytes long).
template <int VB, int PPL>
__device__ __forceinline__ uint32_t v_lane_bits(const uint8_t *row, int li) {
    constexpr int nbits = VB * PPL;
    if constexpr (nbits == 32) {
        return *reinterpret_cast<const uint32_t *>(row + 4 * li);
    } else if constexpr (nbits == 16) {
        return *reinterpret_cast<const uint16_t *>(row + 2 * li);
    } else if constexpr (nbits == 8) {
        return row[li];
    } else {  // 24 or 12 bits: funnel-shift from the two covering dwords of the row
        constexpr int last = (16 * VB) / 4 - 1;
        const int bit = nbits * li, d = bit >> 5, o = bit & 31;
        const uint32_t *w = reinterpret_cast<const uint32_t *>(row);
        const uint32_t lo = w[d], hi = w[d + 1 <= last ? d + 1 : last];
        return __builtin_amdgcn_alignbit(hi, lo, o);
    }
}

template <int VB, int RP, int PPL>
__device__ __forceinline__ void accum_token(uint32_t bits, const float (&wt)[RP], const float *vtab,
                                            float (&acc)[RP][PPL]) {
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        const float cv = vtab[(bits >> (VB * k)) & ((1u << VB) - 1u)];
#pragma unroll
        for (int r = 0; r < RP; ++r) acc[r][k] = __builtin_fmaf(wt[r], cv, acc[r][k]);
    }
}

// Scores of the lane's token for all RP rows (log2 domain), -inf where masked.
template <int KB, int RP>
__device__ __forceinline__ void score_rows(const uint4 (&kw)[KB], float kn, bool active, int t, int last_vis,
                                           const FastDiv &gdiv, cfloat_p qr, const float *ktab, float (&s)[RP]) {
    uint32_t w[4 * KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
        w[4 * i] = kw[i].x; w[4 * i + 1] = kw[i].y; w[4 * i + 2] = kw[i].z; w[4 * i + 3] = kw[i].w;
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) s[r] = 0.f;
    score_groups<KB, RP, score_group<RP>()>(w, launder_sgpr(qr), ktab, s,
                                            std::make_integer_sequence<int, kD / score_group<RP>()>{});
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const bool vis = active && (t <= last_vis + (int)fdiv((uint32_t)r, gdiv));
        s[r] = vis ? s[r] * kn : -INFINITY;
    }
}

// --------------------------------------------------------------------------
// Main pass.  Block = kWaves waves = one (seq, KV head, chunk).  Each wave walks
// its own 64-token slices of the chunk (slice w, w + kWaves, ...) with private
// online-softmax state, private LDS, and the next slice's rows prefetched, so
// no block barrier is needed until the final merge of the waves' partials.
// --------------------------------------------------------------------------
template <int RP>
constexpr int pass_waves_per_eu() { return RP >= 8 ? 2 : 4; }

template <int KB, int VB, int RP, int MODE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(pass_waves_per_eu<RP>(), 8)))
void tq_decode_pass_kernel(DecodeArgs a,
                           const uint8_t *__restrict__ k_codes, const float *__restrict__ k_norms,
                           const uint8_t *__restrict__ v_codes, const float *__restrict__ v_norms,
                           const float *__restrict__ qrot, const int32_t *__restrict__ block_table,
                           const int32_t *__restrict__ seq_lens, const float *__restrict__ tile_in,
                           const float *__restrict__ stats, float *__restrict__ part_ml,
                           float *__restrict__ part_acc, float *__restrict__ tile_out) {
    constexpr bool DENSE = MODE == MODE_DENSE;
    constexpr int RS = RP + 1;                        // padded LDS row stride of the weights
    constexpr int LPT = v_lanes_per_token<RP>();      // V phase: lanes per token
    constexpr int PPL = kD / LPT;                     // V phase: positions per lane
    constexpr int GW = kSlice / LPT;                  // V phase: tokens in flight per wave
    constexpr int VROW = 16 * VB + 4;                 // padded LDS V row (bank spread)
    __shared__ float ktab[TQ_MAX_LEVELS], vtab[TQ_MAX_LEVELS];
    __shared__ float wts[kWaves][kSlice * RS];        // per wave: token weights
    __shared__ __attribute__((aligned(16))) uint8_t vrows[kWaves][DENSE ? kSlice * VROW : 4];
    __shared__ int keep_idx[kWaves][kSlice];
    __shared__ float wstate[kWaves][RP][2];           // per wave: (max, sum) at the end
    __shared__ float accbuf[(MODE == MODE_SCORE) ? 1 : RP * kD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // chunk-major block order (the same as the matrix-core pass)
    const int c = (int)fdiv(blockIdx.x, a.units_div);
    const int bk = blockIdx.x - c * a.n_seqs * a.n_kv;
    const int b = (int)fdiv((uint32_t)bk, a.kv_div), kv = bk - b * a.n_kv;
    const int len = min(seq_lens[b], a.max_blocks * a.block_size);   // (clamped to the table's capacity)
    const int start = c * a.chunk;
    if (start >= len) return;
    const int end = min(start + a.chunk, len);

    if (tid < TQ_MAX_LEVELS) {
        ktab[tid] = a.kc[tid];
        vtab[tid] = a.vc[tid];
    }
    const cfloat_p qr = reinterpret_cast<cfloat_p>(
        reinterpret_cast<uintptr_t>(qrot + ((int64_t)b * a.n_kv + kv) * kD * RP));
    const int32_t *__restrict__ btab = block_table + (int64_t)b * a.max_blocks;
    const int bs = a.block_size;
    const FastDiv bsdiv = a.bs_div;
    const int last_vis = len - a.n_qtok;              // row r sees t <= last_vis + r / G
    const int64_t part = ((int64_t)b * a.n_kv + kv) * a.n_chunks + c;
    const int64_t tile0 = ((int64_t)b * a.n_kv + kv) * a.n_tiles;

    float m_run[RP], l_run[RP], gM[RP], gInvL[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; gM[r] = 0.f; gInvL[r] = 0.f; }
    if constexpr (MODE == MODE_GATED) {
        const float *st = stats + ((int64_t)b * a.n_kv + kv) * RP * 2;
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            gM[r] = in_vgpr(st[2 * r]);
            const float L = st[2 * r + 1];
            gInvL[r] = in_vgpr(L > 0.f ? 1.f / L : 0.f);
        }
    }
    float acc[RP][PPL];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int k = 0; k < PPL; ++k) acc[r][k] = 0.f;

    const int gi = lane / LPT, li = lane % LPT;       // V phase: token group in wave, lane in group
    float *my_w = wts[wave];
    uint8_t *my_v = vrows[wave];
    constexpr int kStride = kWaves * kSlice;           // distance between a wave's slices
    const int first = start + wave * kSlice;

    TokenRows<KB, VB, MODE != MODE_GATED && DENSE> cur;
    int blk_next = 0;
    if constexpr (MODE != MODE_GATED) {
        cur.load(k_codes, k_norms, v_codes, v_norms, bsdiv, bs, a.n_kv, kv, first + lane, end,
                 page_of(btab, bsdiv, first + lane, end, a.max_blocks - 1, a.max_page));
        blk_next = page_of(btab, bsdiv, first + kStride + lane, end, a.max_blocks - 1, a.max_page);
    }
    warm_q<RP>(launder_sgpr(qr));
    __syncthreads();                                   // ktab / vtab

    uint32_t v_rows = 0;   // gated: V rows this wave reads
    for (int base = first; base < end; base += kStride) {   // uniform per wave
        const int t = base + lane;
        float s[RP];
        if constexpr (MODE == MODE_GATED) {
            // tile bound: skip the slice if no row can reach tau with its best score
            const float *tm = tile_in + (tile0 + (base >> 6)) * RP;
            bool cand = false;
#pragma unroll
            for (int r = 0; r < RP; ++r)
                if (r < a.rows) cand |= (exp2_diff(tm[r], gM[r]) * gInvL[r] >= a.tau);
            if (!cand) continue;
            cur.load(k_codes, k_norms, v_codes, v_norms, bsdiv, bs, a.n_kv, kv, t, end,
                     page_of(btab, bsdiv, t, end, a.max_blocks - 1, a.max_page));
            score_rows<KB, RP>(cur.k, cur.kn, cur.active, t, last_vis, a.grp_div, qr, ktab, s);
            bool kept = false;
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                const float p = exp2_diff(s[r], gM[r]) * gInvL[r];
                const bool k = (r < a.rows) && p >= a.tau && p > 0.f;
                my_w[lane * RS + r] = k ? p : 0.f;
                kept |= k;
            }
            const uint64_t bal = __ballot(kept);
            const int total = __popcll(bal);
            v_rows += total;
            if (kept) keep_idx[wave][__popcll(bal & ((1ull << lane) - 1ull))] = lane;
            __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0): this wave's LDS writes done
            __builtin_amdgcn_wave_barrier();
            for (int q = gi; q < total; q += GW) {
                const int tt = keep_idx[wave][q];
                const int tk = base + tt;
                const uint32_t pg = fdiv((uint32_t)tk, bsdiv);
                const int blk = btab[pg];
                const int64_t row = ((int64_t)blk * a.n_kv + kv) * bs + (tk - (int)pg * bs);
                const uint32_t bits = v_lane_bits<VB, PPL>(v_codes + row * (16 * VB), li);
                const float nv = v_norms[row];
                float wt[RP];
#pragma unroll
                for (int r = 0; r < RP; ++r) wt[r] = my_w[tt * RS + r] * nv;
                accum_token<VB, RP, PPL>(bits, wt, vtab, acc);
            }
            __builtin_amdgcn_wave_barrier();
        } else {
            // ---------------- K phase: one token per lane, rows loaded one slice ahead
            score_rows<KB, RP>(cur.k, cur.kn, cur.active, t, last_vis, a.grp_div, qr, ktab, s);
            const float vn = cur.vn;
            if constexpr (DENSE) {
#pragma unroll
                for (int i = 0; i < VB; ++i) {
                    uint32_t *d = reinterpret_cast<uint32_t *>(my_v + lane * VROW) + 4 * i;
                    d[0] = cur.v[i].x; d[1] = cur.v[i].y; d[2] = cur.v[i].z; d[3] = cur.v[i].w;
                }
            }
            if (base + kStride < end) {
                cur.load(k_codes, k_norms, v_codes, v_norms, bsdiv, bs, a.n_kv, kv, t + kStride, end, blk_next);
                blk_next = page_of(btab, bsdiv, t + 2 * kStride, end, a.max_blocks - 1, a.max_page);
            }
            // ---------------- online softmax over the wave's slice
            float e[RP];
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                const float wm = wave_max(s[r]);
                if constexpr (MODE == MODE_SCORE) {
                    if (lane == r) tile_out[(tile0 + (base >> 6)) * RP + r] = wm;
                }
                const float m_new = in_vgpr(fmaxf(m_run[r], wm));
                const float alpha = exp2_diff(m_run[r], m_new);
                e[r] = exp2_diff(s[r], m_new);
                l_run[r] = in_vgpr(l_run[r] * alpha + wave_sum(e[r]));
                m_run[r] = m_new;
                if constexpr (DENSE) {
                    my_w[lane * RS + r] = e[r] * vn;   // V norm folded into the weight
#pragma unroll
                    for (int k = 0; k < PPL; ++k) acc[r][k] *= alpha;
                }
            }
            if constexpr (DENSE) {
                __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): weights and V rows in LDS
                __builtin_amdgcn_wave_barrier();
                // ---------------- V phase from LDS: GW tokens at a time, LPT lanes per token
                const int n_tok = min(kSlice, end - base);
#pragma unroll 2
                for (int tt = gi; tt < n_tok; tt += GW) {
                    const uint32_t bits = v_lane_bits<VB, PPL>(my_v + tt * VROW, li);
                    float wt[RP];
#pragma unroll
                    for (int r = 0; r < RP; ++r) wt[r] = my_w[tt * RS + r];
                    accum_token<VB, RP, PPL>(bits, wt, vtab, acc);
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
    }

    if constexpr (MODE == MODE_GATED) {
        if (a.v_rows_read && lane == 0 && v_rows > 0) atomicAdd(a.v_rows_read, (unsigned long long)v_rows);
    }
    // ---------------- merge the waves' partials and write the chunk's result
    if constexpr (MODE != MODE_GATED) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                wstate[wave][r][0] = m_run[r];
                wstate[wave][r][1] = l_run[r];
            }
        }
    }
    __syncthreads();
    float scale[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        scale[r] = 1.f;
        if constexpr (MODE != MODE_GATED) {
            float M = -INFINITY;
#pragma unroll
            for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, wstate[w2][r][0]);
            scale[r] = exp2_diff(m_run[r], M);
            if (tid == 0) {
                float L = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < kWaves; ++w2) L += wstate[w2][r][1] * exp2_diff(wstate[w2][r][0], M);
                part_ml[(part * RP + r) * 2] = M;
                part_ml[(part * RP + r) * 2 + 1] = L;
            }
        }
    }
    if constexpr (MODE != MODE_SCORE) {
        // sum the token groups of each wave, then the waves in order through LDS
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int k = 0; k < PPL; ++k) {
                float x = acc[r][k] * scale[r];
                if constexpr (LPT == 16) x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                acc[r][k] = x;
            }
        for (int w2 = 0; w2 < kWaves; ++w2) {
            if (wave == w2 && lane < LPT) {
#pragma unroll
                for (int r = 0; r < RP; ++r)
#pragma unroll
                    for (int k = 0; k < PPL; ++k) {
                        float *d = &accbuf[r * kD + PPL * lane + k];
                        *d = (w2 == 0) ? acc[r][k] : *d + acc[r][k];
                    }
            }
            __syncthreads();
        }
        float *dst = part_acc + part * RP * kD;
        for (int i = tid; i < RP * kD; i += kBlock) dst[i] = accbuf[i];
    }
}

#ifndef TQ_DECODE_KB
// --------------------------------------------------------------------------
// Global (max, sum) per row for the sparse path.  One block per (seq, KV head);
// each wave reduces rows wave, wave+4, ... with its lanes striding the chunks.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tq_stats_kernel(DecodeArgs a) {
    const int b = (int)fdiv(blockIdx.x, a.kv_div), kv = blockIdx.x - b * a.n_kv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int len = a.seq_lens[b];
    // (a length past the table's capacity is clamped to the chunks the workspace holds)
    const int nc = min((int)fdiv((uint32_t)(len + a.chunk - 1), a.chunk_div), a.n_chunks);
    const float *ml = a.part_ml + ((int64_t)b * a.n_kv + kv) * a.n_chunks * a.rows_pad * 2;
    for (int r = wave; r < a.rows_pad; r += 4) {
        float m = -INFINITY;
        for (int c = lane; c < nc; c += 64) m = fmaxf(m, ml[(c * a.rows_pad + r) * 2]);
        const float M = wave_max(m);
        float l = 0.f;
        for (int c = lane; c < nc; c += 64)
            l += ml[(c * a.rows_pad + r) * 2 + 1] * exp2_diff(ml[(c * a.rows_pad + r) * 2], M);
        const float L = wave_sum(l);
        if (lane == 0) {
            float *st = a.stats + (((int64_t)b * a.n_kv + kv) * a.rows_pad + r) * 2;
            st[0] = M;
            st[1] = L;
        }
    }
}

// --------------------------------------------------------------------------
// Merge the chunk partials of one 128-element block of one output row and
// inverse-rotate it (both pass kernels write the same partial layout: per chunk
// and row, (max, sum) per head block and acc_w floats: the accumulator
// [block][128], then, with kept V channels, their 16 sums, which replace the
// rotated result at their channels).  One block per (row, head block): 8 chunk
// groups x 32 float4 columns (+ 4 columns of kept sums).  Dense: each thread merges its chunks (c = group,
// group + 8, ...) with the log-sum-exp rule in batches of 16 loads, then the
// groups are merged through LDS and o = s_V * H (acc / L) / sqrt(128).  Gated:
// the partials are already normalised and are summed.
// --------------------------------------------------------------------------
// KEPT: the V side keeps channels (a.n_out > 0); KB: chunks per thread per round
// of loads (2, 4, 8 or 16: the smallest with 8 KB >= n_chunks, so a row's loads are
// one round and the registers, hence the blocks per CU, follow the chunk count)
template <bool SPARSE, bool KEPT, int KB>
__global__ __launch_bounds__(256) void tq_merge_kernel(DecodeArgs a) {
    typedef float f4_t __attribute__((ext_vector_type(4)));
    __shared__ float gm[8], gl[8];
    __shared__ __attribute__((aligned(16))) float gx[8][kD + 16];
    __shared__ float y[kD + 16];
    __shared__ int32_t cslot[kD];   // kept channel -> its slot, or -1
    const int tid = threadIdx.x, lane = tid & 63;
    const int cg = tid >> 5, q4 = tid & 31;
    const int nb = a.nb, hb = blockIdx.x & (nb - 1);      // head block (nb a power of two)
    const uint32_t row_id = blockIdx.x >> a.nb_log2;
    const int bj = (int)fdiv(row_id, a.qh_div);            // b * n_qtok + jq
    const int h = (int)row_id - bj * a.n_q_heads;
    const int b = (int)fdiv((uint32_t)bj, a.qt_div);
    const int jq = bj - b * a.n_qtok;
    const int kv = (int)fdiv((uint32_t)h, a.grp_div);
    const int r = jq * a.group + (h - kv * a.group);
    const int64_t base = ((int64_t)b * a.n_kv + kv) * a.n_chunks;
    const int n_out = KEPT ? a.n_out : 0;   // (head blocks and kept channels do not meet: nb = 1 then)
    if (tid < kD) cslot[tid] = -1;
    // the output stage's sign words and kept-channel indices, loaded up front
    const uint32_t *sg = a.v_signs + (kv * nb + hb) * 4;
    const uint32_t sgw0 = sg[(lane >> 5) & 1], sgw1 = sg[2 + ((lane >> 5) & 1)];
    int oidx = 0;
    if constexpr (KEPT) oidx = a.v_out_idx[kv * 16 + min(tid, 15)];
    // (merge_step 2: only the even chunk slots hold partials)
    const int step = a.merge_step;
    const int64_t mstride = (int64_t)a.rows_pad * nb * 2 * step, astride = (int64_t)a.rows_pad * a.acc_w * step;
    const float *ml = a.part_ml + ((base * a.rows_pad + r) * nb + hb) * 2;                // chunk c at ml[c * mstride]
    const float *pa = a.part_acc + (base * a.rows_pad + r) * a.acc_w + hb * kD + 4 * q4;  // chunk c at pa[c * astride]
    const bool xo = KEPT && q4 < 4;   // this thread also merges kept sums 4 q4 .. 4 q4 + 3
    // kept sums of the row (threads with q4 >= 4 read those of q4 = 3, unused)
    const float *pa2 = pa - 4 * q4 + kD + 4 * min(q4, 3);
    float M = -INFINITY, L = 0.f;
    f4_t x = {0.f, 0.f, 0.f, 0.f}, x2 = {0.f, 0.f, 0.f, 0.f};
    constexpr int kB = KB;   // chunks per thread per batch (one round of loads)
    typedef float f2_t __attribute__((ext_vector_type(2)));
    f2_t mlr[kB];
    float m[kB], l[kB];
    f4_t v[kB], v2[kB];
    // One round: chunks c0, c0 + 8, ..., every load issued (indices clamped below
    // `issue`, so no load sits behind a branch and each waits only where it is used);
    // then those at or past `lim` are replaced by empty ones.
    auto load_round = [&](int c0, int issue) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const int ci = min(c0 + 8 * i, issue - 1);
            if constexpr (!SPARSE) mlr[i] = *reinterpret_cast<const f2_t *>(ml + ci * mstride);
            v[i] = *reinterpret_cast<const f4_t *>(pa + ci * astride);
        }
        if constexpr (KEPT) {
#pragma unroll
            for (int i = 0; i < kB; ++i)
                v2[i] = *reinterpret_cast<const f4_t *>(pa2 + min(c0 + 8 * i, issue - 1) * astride);
        } else {
#pragma unroll
            for (int i = 0; i < kB; ++i) v2[i] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto mask_round = [&](int c0, int lim) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const bool ok = c0 + 8 * i < lim;
            m[i] = (!SPARSE && ok) ? mlr[i].x : -INFINITY;
            l[i] = (!SPARSE && ok) ? mlr[i].y : 0.f;
            v[i] = ok ? v[i] : f4_t{0.f, 0.f, 0.f, 0.f};
            v2[i] = (ok && xo) ? v2[i] : f4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto fold_round = [&]() __attribute__((always_inline)) {
        if (SPARSE) {
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                x += v[i];
                x2 += v2[i];
            }
        } else {
            float mb = M;
#pragma unroll
            for (int i = 0; i < kB; ++i) mb = fmaxf(mb, m[i]);
            const float sc = exp2_diff(M, mb);
            x *= sc;
            x2 *= sc;
            L *= sc;
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                const float f = exp2_diff(m[i], mb);
                x += f * v[i];
                x2 += f * v2[i];
                L += f * l[i];
            }
            M = mb;
        }
    };
    // The first round goes out before the sequence length is read: every chunk the
    // workspace holds for this row (n_chunks >= 1) is loaded, and those past the
    // sequence's own chunks (not written by this call) are then dropped.
    load_round(cg, min((a.n_chunks + step - 1) / step, 8 * kB));
    __builtin_amdgcn_sched_barrier(0);
    const int len = a.seq_lens[b];
    // (clamped to the chunks the workspace holds, whatever the length; counted in slots)
    const int nc = len > 0 ? (min((int)fdiv((uint32_t)(len + a.chunk - 1), a.chunk_div), a.n_chunks) + step - 1) / step
                           : 0;
    mask_round(cg, nc);
    fold_round();
    for (int c0 = cg + 8 * kB; c0 < nc; c0 += 8 * kB) {
        load_round(c0, nc);
        mask_round(c0, nc);
        fold_round();
    }
    if (q4 == 0) {
        gm[cg] = M;
        gl[cg] = L;
    }
    *reinterpret_cast<f4_t *>(&gx[cg][4 * q4]) = x;
    if (xo) *reinterpret_cast<f4_t *>(&gx[cg][kD + 4 * q4]) = x2;
    __syncthreads();
    const int ny = kD + (n_out > 0 ? 16 : 0);
    if (tid < ny) {
        float Mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 8; ++k) Mx = fmaxf(Mx, gm[k]);
        float ys = 0.f, Ls = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float f = SPARSE ? 1.f : exp2_diff(gm[k], Mx);
            ys += f * gx[k][tid];
            Ls += f * gl[k];
        }
        y[tid] = SPARSE ? ys : (Ls > 0.f ? ys / Ls : 0.f);
    }
    if (tid < n_out) cslot[oidx & (kD - 1)] = tid;
    __syncthreads();
    if (tid >= 64) return;
    // o = s_V * H acc / sqrt(128)
    float a0 = y[lane], a1 = y[lane + 64];
    hadamard128(a0, a1, lane);
    const float k = 0.088388347648318440550f;
    a0 *= ((sgw0 >> (lane & 31)) & 1u) ? -k : k;
    a1 *= ((sgw1 >> (lane & 31)) & 1u) ? -k : k;
    if (n_out > 0) {   // kept channels: their own sums
        const int s0 = cslot[lane], s1 = cslot[lane + 64];
        if (s0 >= 0) a0 = y[kD + s0];
        if (s1 >= 0) a1 = y[kD + s1];
    }
    float *o = a.out + ((((int64_t)b * a.n_qtok + jq) * a.n_q_heads + h) * nb + hb) * kD;
    o[lane] = a0;
    o[lane + 64] = a1;
}

// --------------------------------------------------------------------------
// Merge for few chunk slots (at most KS in the workspace, no kept V channels): one
// block takes 8 consecutive (row, head block) outputs t, 32 float4 columns each, and
// every thread merges all chunk slots of its column in one round of loads (issued
// before the sequence length is read; slots past the sequence's own are then
// dropped).  Same log-sum-exp rule and output stage as tq_merge_kernel, without
// the chunk groups and their LDS reduction, and with about one block per 8
// outputs instead of one per output: ragged batches of short sequences are many
// rows with a handful of partials each.
// --------------------------------------------------------------------------
template <bool SPARSE, int KS>
__global__ __launch_bounds__(256) void tq_merge_rows_kernel(DecodeArgs a, uint32_t n_out_rows) {
    typedef float f4_t __attribute__((ext_vector_type(4)));
    typedef float f2_t __attribute__((ext_vector_type(2)));
    __shared__ __attribute__((aligned(16))) float y[8][kD + 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rr = tid >> 5, q4 = tid & 31;
    const int nb = a.nb;
    // this thread's output t = (row, head block), row = (b, jq, h)
    const uint32_t t = min(blockIdx.x * 8u + (uint32_t)rr, n_out_rows - 1);
    const int hb = (int)(t & (uint32_t)(nb - 1));
    const uint32_t row_id = t >> a.nb_log2;
    const int bj = (int)fdiv(row_id, a.qh_div);
    const int h = (int)row_id - bj * a.n_q_heads;
    const int b = (int)fdiv((uint32_t)bj, a.qt_div);
    const int jq = bj - b * a.n_qtok;
    const int kv = (int)fdiv((uint32_t)h, a.grp_div);
    const int r = jq * a.group + (h - kv * a.group);
    const int64_t base = ((int64_t)b * a.n_kv + kv) * a.n_chunks;
    const int step = a.merge_step;   // 2: only the even chunk slots hold partials
    const int64_t mstride = (int64_t)a.rows_pad * nb * 2 * step, astride = (int64_t)a.rows_pad * a.acc_w * step;
    const float *ml = a.part_ml + ((base * a.rows_pad + r) * nb + hb) * 2;
    const float *pa = a.part_acc + (base * a.rows_pad + r) * a.acc_w + hb * kD + 4 * q4;
    const int slots = (a.n_chunks + step - 1) / step;   // <= KS
    f2_t mlr[KS];
    f4_t v[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        const int ci = min(i, slots - 1);
        if constexpr (!SPARSE) mlr[i] = *reinterpret_cast<const f2_t *>(ml + ci * mstride);
        v[i] = *reinterpret_cast<const f4_t *>(pa + ci * astride);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int len = a.seq_lens[b];
    const int nc = len > 0 ? (min((int)fdiv((uint32_t)(len + a.chunk - 1), a.chunk_div), a.n_chunks) + step - 1) / step
                           : 0;
    f4_t x = {0.f, 0.f, 0.f, 0.f};
    if constexpr (SPARSE) {
#pragma unroll
        for (int i = 0; i < KS; ++i) x += i < nc ? v[i] : f4_t{0.f, 0.f, 0.f, 0.f};
    } else {
        float M = -INFINITY, L = 0.f;
#pragma unroll
        for (int i = 0; i < KS; ++i) M = fmaxf(M, i < nc ? mlr[i].x : -INFINITY);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            const float f = i < nc ? exp2_diff(mlr[i].x, M) : 0.f;
            x += f * (i < nc ? v[i] : f4_t{0.f, 0.f, 0.f, 0.f});
            L += f * (i < nc ? mlr[i].y : 0.f);
        }
        x = L > 0.f ? x / L : f4_t{0.f, 0.f, 0.f, 0.f};
    }
    *reinterpret_cast<f4_t *>(&y[rr][4 * q4]) = x;
    __syncthreads();
    // o = s_V * H y / sqrt(128): wave w takes outputs 2w and 2w + 1 of the block
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int ro = 2 * wave + k;
        const uint32_t to = blockIdx.x * 8u + (uint32_t)ro;
        if (to >= n_out_rows) break;
        const int hbo = (int)(to & (uint32_t)(nb - 1));
        const uint32_t hro = to >> a.nb_log2;
        const int ho = (int)hro - (int)fdiv(hro, a.qh_div) * a.n_q_heads;
        const int kvo = (int)fdiv((uint32_t)ho, a.grp_div);
        const uint32_t *sg = a.v_signs + (kvo * nb + hbo) * 4;
        const uint32_t sgw0 = sg[(lane >> 5) & 1], sgw1 = sg[2 + ((lane >> 5) & 1)];
        float a0 = y[ro][lane], a1 = y[ro][lane + 64];
        hadamard128(a0, a1, lane);
        const float kk = 0.088388347648318440550f;
        a0 *= ((sgw0 >> (lane & 31)) & 1u) ? -kk : kk;
        a1 *= ((sgw1 >> (lane & 31)) & 1u) ? -kk : kk;
        float *o = a.out + (int64_t)to * kD;
        o[lane] = a0;
        o[lane + 64] = a1;
    }
}

// --------------------------------------------------------------------------
// Work list of the persistent matrix-core passes, one block: the non-empty
// (chunk, unit) items in chunk-major order (every unit's chunk 0, then chunk 1,
// ...), so the full chunks are taken first and the short last chunks of ragged
// sequences last.  With a.pair the items of the first part are pairs of chunks
// (2p, 2p + 1), pair-major, and the last chunk of every unit with an odd count
// follows as an item of its own: long items first, a tail of short ones.  Units
// are counting-sorted by their item count k(u) (decreasing): the units with more
// than c items are then a prefix of that order, cnt[c] of them, and item row c is
// list[off[c] .. off[c] + cnt[c]).  Also zeroes the passes' item counters.
// (n_chunks <= kMaxListChunks.)
// --------------------------------------------------------------------------
// Exclusive prefix sum of v[0 .. n) in place by wave 0 (16 elements per lane at a
// time); returns the total in every lane of wave 0.
__device__ int wave0_exclusive_scan(int *v, int n) {
    const int lane = threadIdx.x & 63;
    int carry = 0;
    for (int base = 0; base < n; base += 64 * 16) {
        int loc[16], sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = base + lane * 16 + i;
            loc[i] = k < n ? v[k] : 0;
            sum += loc[i];
        }
        int incl = sum;   // inclusive scan of the lane sums
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        int run = carry + incl - sum;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = base + lane * 16 + i;
            if (k < n) v[k] = run;
            run += loc[i];
        }
        carry += __shfl(incl, 63);
    }
    return carry;
}

__global__ __launch_bounds__(1024) void tq_worklist_kernel(DecodeArgs a) {
    constexpr int kUnitsHeld = 4;               // units per thread whose counts stay in registers
    constexpr int kSortedLds = 1024 * kUnitsHeld;   // units whose sorted order stays in LDS
    __shared__ int hist[kMaxListChunks + 2];   // units with k(u) = k
    __shared__ int cnt[kMaxListChunks + 2];    // units with k(u) > c
    __shared__ int off[kMaxListChunks + 2];    // first list entry of item row c
    __shared__ int fill[kMaxListChunks + 2];
    __shared__ int sorted_l[kSortedLds];
    __shared__ int n_single;
    const int tid = threadIdx.x, nch = a.n_chunks, n_units = a.n_seqs * a.n_kv;
    const bool pair = a.pair != 0;
    const int nk = pair ? nch / 2 : nch;       // item rows of the first part
    const bool in_lds = n_units <= kSortedLds;
    int32_t *const sorted = reinterpret_cast<int32_t *>(a.ctrl + kCtrlWords);   // (more units)
    int32_t *const list = sorted + n_units;
    const int cap = a.max_blocks * a.block_size;
    auto nc_of = [&](int u) {   // chunks holding tokens of unit u
        const int b = (int)fdiv((uint32_t)u, a.kv_div);
        const int len = min(max(a.seq_lens[b], 0), cap);
        return min((int)fdiv((uint32_t)(len + a.chunk - 1), a.chunk_div), nch);
    };
    // the chunk counts of this thread's first units (u = tid + 1024 i), read once
    int ncr[kUnitsHeld];
#pragma unroll
    for (int i = 0; i < kUnitsHeld; ++i) ncr[i] = tid + 1024 * i < n_units ? nc_of(tid + 1024 * i) : 0;
    auto nc_at = [&](int i, int u) { return i < kUnitsHeld ? ncr[i] : nc_of(u); };   // u = tid + 1024 i
    auto k_at = [&](int i, int u) { return pair ? nc_at(i, u) >> 1 : nc_at(i, u); };
    for (int i = tid; i <= nk + 1; i += 1024) {
        hist[i] = 0;
        fill[i] = 0;
    }
    if (tid == 0) n_single = 0;
    __syncthreads();
    for (int u = tid, i = 0; u < n_units; u += 1024, ++i) atomicAdd(&hist[k_at(i, u)], 1);
    __syncthreads();
    // cnt[c] = sum of hist[k] over k > c, as an exclusive scan of the reversed
    // histogram; off = exclusive scan of cnt
    for (int i = tid; i <= nk; i += 1024) cnt[i] = hist[nk - i];
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(cnt, nk + 1);   // cnt[i] = units with k > nk - i
    __syncthreads();
    for (int i = tid; i <= nk; i += 1024) off[i] = cnt[nk - i];   // units with k > i
    __syncthreads();
    for (int i = tid; i <= nk; i += 1024) cnt[i] = off[i];
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(off, nk + 1);   // off[nk] = items of the first part
    __syncthreads();
    // units in order of decreasing k: those with k(u) = k take positions
    // [cnt[k], cnt[k] + hist[k]) (the order inside a group does not matter)
    for (int u = tid, i = 0; u < n_units; u += 1024, ++i) {
        const int k = k_at(i, u);
        if (k > 0) {
            const int pos = cnt[k] + atomicAdd(&fill[k], 1);
            if (in_lds) sorted_l[pos] = u;
            else sorted[pos] = u;
        }
    }
    __threadfence_block();
    __syncthreads();
    const int n_main = off[nk];
    for (int t = tid; t < n_main; t += 1024) {
        int lo = 0, hi = nk - 1;   // the last c with off[c] <= t
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int u = in_lds ? sorted_l[t - off[lo]] : sorted[t - off[lo]];
        list[t] = pair ? ((2 * lo) * n_units + u) | kListDouble : lo * n_units + u;
    }
    // pairs: the odd last chunks, after every pair
    if (pair) {
        for (int u = tid, i = 0; u < n_units; u += 1024, ++i) {
            const int f = nc_at(i, u);
            if (f & 1) list[n_main + atomicAdd(&n_single, 1)] = (f - 1) * n_units + u;
        }
    }
    __syncthreads();
    if (tid < 2 * kListParts) a.ctrl[tid * kCtrlLine] = 0u;
    if (tid == 0) a.ctrl[kCtrlCount] = (uint32_t)(n_main + n_single);
}

#endif  // !TQ_DECODE_KB

// --------------------------------------------------------------------------
// Dispatch.  The pass kernels are instantiated per K bit width in separate
// translation units (this file compiled with TQ_DECODE_KB=2, 3, 4) so the
// build runs in parallel; the unit without TQ_DECODE_KB holds the rest.
// --------------------------------------------------------------------------
// ev0 / ev1 (may be null): recorded at the start and the end of the pass kernel's
// execution (hipExtLaunchKernelGGL), for timing.
void launch_pass_kb2(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
void launch_pass_kb3(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
void launch_pass_kb4(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

#ifdef TQ_DECODE_KB
template <int KB, int VB, int RP>
static void launch_pass(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const dim3 grid((unsigned)((int64_t)a.n_seqs * a.n_kv * a.n_chunks));
#define TQ_PASS_ARGS a, a.k_codes, a.k_norms, a.v_codes, a.v_norms, a.qrot, a.block_table, a.seq_lens, \
        a.tilemax, a.stats, a.part_ml, a.part_acc, a.tilemax
    if (mode == MODE_DENSE)
        hipExtLaunchKernelGGL((tq_decode_pass_kernel<KB, VB, RP, MODE_DENSE>), grid, dim3(kBlock), 0, s, ev0, ev1, 0,
                              TQ_PASS_ARGS);
    else if (mode == MODE_SCORE)
        hipExtLaunchKernelGGL((tq_decode_pass_kernel<KB, 2, RP, MODE_SCORE>), grid, dim3(kBlock), 0, s, ev0, ev1, 0,
                              TQ_PASS_ARGS);
    else
        hipExtLaunchKernelGGL((tq_decode_pass_kernel<KB, VB, RP, MODE_GATED>), grid, dim3(kBlock), 0, s, ev0, ev1, 0,
                              TQ_PASS_ARGS);
#undef TQ_PASS_ARGS
}

template <int KB, int VB>
static void launch_pass_rp(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    switch (a.rows_pad) {
        case 1: launch_pass<KB, VB, 1>(a, mode, s, ev0, ev1); break;
        case 2: launch_pass<KB, VB, 2>(a, mode, s, ev0, ev1); break;
        case 4: launch_pass<KB, VB, 4>(a, mode, s, ev0, ev1); break;
        case 8: launch_pass<KB, VB, 8>(a, mode, s, ev0, ev1); break;
        case 12: launch_pass<KB, VB, 12>(a, mode, s, ev0, ev1); break;
        default: launch_pass<KB, VB, 16>(a, mode, s, ev0, ev1); break;
    }
}

template <int KB>
static void launch_pass_vb(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    switch (a.v_bits) {
        case 2: launch_pass_rp<KB, 2>(a, mode, s, ev0, ev1); break;
        case 3: launch_pass_rp<KB, 3>(a, mode, s, ev0, ev1); break;
        default: launch_pass_rp<KB, 4>(a, mode, s, ev0, ev1); break;
    }
}

#define TQ_CAT2(a, b) a##b
#define TQ_CAT(a, b) TQ_CAT2(a, b)
void TQ_CAT(launch_pass_kb, TQ_DECODE_KB)(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0,
                                          hipEvent_t ev1) {
    launch_pass_vb<TQ_DECODE_KB>(a, mode, s, ev0, ev1);
}

#else

#define TQ_DECL_MFMA(KB, NB)                                                                                  \
    bool launch_mfma_kb##KB##_nb##NB(const DecodeArgs &a, const PairTables &pt, int mode, hipStream_t s,        \
                                     hipEvent_t ev0, hipEvent_t ev1);
#define TQ_DECL_MFMA_KB(KB) TQ_DECL_MFMA(KB, 1) TQ_DECL_MFMA(KB, 2) TQ_DECL_MFMA(KB, 4)
TQ_DECL_MFMA_KB(2)
TQ_DECL_MFMA_KB(3)
TQ_DECL_MFMA_KB(4)
TQ_DECL_MFMA_KB(16)   // K float16
#undef TQ_DECL_MFMA_KB
#undef TQ_DECL_MFMA

// Returns whether the pass launch is persistent.
static bool launch_mfma_any(const DecodeArgs &a, const PairTables &pt, int mode, hipStream_t s,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
#define TQ_CASE_NB(KB)                                                                  \
    switch (a.nb) {                                                                     \
        case 2: return launch_mfma_kb##KB##_nb2(a, pt, mode, s, ev0, ev1);              \
        case 4: return launch_mfma_kb##KB##_nb4(a, pt, mode, s, ev0, ev1);              \
        default: return launch_mfma_kb##KB##_nb1(a, pt, mode, s, ev0, ev1);             \
    }
    switch (a.k_bits) {
        case 2: TQ_CASE_NB(2)
        case 3: TQ_CASE_NB(3)
        case 16: TQ_CASE_NB(16)
        default: TQ_CASE_NB(4)
    }
#undef TQ_CASE_NB
}

static void launch_pass_any(const DecodeArgs &a, int mode, hipStream_t s, hipEvent_t ev0 = nullptr,
                            hipEvent_t ev1 = nullptr) {
    switch (a.k_bits) {
        case 2: launch_pass_kb2(a, mode, s, ev0, ev1); break;
        case 3: launch_pass_kb3(a, mode, s, ev0, ev1); break;
        default: launch_pass_kb4(a, mode, s, ev0, ev1); break;
    }
}

template <bool SPARSE, int KB>
static void launch_merge_kb(const DecodeArgs &a, dim3 grid, hipStream_t s) {
    if (a.n_out > 0) hipLaunchKernelGGL((tq_merge_kernel<SPARSE, true, KB>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((tq_merge_kernel<SPARSE, false, KB>), grid, dim3(256), 0, s, a);
}

template <bool SPARSE>
static void launch_merge(const DecodeArgs &a, dim3 grid, hipStream_t s) {
    const int slots = (a.n_chunks + a.merge_step - 1) / a.merge_step;
    if (a.n_out == 0 && slots <= 8) {   // few partials per row: 8 outputs per block
        const dim3 g((grid.x + 7) / 8);
        if (slots <= 4) hipLaunchKernelGGL((tq_merge_rows_kernel<SPARSE, 4>), g, dim3(256), 0, s, a, grid.x);
        else hipLaunchKernelGGL((tq_merge_rows_kernel<SPARSE, 8>), g, dim3(256), 0, s, a, grid.x);
        return;
    }
    if (a.n_chunks <= 16) launch_merge_kb<SPARSE, 2>(a, grid, s);
    else if (a.n_chunks <= 32) launch_merge_kb<SPARSE, 4>(a, grid, s);
    else if (a.n_chunks <= 64) launch_merge_kb<SPARSE, 8>(a, grid, s);
    else launch_merge_kb<SPARSE, 16>(a, grid, s);
}

// CUs of the current device (looked up once per device; 0 if unknown).
static int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

hipError_t launch_decode(const DecodeArgs &a, const PairTables &pt, hipStream_t s, hipEvent_t ev_before,
                         hipEvent_t ev_after) {
    const dim3 rows_grid((unsigned)((int64_t)a.n_seqs * a.n_qtok * a.n_q_heads * a.nb));   // x head blocks
    if (a.mfma) {   // q rotation runs inside the pass kernels
        // More (chunk, unit) items than two blocks per CU: build the work list of the
        // persistent passes (each pass launch then decides from its own occupancy).
        DecodeArgs b = a;
        b.persist = 0;
        const int64_t items = (int64_t)a.n_seqs * a.n_kv * a.n_chunks;
        const int cus = device_cus();
        if (a.ctrl && cus > 0 && items > 2 * (int64_t)cus && !a.gate_pairs) {
            hipLaunchKernelGGL(tq_worklist_kernel, dim3(1), dim3(1024), 0, s, a);
            b.persist = 1;
        }
        // (a persistent pass over a paired list, and a gated pass over pairs of chunks,
        // leave their partials in the even chunk slots only: the merge reads those)
        DecodeArgs m = a;
        if (a.tau > 0.f) {
            launch_mfma_any(b, pt, MODE_SCORE, s, ev_before, ev_after);
            m.merge_step = (launch_mfma_any(b, pt, MODE_GATED, s) && a.pair) || a.gate_pairs ? 2 : 1;
            launch_merge<true>(m, rows_grid, s);
        } else {
            m.merge_step = launch_mfma_any(b, pt, MODE_DENSE, s, ev_before, ev_after) && a.pair ? 2 : 1;
            launch_merge<false>(m, rows_grid, s);
        }
        return hipGetLastError();
    }
    hipLaunchKernelGGL(tq_qrot_kernel, dim3(a.n_seqs * a.n_kv), dim3(64 * a.rows_pad), 0, s, a);
    if (a.tau > 0.f) {
        launch_pass_any(a, MODE_SCORE, s, ev_before, ev_after);
        hipLaunchKernelGGL(tq_stats_kernel, dim3(a.n_seqs * a.n_kv), dim3(256), 0, s, a);
        launch_pass_any(a, MODE_GATED, s);
        launch_merge<true>(a, rows_grid, s);
    } else {
        launch_pass_any(a, MODE_DENSE, s, ev_before, ev_after);
        launch_merge<false>(a, rows_grid, s);
    }
    return hipGetLastError();
}

#endif

}  // namespace tq
