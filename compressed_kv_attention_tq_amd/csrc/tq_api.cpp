// C ABI of libtq: argument validation, codebook construction, workspace sizing
// and kernel dispatch.  Everything here runs on the host; nothing allocates.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "tq_internal.h"

using namespace tq;

namespace {

bool is_aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Round a double to the nearest float16 value (ties to even), returned as double.
double round_to_half(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(fabs(x), &e);               // |x| = m * 2^e, m in [0.5, 1)
    int E = e - 1;                    // |x| in [2^E, 2^(E+1))
    if (E < -14) E = -14;             // subnormal spacing 2^-24
    const double ulp = ldexp(1.0, E - 10);
    const double q = nearbyint(fabs(x) / ulp);
    return copysign(q * ulp, x);
}

double std_normal_cdf(double z) {
    if (isinf(z)) return z > 0 ? 1.0 : 0.0;
    return 0.5 * erfc(-z / sqrt(2.0));
}

double std_normal_pdf(double z) {
    if (isinf(z)) return 0.0;
    return exp(-0.5 * z * z) / sqrt(2.0 * M_PI);
}

// Expected squared error of a scalar quantizer on N(0, sigma^2), cell by cell in
// closed form: on a standardised cell [a, b] with centre c,
//   int (x-c)^2 phi = (1 + c^2)(Phi(b) - Phi(a)) + (a - 2c) phi(a) - (b - 2c) phi(b).
double gaussian_mse(const double *c, const double *bnd, int L, double sigma) {
    double tot = 0.0;
    for (int j = 0; j < L; ++j) {
        const double a = j == 0 ? -INFINITY : bnd[j - 1] / sigma;
        const double b = j == L - 1 ? INFINITY : bnd[j] / sigma;
        const double cj = c[j] / sigma;
        const double mass = std_normal_cdf(b) - std_normal_cdf(a);
        const double ta = isinf(a) ? 0.0 : (a - 2.0 * cj) * std_normal_pdf(a);
        const double tb = isinf(b) ? 0.0 : (b - 2.0 * cj) * std_normal_pdf(b);
        tot += (1.0 + cj * cj) * mass + ta - tb;
    }
    return tot * sigma * sigma;
}

tq_status check_codebook(const tq_codebook &cb, int bits) {
    if (cb.bits != bits || cb.n_levels != (1 << bits)) return TQ_ERR_INVALID_ARG;
    for (int i = 0; i < cb.n_levels; ++i)
        if (!isfinite(cb.centroids[i])) return TQ_ERR_INVALID_ARG;
    for (int i = 0; i + 1 < cb.n_levels; ++i) {
        if (!isfinite(cb.boundaries[i])) return TQ_ERR_INVALID_ARG;
        if (i > 0 && !(cb.boundaries[i] > cb.boundaries[i - 1])) return TQ_ERR_INVALID_ARG;
    }
    return TQ_OK;
}

// 128-element blocks per head; heads of 128, 256 or 512 elements are supported
int blocks_per_head(const tq_cache *c) { return c->head_dim / TQ_HEAD_DIM; }

// cache sub-heads: block i of head j is sub-head nb j + i
int sub_heads(const tq_cache *c) { return c->n_kv_heads * blocks_per_head(c); }

tq_status check_cache(const tq_cache *c) {
    if (!c) return TQ_ERR_INVALID_ARG;
    if (c->head_dim != TQ_HEAD_DIM && c->head_dim != 2 * TQ_HEAD_DIM && c->head_dim != 4 * TQ_HEAD_DIM)
        return TQ_ERR_UNSUPPORTED;
    const bool fp16 = c->bits == TQ_BITS_FP16;
    if (!fp16 && (c->bits < 2 || c->bits > 4)) return TQ_ERR_UNSUPPORTED;
    if (c->n_kv_heads < 1 || c->block_size < 1 || c->n_blocks < 1) return TQ_ERR_INVALID_ARG;
    if (!c->codes || !is_aligned(c->codes, 16)) return TQ_ERR_INVALID_ARG;
    // slots are handled as 32-bit values on the device
    if ((double)c->n_blocks * c->block_size > 2147483647.0) return TQ_ERR_UNSUPPORTED;
    if (c->n_outliers < 0 || c->n_outliers > TQ_MAX_OUTLIERS) return TQ_ERR_INVALID_ARG;
    if (c->n_outliers > 0) {
        if (fp16 || c->head_dim != TQ_HEAD_DIM) return TQ_ERR_UNSUPPORTED;
        if (!c->outlier_channels || !is_aligned(c->outlier_channels, 16) || !c->outliers ||
            !is_aligned(c->outliers, 8))
            return TQ_ERR_INVALID_ARG;
    }
    if (fp16) return TQ_OK;   // rows of float16: no norms, signs or codebook
    if (!c->norms || !c->signs || !is_aligned(c->norms, 4) || !is_aligned(c->signs, 4)) return TQ_ERR_INVALID_ARG;
    return check_codebook(c->cb, c->bits);
}

// Groups of 8 vectors each quantize wave takes in a row: when n_kv divides 8 (the
// vector path's groups of 8 then hold whole tokens), or, for a side the matrix-core
// transform quantizes (compressed, no kept channels), when n_kv divides its tiles
// of 16 vectors.
constexpr int kQuantGroups = 4;
int quant_gpw(int n_kv, bool mfma_side) {
    if (n_kv <= 0) return 0;
    return (8 % n_kv == 0 || (mfma_side && 16 % n_kv == 0)) ? kQuantGroups : 0;
}

// Encode grid for one codebook: cells of width 1/grid in y, at most one boundary
// per (slightly widened) cell; the table covers y in [-1, 1] (|y| <= 1 because y
// is a rotated unit vector).
tq_status fill_quant_side(const tq_cache *c, const void *src, int64_t stride, int32_t n_tokens,
                          QuantSide &q) {
    // (a head of several blocks is quantized as that many sub-heads of 128)
    if (c->bits == TQ_BITS_FP16) {   // the rows are stored as they come
        q.src = static_cast<const uint16_t *>(src);
        q.codes = c->codes;
        q.src_stride = stride;
        q.n_vec = (int64_t)n_tokens * sub_heads(c);
        q.n_tokens = n_tokens;
        q.cap = c->n_blocks * c->block_size;
        q.gpw = quant_gpw(sub_heads(c), false);
        q.n_kv = sub_heads(c);
        q.block_size = c->block_size;
        q.bits = c->bits;
        q.bs_div = make_fastdiv((uint32_t)c->block_size);
        q.kv_div = make_fastdiv((uint32_t)sub_heads(c));
        return TQ_OK;
    }
    double min_gap = INFINITY;
    const int nb = c->cb.n_levels - 1;
    for (int i = 0; i + 1 < nb; ++i) min_gap = std::min(min_gap, (double)c->cb.boundaries[i + 1] - c->cb.boundaries[i]);
    int grid = 1;
    if (nb > 1) {
        const double g = ceil(1.25 / min_gap);
        if (!(g <= (kLutMax - 5) / 2)) return TQ_ERR_UNSUPPORTED;
        grid = std::max(1, (int)g);
    }
    q.src = static_cast<const uint16_t *>(src);
    q.codes = c->codes;
    q.norms = c->norms;
    q.signs = c->signs;
    q.src_stride = stride;
    q.n_vec = (int64_t)n_tokens * sub_heads(c);
    q.n_tokens = n_tokens;
    q.cap = c->n_blocks * c->block_size;
    q.gpw = quant_gpw(sub_heads(c), c->n_outliers == 0);
    q.n_kv = sub_heads(c);
    q.block_size = c->block_size;
    q.bits = c->bits;
    q.grid = (float)grid;
    q.lut_half = grid + 2;
    q.bs_div = make_fastdiv((uint32_t)c->block_size);
    q.kv_div = make_fastdiv((uint32_t)sub_heads(c));
    q.n_bnd = nb;
    for (int i = 0; i < TQ_MAX_LEVELS - 1; ++i) q.bnd[i] = i < nb ? c->cb.boundaries[i] : 0.f;
    q.n_out = c->n_outliers;
    q.out_idx = c->outlier_channels;
    q.outliers = c->outliers;
    return TQ_OK;
}

int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// Blocks for one quantize side (4 waves per block).  With gpw > 0 (quant_gpw) every
// wave takes kQuantGroups consecutive groups of 8 vectors; otherwise at most 512
// blocks (with both sides, about 4 waves per SIMD, each pipelining several
// groups), rounded so the grid stride is a multiple of n_kv.
int quant_blocks(int64_t n_vec, int n_kv, int gpw) {
    if (n_vec == 0) return 0;
    if (gpw > 0) return (int)((n_vec + 32 * kQuantGroups - 1) / (32 * kQuantGroups));
    const int64_t need = (n_vec + 31) / 32;
    int blocks = (int)std::min<int64_t>(need, 512);
    const int m = n_kv / gcd_int(n_kv, 32);
    blocks = std::max(m, (blocks / m) * m);
    return blocks;
}

struct DecodePlan {
    int rows, rows_pad, chunk, n_chunks, n_tiles;
    size_t off_qrot, off_ml, off_acc, off_tile, off_stats, off_ctrl, total;
    bool list;   // the workspace holds a work list (persistent matrix-core passes)
    bool pair;   // the list pairs chunks (the library's chunk, halved)
    bool gate_pairs;   // sparse: the gated pass takes pairs of chunks
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Tokens per pass block: a multiple of the unit (one 64-token slice per wave),
// doubled while at least kTargetBlocks blocks remain and at most 16384 tokens;
// chunk_opt > 0 (a multiple of the unit, checked by the caller) overrides it.
DecodePlan plan_decode(int n_seqs, int n_kv, int nb, int acc_w, int rows, int max_blocks, int block_size,
                       bool sparse, bool mfma, int chunk_opt) {
    DecodePlan p{};
    p.rows = rows;
    if (mfma) p.rows_pad = rows <= 8 ? 8 : 16;
    else p.rows_pad = rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : rows <= 12 ? 12 : 16;
    const int64_t cap = (int64_t)max_blocks * block_size;
    const int64_t total = (int64_t)n_seqs * n_kv * cap;
    const int unit = mfma ? kMBlock : kChunkUnit;
    const int64_t target = 512;
    int chunk = unit;
    while (chunk < 16384 && total / (2 * chunk) >= target) chunk *= 2;
    // Matrix-core pass with more items than two blocks per CU of the largest GPUs
    // hold (a persistent launch): half the chunk, taken in pairs by the work list,
    // so the items are as long but the last ones half as long.
    p.pair = false;
    p.gate_pairs = false;
    if (chunk_opt > 0) {
        chunk = chunk_opt;
    } else if (mfma && chunk >= 2 * unit && (int64_t)n_seqs * n_kv * ((cap + chunk - 1) / chunk) > 2 * target) {
        chunk /= 2;
        p.pair = true;
    } else if (mfma && sparse && nb == 1) {
        // Sparse V, one block per item: the scoring pass holds three blocks per CU and
        // the gated pass two, so the chunks are sized for about three scoring blocks per
        // CU of the largest GPUs and the gated pass takes them in pairs.
        const int64_t want = 3 * target / 2;
        const int64_t cs = ((total + want - 1) / want + unit - 1) / unit * unit;
        chunk = (int)std::min<int64_t>(std::max<int64_t>(cs, unit), 16384);
        p.gate_pairs = true;
    }
    p.chunk = chunk;
    p.n_chunks = (int)((cap + chunk - 1) / chunk);
    p.n_tiles = p.n_chunks * (chunk / kSlice);
    const size_t units = (size_t)n_seqs * n_kv;
    size_t off = 0;
    p.off_qrot = off;  if (!mfma) off = align256(off + units * kD * p.rows_pad * sizeof(float));
    p.off_ml = off;    off = align256(off + units * p.n_chunks * p.rows_pad * nb * 2 * sizeof(float));
    p.off_acc = off;   off = align256(off + units * p.n_chunks * p.rows_pad * acc_w * sizeof(float));
    p.off_tile = off;  if (sparse) off = align256(off + units * p.n_tiles * p.rows_pad * sizeof(float));
    p.off_stats = off; if (sparse && !mfma) off = align256(off + units * p.rows_pad * 2 * sizeof(float));
    // control words, units by chunk count, (chunk, unit) items
    const int64_t items = (int64_t)units * p.n_chunks;
    p.list = mfma && p.n_chunks <= kMaxListChunks && items <= kMaxListItems;
    p.off_ctrl = off;  if (p.list) off = align256(off + (kCtrlWords + units + items) * sizeof(uint32_t));
    p.total = off;
    return p;
}

// float16 bits -> double (exact)
double half_to_double(uint16_t h) {
    const int e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m | 1024), e - 25);
    return (h >> 15) ? -v : v;
}

// In-place unnormalised Walsh-Hadamard transform of 128 values, natural order.
void fwht128(double *x) {
    for (int h = 1; h < 128; h <<= 1)
        for (int i = 0; i < 128; i += 2 * h)
            for (int k = i; k < i + h; ++k) {
                const double a = x[k], b = x[k + h];
                x[k] = a + b;
                x[k + h] = a - b;
            }
}

}  // namespace

extern "C" {

const char *tq_status_string(tq_status s) {
    switch (s) {
        case TQ_OK: return "TQ_OK";
        case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
        case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
        case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
        case TQ_ERR_HIP: return "TQ_ERR_HIP";
    }
    return "TQ_ERR_UNKNOWN";
}

tq_status tq_build_codebook(int32_t bits, double sigma, tq_codebook *out) {
    if (!out) return TQ_ERR_INVALID_ARG;
    if (!(sigma > 0.0) || !isfinite(sigma)) return TQ_ERR_INVALID_ARG;
    if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
    const int L = 1 << bits;
    double c[TQ_MAX_LEVELS], cn[TQ_MAX_LEVELS], bnd[TQ_MAX_LEVELS];
    // standardised units; uniform start on [-2, 2]
    for (int j = 0; j < L; ++j) c[j] = -2.0 + 4.0 * j / (L - 1);
    for (int it = 0; it < 20000; ++it) {
        for (int j = 0; j + 1 < L; ++j) bnd[j] = 0.5 * (c[j] + c[j + 1]);
        for (int j = 0; j < L; ++j) {
            const double lo = j == 0 ? -INFINITY : bnd[j - 1];
            const double hi = j == L - 1 ? INFINITY : bnd[j];
            const double mass = std_normal_cdf(hi) - std_normal_cdf(lo);
            cn[j] = (std_normal_pdf(lo) - std_normal_pdf(hi)) / mass;
        }
        double moved = 0.0;
        for (int j = 0; j < L; ++j) {
            const double v = 0.5 * (cn[j] - cn[L - 1 - j]);
            moved = std::max(moved, fabs(v - c[j]));
            bnd[j] = v;   // temporary
        }
        for (int j = 0; j < L; ++j) c[j] = bnd[j];
        if (moved < 1e-14) break;
    }
    memset(out, 0, sizeof(*out));
    out->bits = bits;
    out->n_levels = L;
    out->sigma = (float)sigma;
    double cs[TQ_MAX_LEVELS], bs[TQ_MAX_LEVELS];
    for (int j = 0; j < L; ++j) cs[j] = round_to_half(c[j] * sigma);
    for (int j = 0; j < L; ++j) cs[j] = 0.5 * (cs[j] - cs[L - 1 - j]);
    for (int j = 0; j + 1 < L; ++j) bs[j] = 0.5 * (cs[j] + cs[j + 1]);
    for (int j = 0; j < L; ++j) out->centroids[j] = (float)cs[j];
    for (int j = 0; j + 1 < L; ++j) out->boundaries[j] = (float)bs[j];
    out->mse = gaussian_mse(cs, bs, L, sigma);
    return TQ_OK;
}

tq_status tq_fit_codebook(int32_t bits, const uint16_t *vectors, int64_t n_vectors, int32_t n_heads,
                          const uint32_t *signs, int32_t max_iter, tq_codebook *out) {
    if (!out || !vectors || !signs || n_vectors < 1 || n_heads < 1 || max_iter < 1) return TQ_ERR_INVALID_ARG;
    if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
    const int L = 1 << bits;
    const double sigma = 1.0 / sqrt(128.0);
    // samples: the rotated coordinates of every nonzero, finite vector
    std::vector<double> ys;
    ys.reserve((size_t)n_vectors * 128);
    double x[128];
    for (int64_t i = 0; i < n_vectors; ++i) {
        const uint16_t *v = vectors + i * 128;
        const uint32_t *sw = signs + (i % n_heads) * 4;
        double ss = 0.0;
        bool finite = true;
        for (int k = 0; k < 128; ++k) {
            x[k] = half_to_double(v[k]);
            finite = finite && isfinite(x[k]);
            ss += x[k] * x[k];
        }
        if (!finite || !(ss > 0.0)) continue;
        const double inv = 1.0 / sqrt(ss);
        for (int k = 0; k < 128; ++k) x[k] = (((sw[k >> 5] >> (k & 31)) & 1u) ? -x[k] : x[k]) * inv;
        fwht128(x);
        for (int k = 0; k < 128; ++k) ys.push_back(x[k] * sigma);
    }
    if (ys.empty()) return TQ_ERR_INVALID_ARG;
    // cells are runs of the sorted samples: each round is a search per boundary
    std::sort(ys.begin(), ys.end());
    const size_t n = ys.size();
    std::vector<double> s1(n + 1, 0.0), s2(n + 1, 0.0);
    for (size_t k = 0; k < n; ++k) {
        s1[k + 1] = s1[k] + ys[k];
        s2[k + 1] = s2[k] + ys[k] * ys[k];
    }
    tq_codebook init;
    tq_build_codebook(bits, sigma, &init);
    double c[TQ_MAX_LEVELS];
    for (int j = 0; j < L; ++j) c[j] = init.centroids[j];
    size_t idx[TQ_MAX_LEVELS + 1], prev[TQ_MAX_LEVELS + 1];
    for (int it = 0; it < max_iter; ++it) {
        // assignment: a sample above the midpoint of two centres goes to the upper
        idx[0] = 0;
        idx[L] = n;
        for (int j = 0; j + 1 < L; ++j)
            idx[j + 1] = (size_t)(std::upper_bound(ys.begin(), ys.end(), 0.5 * (c[j] + c[j + 1])) - ys.begin());
        if (it > 0 && std::equal(idx, idx + L + 1, prev)) break;   // stable: done
        std::copy(idx, idx + L + 1, prev);
        // update: each centre moves to the mean of its samples (an empty cell keeps its centre)
        for (int j = 0; j < L; ++j)
            if (idx[j + 1] > idx[j]) c[j] = (s1[idx[j + 1]] - s1[idx[j]]) / (double)(idx[j + 1] - idx[j]);
    }
    memset(out, 0, sizeof(*out));
    out->bits = bits;
    out->n_levels = L;
    out->sigma = (float)sigma;
    double cs[TQ_MAX_LEVELS], bs[TQ_MAX_LEVELS];
    for (int j = 0; j < L; ++j) cs[j] = round_to_half(c[j]);
    for (int j = 0; j + 1 < L; ++j) bs[j] = 0.5 * (cs[j] + cs[j + 1]);
    for (int j = 0; j < L; ++j) out->centroids[j] = (float)cs[j];
    for (int j = 0; j + 1 < L; ++j) out->boundaries[j] = (float)bs[j];
    // mean squared error of the samples under the stored codebook
    double err = 0.0;
    size_t lo = 0;
    for (int j = 0; j < L; ++j) {
        const size_t hi = j + 1 < L ? (size_t)(std::upper_bound(ys.begin(), ys.end(), bs[j]) - ys.begin()) : n;
        err += (s2[hi] - s2[lo]) - 2.0 * cs[j] * (s1[hi] - s1[lo]) + (double)(hi - lo) * cs[j] * cs[j];
        lo = hi;
    }
    out->mse = err / (double)n;
    return TQ_OK;
}

tq_status tq_select_outlier_channels(const uint16_t *vectors, int64_t n_vectors, int32_t n_heads, int32_t k,
                                     uint8_t *channels) {
    if (!vectors || !channels || n_vectors < 1 || n_heads < 1 || k < 1 || k > TQ_MAX_OUTLIERS)
        return TQ_ERR_INVALID_ARG;
    // sums of squares per (head, channel) over the finite vectors
    std::vector<double> ss((size_t)n_heads * 128, 0.0);
    double x[128];
    for (int64_t i = 0; i < n_vectors; ++i) {
        const uint16_t *v = vectors + i * 128;
        bool finite = true;
        for (int c = 0; c < 128; ++c) {
            x[c] = half_to_double(v[c]);
            finite = finite && isfinite(x[c]);
        }
        if (!finite) continue;
        double *acc = ss.data() + (size_t)(i % n_heads) * 128;
        for (int c = 0; c < 128; ++c) acc[c] += x[c] * x[c];
    }
    // the count of a head's vectors is the same for all its channels: sums rank as means
    for (int h = 0; h < n_heads; ++h) {
        const double *acc = ss.data() + (size_t)h * 128;
        int order[128];
        for (int c = 0; c < 128; ++c) order[c] = c;
        std::stable_sort(order, order + 128, [&](int a, int b) { return acc[a] > acc[b]; });
        std::sort(order, order + k);
        uint8_t *out = channels + (size_t)h * 16;
        for (int s = 0; s < 16; ++s) out[s] = s < k ? (uint8_t)order[s] : 0;
    }
    return TQ_OK;
}

tq_status tq_quantize_kv(const tq_cache *k, const void *k_src, const tq_cache *v, const void *v_src,
                         int64_t src_token_stride, int32_t n_tokens, const int64_t *slot_mapping,
                         void *stream) {
    if (n_tokens < 0) return TQ_ERR_INVALID_ARG;
    const tq_cache *sides[2] = {k, v};
    const void *srcs[2] = {k_src, v_src};
    QuantArgs a;
    memset(&a, 0, sizeof(a));
    int n_kv = -1, head_dim = -1;
    for (int i = 0; i < 2; ++i) {
        if (!sides[i]) continue;
        tq_status st = check_cache(sides[i]);
        if (st != TQ_OK) return st;
        if (!srcs[i] || !is_aligned(srcs[i], 16)) return TQ_ERR_INVALID_ARG;
        if (!is_aligned(sides[i]->codes, 8)) return TQ_ERR_INVALID_ARG;
        if (n_kv >= 0 && (n_kv != sides[i]->n_kv_heads || head_dim != sides[i]->head_dim)) return TQ_ERR_INVALID_ARG;
        n_kv = sides[i]->n_kv_heads;
        head_dim = sides[i]->head_dim;
        if (src_token_stride < (int64_t)n_kv * head_dim || src_token_stride % 8 != 0) return TQ_ERR_INVALID_ARG;
        st = fill_quant_side(sides[i], srcs[i], src_token_stride, n_tokens, a.side[i]);
        if (st != TQ_OK) return st;
    }
    if (n_tokens == 0 || n_kv < 0) return TQ_OK;
    if (!slot_mapping) return TQ_ERR_INVALID_ARG;
    if ((int64_t)n_tokens * n_kv * (head_dim / kD) > (1LL << 31) - (1LL << 20)) return TQ_ERR_UNSUPPORTED;
    const int bk = quant_blocks(a.side[0].n_vec, std::max(1, a.side[0].n_kv), a.side[0].gpw);
    const int bv = quant_blocks(a.side[1].n_vec, std::max(1, a.side[1].n_kv), a.side[1].gpw);
    a.slots = slot_mapping;
    a.blocks_k = bk;
    if (launch_quantize(a, bk + bv, static_cast<hipStream_t>(stream)) != hipSuccess) return TQ_ERR_HIP;
    return TQ_OK;
}

tq_status tq_dequantize(const tq_cache *c, const int64_t *slots, int32_t n_tokens, void *dst,
                        int32_t dst_is_fp16, void *stream) {
    tq_status st = check_cache(c);
    if (st != TQ_OK) return st;
    if (n_tokens < 0) return TQ_ERR_INVALID_ARG;
    if (n_tokens == 0) return TQ_OK;
    if (!slots || !dst || !is_aligned(dst, 16) || !is_aligned(c->codes, 8)) return TQ_ERR_INVALID_ARG;
    if ((int64_t)n_tokens * sub_heads(c) > (1LL << 31) - (1LL << 20)) return TQ_ERR_UNSUPPORTED;
    // a head of several blocks is that many sub-heads of 128: dst [n_tokens][n_kv][nb][128]
    DequantArgs a;
    memset(&a, 0, sizeof(a));
    a.codes = c->codes;
    a.norms = c->norms;
    a.signs = c->signs;
    a.slots = slots;
    a.dst = dst;
    a.n_vec = (int64_t)n_tokens * sub_heads(c);
    a.cap = c->n_blocks * c->block_size;
    a.n_kv = sub_heads(c);
    a.block_size = c->block_size;
    a.dst_fp16 = dst_is_fp16 ? 1 : 0;
    a.kv_div = make_fastdiv((uint32_t)sub_heads(c));
    a.bs_div = make_fastdiv((uint32_t)c->block_size);
    if (c->bits != TQ_BITS_FP16)
        for (int i = 0; i < TQ_MAX_LEVELS; ++i) a.cent[i] = i < c->cb.n_levels ? c->cb.centroids[i] : 0.f;
    a.n_out = c->n_outliers;
    a.out_idx = c->outlier_channels;
    a.outliers = c->outliers;
    if (launch_dequantize(a, c->bits, static_cast<hipStream_t>(stream)) != hipSuccess) return TQ_ERR_HIP;
    return TQ_OK;
}

tq_status tq_decode_attention(const tq_cache *k, const tq_cache *v, const void *q, int32_t n_seqs,
                              int32_t n_qtok, int32_t n_q_heads, const int32_t *seq_lens,
                              const int32_t *block_table, int32_t max_blocks_per_seq,
                              float softmax_scale, float sparse_v_tau, float *out, void *workspace,
                              size_t *workspace_bytes, void *stream) {
    return tq_decode_attention_ex(k, v, q, n_seqs, n_qtok, n_q_heads, seq_lens, block_table, max_blocks_per_seq,
                                  softmax_scale, sparse_v_tau, out, workspace, workspace_bytes, stream, nullptr,
                                  nullptr);
}

}  // extern "C"

namespace {

// The new tokens of a fused append (tq_append_decode_attention), or none.
struct AppendIn {
    const void *k_new, *v_new;
    int64_t stride;
};

tq_status decode_impl(const tq_cache *k, const tq_cache *v, const void *q, int32_t n_seqs, int32_t n_qtok,
                      int32_t n_q_heads, const int32_t *seq_lens, const int32_t *block_table,
                      int32_t max_blocks_per_seq, float softmax_scale, float sparse_v_tau, float *out,
                      void *workspace, size_t *workspace_bytes, void *stream, const tq_decode_options *opts,
                      void *const *events, const AppendIn *app) {
    if (!workspace_bytes) return TQ_ERR_INVALID_ARG;
    // the kernel and the chunk of this call (explicit options; no process state)
    const int kern = opts ? opts->kernel : TQ_DECODE_KERNEL_DEFAULT;
    if (kern != TQ_DECODE_KERNEL_DEFAULT && kern != TQ_DECODE_KERNEL_MFMA && kern != TQ_DECODE_KERNEL_VALU)
        return TQ_ERR_INVALID_ARG;
    const bool mfma = kern != TQ_DECODE_KERNEL_VALU;
    const int chunk_opt = opts ? opts->chunk : 0;
    if (chunk_opt != 0 && (chunk_opt < 0 || chunk_opt > (1 << 20) || chunk_opt % (mfma ? kMBlock : kChunkUnit) != 0))
        return TQ_ERR_INVALID_ARG;
    tq_status st = check_cache(k);
    if (st != TQ_OK) return st;
    st = check_cache(v);
    if (st != TQ_OK) return st;
    if (k->n_kv_heads != v->n_kv_heads || k->block_size != v->block_size || k->head_dim != v->head_dim)
        return TQ_ERR_INVALID_ARG;
    // float16 K and heads of several blocks need the matrix-core pass; V is always
    // a compressed side
    const bool k_fp16 = k->bits == TQ_BITS_FP16;
    const int nb = blocks_per_head(k);
    const bool v_out = v->n_outliers > 0;
    if (k->n_outliers > 0) return TQ_ERR_UNSUPPORTED;
    if (v->bits == TQ_BITS_FP16 || ((k_fp16 || nb > 1 || v_out) && !mfma)) return TQ_ERR_UNSUPPORTED;
    if (!is_aligned(v->codes, 4)) return TQ_ERR_INVALID_ARG;
    if (n_seqs < 0 || n_qtok < 1 || n_q_heads < 1 || max_blocks_per_seq < 1) return TQ_ERR_INVALID_ARG;
    if (n_q_heads % k->n_kv_heads != 0) return TQ_ERR_INVALID_ARG;
    if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale)) return TQ_ERR_INVALID_ARG;
    if (!(sparse_v_tau >= 0.f) || !isfinite(sparse_v_tau)) return TQ_ERR_INVALID_ARG;
    const int group = n_q_heads / k->n_kv_heads;
    const int64_t rows = (int64_t)group * n_qtok;
    if (rows > TQ_MAX_ROWS_PER_KV_HEAD) return TQ_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks_per_seq * k->block_size > (1LL << 30)) return TQ_ERR_UNSUPPORTED;
    // cache rows are indexed with 32-bit integers on the device
    if ((double)k->n_blocks * sub_heads(k) * k->block_size > 2147483647.0 ||
        (double)v->n_blocks * sub_heads(v) * v->block_size > 2147483647.0)
        return TQ_ERR_UNSUPPORTED;
    const bool sparse = sparse_v_tau > 0.f;
    if (app) {   // the fused append: matrix-core pass, 128-wide heads, compressed K, V without kept channels
        if (!mfma || nb != 1 || k_fp16 || v_out) return TQ_ERR_UNSUPPORTED;
        if (!app->k_new || !app->v_new || !is_aligned(app->k_new, 16) || !is_aligned(app->v_new, 16))
            return TQ_ERR_INVALID_ARG;
        if (app->stride < (int64_t)k->n_kv_heads * kD || app->stride % 8 != 0) return TQ_ERR_INVALID_ARG;
        if (!is_aligned(k->codes, 8) || !is_aligned(v->codes, 8)) return TQ_ERR_INVALID_ARG;
    }
    const int acc_w = nb * kD + (v_out ? TQ_MAX_OUTLIERS : 0);
    const DecodePlan p = plan_decode(n_seqs, k->n_kv_heads, nb, acc_w, (int)rows, max_blocks_per_seq,
                                     k->block_size, sparse, mfma, chunk_opt);
    if ((int64_t)n_seqs * k->n_kv_heads * p.n_chunks > 0x7FFFFFFFLL) return TQ_ERR_UNSUPPORTED;
    if (!workspace) {
        *workspace_bytes = n_seqs == 0 ? 0 : p.total;
        return TQ_OK;
    }
    if (n_seqs == 0) return TQ_OK;
    if (!q || !seq_lens || !block_table || !out) return TQ_ERR_INVALID_ARG;
    if (!is_aligned(workspace, 256) || !is_aligned(out, 4) || !is_aligned(q, 2)) return TQ_ERR_INVALID_ARG;
    if (*workspace_bytes < p.total) return TQ_ERR_WORKSPACE;

    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.k_codes = k->codes;
    a.k_norms = k->norms;
    a.v_codes = v->codes;
    a.v_norms = v->norms;
    a.k_signs = k->signs;
    a.v_signs = v->signs;
    a.q = static_cast<const uint16_t *>(q);
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.out = out;
    char *ws = static_cast<char *>(workspace);
    a.qrot = mfma ? nullptr : reinterpret_cast<float *>(ws + p.off_qrot);
    a.part_ml = reinterpret_cast<float *>(ws + p.off_ml);
    a.part_acc = reinterpret_cast<float *>(ws + p.off_acc);
    a.tilemax = sparse ? reinterpret_cast<float *>(ws + p.off_tile) : nullptr;
    a.stats = (sparse && !mfma) ? reinterpret_cast<float *>(ws + p.off_stats) : nullptr;
    a.ctrl = p.list ? reinterpret_cast<uint32_t *>(ws + p.off_ctrl) : nullptr;
    a.persist = 0;
    a.pass_slot = 0;
    a.pair = p.pair && p.list ? 1 : 0;
    a.merge_step = 1;
    a.gate_pairs = p.gate_pairs ? 1 : 0;
    a.n_seqs = n_seqs;
    a.n_qtok = n_qtok;
    a.n_q_heads = n_q_heads;
    a.n_kv = k->n_kv_heads;
    a.group = group;
    a.rows = (int)rows;
    a.rows_pad = p.rows_pad;
    a.max_blocks = max_blocks_per_seq;
    a.block_size = k->block_size;
    a.chunk = p.chunk;
    a.n_chunks = p.n_chunks;
    a.n_tiles = p.n_tiles;
    const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / sqrt((double)k->head_dim);
    // q'' = scale log2(e) H (s q) / sqrt(128); float16 K scores q itself
    a.qscale = (float)(scale * M_LOG2E / (k_fp16 ? 1.0 : sqrt((double)kD)));
    a.max_page = (int32_t)(std::min(k->n_blocks, v->n_blocks) - 1);
    a.bs_div = make_fastdiv((uint32_t)a.block_size);
    a.chunk_div = make_fastdiv((uint32_t)a.chunk);
    a.units_div = make_fastdiv((uint32_t)(n_seqs * k->n_kv_heads));
    a.kv_div = make_fastdiv((uint32_t)a.n_kv);
    a.grp_div = make_fastdiv((uint32_t)a.group);
    a.qh_div = make_fastdiv((uint32_t)a.n_q_heads);
    a.qt_div = make_fastdiv((uint32_t)a.n_qtok);
    a.tau = sparse_v_tau;
    a.k_bits = k->bits;
    a.v_bits = v->bits;
    a.nb = nb;
    a.nb_log2 = nb == 4 ? 2 : nb == 2 ? 1 : 0;
    a.n_out = v->n_outliers;
    a.v_out_idx = v->outlier_channels;
    a.v_outliers = v->outliers;
    a.acc_w = acc_w;
    a.mfma = mfma ? 1 : 0;
    a.v_rows_read = (sparse && opts) ? reinterpret_cast<unsigned long long *>(opts->v_rows_read) : nullptr;
    a.contig = (k->block_size % kSlice == 0 && is_aligned(k->norms, 16) && is_aligned(v->norms, 16)) ? 1 : 0;
    for (int i = 0; i < TQ_MAX_LEVELS; ++i) {
        a.kc[i] = !k_fp16 && i < k->cb.n_levels ? k->cb.centroids[i] : 0.f;
        a.vc[i] = i < v->cb.n_levels ? v->cb.centroids[i] : 0.f;
    }
    if (app) {
        a.append = 1;
        a.k_new = static_cast<const uint16_t *>(app->k_new);
        a.v_new = static_cast<const uint16_t *>(app->v_new);
        a.new_stride = app->stride;
        a.k_codes_w = k->codes;
        a.v_codes_w = v->codes;
        a.k_norms_w = k->norms;
        a.v_norms_w = v->norms;
        for (int i = 0; i < TQ_MAX_LEVELS - 1; ++i) {
            a.kbnd[i] = i + 1 < k->cb.n_levels ? k->cb.boundaries[i] : INFINITY;
            a.vbnd[i] = i + 1 < v->cb.n_levels ? v->cb.boundaries[i] : INFINITY;
        }
    }
    PairTables pt;
    memset(&pt, 0, sizeof(pt));
    if (!k_fp16)
        for (int e = 0; e < (1 << (2 * k->bits)); ++e)
            pt.k[e] = half2_bits(a.kc[e & ((1 << k->bits) - 1)], a.kc[e >> k->bits]);
    for (int e = 0; e < (1 << (2 * v->bits)); ++e)
        pt.v[e] = half2_bits(a.vc[e & ((1 << v->bits) - 1)], a.vc[e >> v->bits]);
    hipEvent_t ev0 = events ? static_cast<hipEvent_t>(events[0]) : nullptr;
    hipEvent_t ev1 = events ? static_cast<hipEvent_t>(events[1]) : nullptr;
    if (launch_decode(a, pt, static_cast<hipStream_t>(stream), ev0, ev1) != hipSuccess) return TQ_ERR_HIP;
    return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_decode_attention_ex(const tq_cache *k, const tq_cache *v, const void *q, int32_t n_seqs,
                                 int32_t n_qtok, int32_t n_q_heads, const int32_t *seq_lens,
                                 const int32_t *block_table, int32_t max_blocks_per_seq, float softmax_scale,
                                 float sparse_v_tau, float *out, void *workspace, size_t *workspace_bytes,
                                 void *stream, const tq_decode_options *opts, void *const *events) {
    return decode_impl(k, v, q, n_seqs, n_qtok, n_q_heads, seq_lens, block_table, max_blocks_per_seq,
                       softmax_scale, sparse_v_tau, out, workspace, workspace_bytes, stream, opts, events, nullptr);
}

tq_status tq_append_decode_attention(const tq_cache *k, const void *k_new, const tq_cache *v, const void *v_new,
                                     int64_t new_token_stride, const void *q, int32_t n_seqs, int32_t n_qtok,
                                     int32_t n_q_heads, const int32_t *seq_lens, const int32_t *block_table,
                                     int32_t max_blocks_per_seq, float softmax_scale, float sparse_v_tau,
                                     float *out, void *workspace, size_t *workspace_bytes, void *stream,
                                     const tq_decode_options *opts, void *const *events) {
    const AppendIn app{k_new, v_new, new_token_stride};
    return decode_impl(k, v, q, n_seqs, n_qtok, n_q_heads, seq_lens, block_table, max_blocks_per_seq,
                       softmax_scale, sparse_v_tau, out, workspace, workspace_bytes, stream, opts, events, &app);
}

}  // extern "C"
