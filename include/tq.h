/*
 * tq.h - C ABI of libtq: TurboQuant-style KV-cache compression and the decode
 * attention that reads the compressed cache, for AMD MI355X (gfx950).
 *
 * Sources, cited by key (page title, then the section / table used):
 *   [llama-tq]    zingnex thread "llama-tq：让大模型在消费级显卡上跑起10万token长上下文的
 *                 技术突破", section "KV缓存量化的技术困境与TurboQuant的解决方案": K is
 *                 compressed with a randomized Hadamard transform plus a Lloyd-Max
 *                 codebook, and Q.K is computed in the Hadamard domain so K is never
 *                 dequantized during attention; K and V types are chosen separately.
 *   [TQ+ README]  bittide repost of the "TheTom/llama-cpp-turboquant" README
 *                 ("llama.cpp + TurboQuant+"): "量化类型" table and note (Walsh-Hadamard
 *                 rotation then codebook quantization of 128-element blocks; turbo2 /
 *                 turbo3 / turbo4); "压缩策略" (sparse V dequantization below a softmax
 *                 weight threshold); "后端覆盖" table (SET_ROWS quantize-on-append for
 *                 turbo types; VEC flash attention forced for quantized KV on HIP).
 *   [TQ+ article] zingnex thread "TurboQuant+：面向生产环境的LLM KV缓存与权重量化技术",
 *                 "注意力门控稀疏V解压" (skipped V positions are treated as zero).
 *                 The same README's backend table lists flash attention for a 512-element
 *                 head on its Metal row.
 *   [TQ blog]     intelliparadigm TurboQuant article: section 3.2 (H_random = D x H,
 *                 D a random +-1 diagonal; fast Hadamard transform O(d log d)),
 *                 section 3.3 (Lloyd-Max: nearest-centre assignment and mean update,
 *                 separate quantizers for K and V), section 4.1 table (3.25 / 4.25 bits
 *                 per value for turbo3 / turbo4).
 *
 * Format (fixed here where the pages are silent):
 *   - Block = one 128-element K or V head vector x (float16).
 *   - n = ||x||_2 stored as float32; u = x / n (u = 0 for a zero vector).
 *   - y = H (s * u) / sqrt(128): s the +-1 signs of the KV head (signs first,
 *     then the natural-order Sylvester Hadamard matrix H[i][j] = (-1)^popcount(i&j)).
 *   - code_i = number of codebook boundaries strictly below y_i.
 *   - 128 codes packed LSB-first: code i occupies bits [b*i, b*i+b) of the block's
 *     16*b-byte bitstream, stream bit k being bit k%8 of byte k/8.
 *   - Dequantized vector: x_hat = n * s * (H c[code]) / sqrt(128).
 *   - A head of head_dim = 128 nb elements (nb = 1, 2 or 4) is nb such blocks
 *     ([TQ+ README] types note: every format works on 128-element blocks):
 *     elements [128 i, 128 i + 128) form block i, with its own norm and its own
 *     sign words; the cache keeps block i of head j as sub-head nb j + i.
 *   Storage is b + 0.25 bits per value (the [TQ blog] 4.1 figures for b = 3, 4).
 *
 * Conventions for every call:
 *   - Pointers documented "device" are HIP device pointers; "host" are host memory.
 *   - The library allocates no device memory and keeps no global state; every
 *     buffer belongs to the caller.  Calls are asynchronous on `stream` (a
 *     hipStream_t; NULL is the default stream) and may be captured in a HIP graph.
 *   - All arguments are validated on the host before anything is launched; an
 *     invalid call returns an error and launches nothing.  Contents of device
 *     buffers (slots, block ids, lengths) cannot be checked on the host; the
 *     kernels keep every access inside the given buffers whatever they hold
 *     (slots outside the cache are skipped, page ids are clamped to the pool,
 *     lengths to the page table's capacity), but the results for values outside
 *     the documented ranges are unspecified.
 *   - TQ_ERR_HIP is returned when a kernel launch fails; faults inside kernels
 *     surface on the stream, as for any HIP kernel.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
    TQ_OK = 0,
    TQ_ERR_INVALID_ARG = 1,   /* NULL pointer, negative size, inconsistent shape */
    TQ_ERR_UNSUPPORTED = 2,   /* bits not in the supported set, head_dim not 128/256/512, too many rows */
    TQ_ERR_WORKSPACE = 3,     /* workspace smaller than the size this call needs */
    TQ_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} tq_status;

#define TQ_HEAD_DIM 128          /* elements per block; head_dim is 1, 2 or 4 blocks */
#define TQ_MAX_LEVELS 16
#define TQ_BITS_FP16 16   /* a cache side kept in float16: see tq_cache */
#define TQ_MAX_ROWS_PER_KV_HEAD 16   /* (n_q_heads / n_kv_heads) * n_qtok */
#define TQ_MAX_OUTLIERS 16           /* channels per head a side may keep in float16 */

/* Scalar codebook of one cache side ([TQ blog] 3.3).  Centroids are the Lloyd-Max
 * quantizer of N(0, sigma^2) rounded to float16-exact values; boundaries are the
 * exact midpoints of neighbouring centroids. */
typedef struct tq_codebook {
    int32_t bits;                          /* 1..4 (caches use 2..4) */
    int32_t n_levels;                      /* 1 << bits */
    float   centroids[TQ_MAX_LEVELS];      /* ascending, antisymmetric; unused tail is 0 */
    float   boundaries[TQ_MAX_LEVELS - 1]; /* boundaries[j] = (c[j] + c[j+1]) / 2 */
    float   sigma;                         /* the sigma the codebook was built for */
    double  mse;                           /* expected squared error for N(0, sigma^2) */
} tq_codebook;

/* One side (K or V) of a paged compressed cache.  A contiguous cache is the case
 * of an identity page table.  Descriptor lives in host memory; the arrays it
 * points to are device memory owned by the caller. */
typedef struct tq_cache {
    int32_t  bits;          /* 2, 3 or 4; must equal cb.bits.  Or TQ_BITS_FP16: the side
                               keeps its rows as float16 (the "f16 K, turbo V" start of
                               the [TQ+ README] usage steps; [TQ+ article] deployment
                               advice): codes holds [n_blocks][n_kv_heads][head_dim/128]
                               [block_size][128] float16 (256 bytes a row, 16*bits as for
                               the others), and
                               norms, signs and cb are not used (norms and signs may be
                               NULL).  Only a K side may be float16 in tq_decode_attention,
                               which then scores q . k directly (no rotation of q). */
    int32_t  n_kv_heads;    /* >= 1 */
    int32_t  head_dim;      /* 128, 256 or 512 (nb = head_dim / 128 blocks per head) */
    int32_t  block_size;    /* tokens per page, >= 1 */
    int64_t  n_blocks;      /* pages in the pool, >= 1 */
    uint8_t *codes;         /* device uint8 [n_blocks][n_kv_heads][nb][block_size][16*bits] */
    float   *norms;         /* device float [n_blocks][n_kv_heads][nb][block_size] */
    const uint32_t *signs;  /* device uint32 [n_kv_heads][nb][4]; bit i of word w of block k
                               set means element 128*k+32*w+i is multiplied by -1 before H */
    tq_codebook cb;         /* by value */
    /* Kept channels ([llama-tq]: the V family with outlier-channel separation, its
     * high-quality tier): 0, or 1..TQ_MAX_OUTLIERS channels of every head stored
     * exactly as float16 for each token.  The vector with those channels set to
     * zero is what the norm, rotation and codes above describe; the dequantized
     * vector carries the stored values at those channels.  Only a compressed side
     * (bits 2..4) with head_dim 128; in tq_decode_attention only the V side.
     * Zero n_outliers: the two pointers are not used (may be NULL). */
    int32_t  n_outliers;
    const uint8_t *outlier_channels;   /* device uint8 [n_kv_heads][16], 16-byte aligned: the
                                          first n_outliers bytes of each row are the head's
                                          channels, distinct and < 128 (see
                                          tq_select_outlier_channels) */
    uint16_t *outliers;     /* device float16 [n_blocks][n_kv_heads][n_outliers][block_size]
                               (slot-major within a page), 8-byte aligned */
} tq_cache;

/* Human-readable name of a status code (static string, never NULL). */
const char *tq_status_string(tq_status status);

/* Lloyd-Max codebook for N(0, sigma^2) ([TQ blog] 3.3: centres and nearest-centre
 * cells refined alternately until they stop moving; here with the Gaussian density
 * in place of data points, which is the law of a rotated coordinate of a random
 * unit 128-vector for sigma = 1/sqrt(128)).  Host only; deterministic.
 *   bits  : 1..4            sigma : > 0 (caches use 1/sqrt(128))
 *   out   : host, filled on success.
 * Errors: TQ_ERR_INVALID_ARG (out NULL, sigma <= 0 or not finite),
 *         TQ_ERR_UNSUPPORTED (bits outside 1..4). */
tq_status tq_build_codebook(int32_t bits, double sigma, tq_codebook *out);

/* Data-fitted Lloyd-Max codebook for one cache side ([TQ blog] 3.3, the steps as
 * the article lists them: assign every sample to its nearest centre, move every
 * centre to the mean of its samples, repeat until the assignment stops changing,
 * with K and V fitted separately; [TQ blog] 5.3 advises a warm-up on typical
 * inputs so the quantizer adapts to the task's data).  The samples
 * are the 128 rotated coordinates y = H (s o x / |x|) / sqrt(128) of each of
 * n_vectors float16 vectors (host memory, [n_vectors][128]; vector i belongs to
 * head i % n_heads, so a token-major [n_tokens][n_heads][128] array works as
 * is, with that head's signs signs[head][4], host memory, bit i of word w
 * meaning element 32*w+i is negated; for heads of nb blocks, pass the blocks as
 * vectors [n_tokens][n_heads * nb][128] with the sign words [n_heads * nb][4]).  Zero and non-finite vectors are skipped.
 * It starts from tq_build_codebook(bits, 1/sqrt(128)) and runs at most max_iter
 * rounds.  The stored codebook follows the same format: float16-exact centroids
 * (ascending; not forced antisymmetric), exact midpoints as boundaries,
 * sigma = 1/sqrt(128), and mse = the mean squared error over the samples.
 * Host only; deterministic; allocates host memory for the samples only.
 * A cache built with it is quantized and decoded by the same kernels; its
 * boundaries must be at least 0.01 apart (tq_quantize_kv returns
 * TQ_ERR_UNSUPPORTED otherwise).
 * Errors: TQ_ERR_INVALID_ARG (NULL pointer, n_vectors, n_heads or max_iter < 1,
 *         no nonzero finite vector), TQ_ERR_UNSUPPORTED (bits outside 1..4). */
tq_status tq_fit_codebook(int32_t bits, const uint16_t *vectors, int64_t n_vectors, int32_t n_heads,
                          const uint32_t *signs, int32_t max_iter, tq_codebook *out);

/* Kept channels of each head from warm-up data (the [TQ blog] 5.3 advice to adapt
 * to the task's data): for every head, the k channels with the largest mean
 * square over its vectors, ties to the lower channel, in ascending order.
 *   vectors  : host float16 [n_vectors][128]; vector i belongs to head i % n_heads
 *              (a token-major [n_tokens][n_heads][128] array works as is); vectors
 *              with a non-finite element are skipped.
 *   k        : 1..TQ_MAX_OUTLIERS.
 *   channels : host uint8 [n_heads][16], filled: k channels, then zeros (the
 *              layout of tq_cache.outlier_channels, to be copied to the device).
 * Host only; deterministic; allocates host memory for the sums only.
 * Errors: TQ_ERR_INVALID_ARG (NULL pointer, n_vectors or n_heads < 1, k outside
 *         1..TQ_MAX_OUTLIERS). */
tq_status tq_select_outlier_channels(const uint16_t *vectors, int64_t n_vectors, int32_t n_heads, int32_t k,
                                     uint8_t *channels);

/* Quantize-on-append ([TQ+ README] backend table, SET_ROWS for turbo types):
 * compress n_tokens new K and V rows and write them into their cache slots.
 *   k, v            : host descriptors; either may be NULL to skip that side.
 *   k_src, v_src    : device float16 [n_tokens][n_kv_heads][head_dim] of the side's cache
 *                     (both sides given share n_kv_heads and head_dim); heads of one
 *                     token are contiguous, tokens are src_token_stride elements
 *                     apart (>= n_kv_heads * head_dim).
 *   slot_mapping    : device int64 [n_tokens]; slot = block * block_size + offset,
 *                     0 <= slot < n_blocks * block_size of the side; a slot outside that
 *                     range (a negative one marks padding) skips the token on that side.
 *   n_tokens        : >= 0 (0 is a no-op).
 * For each (token, head): norm -> cache.norms, 16*bits code bytes -> cache.codes,
 * and (n_outliers > 0) the kept channels' values -> cache.outliers.
 * Errors: TQ_ERR_INVALID_ARG (missing pointers for a side that is given, bad
 *         stride or sizes, codebook inconsistent with bits), TQ_ERR_UNSUPPORTED
 *         (bits not 2..4 or 16, head_dim not 128/256/512), TQ_ERR_HIP. */
tq_status tq_quantize_kv(const tq_cache *k, const void *k_src,
                         const tq_cache *v, const void *v_src,
                         int64_t src_token_stride, int32_t n_tokens,
                         const int64_t *slot_mapping, void *stream);

/* Decode attention over the compressed cache ([llama-tq] Hadamard-domain Q.K;
 * [TQ+ README] VEC flash attention for quantized KV and sparse V dequantization;
 * [TQ+ article] skipped V treated as zero).
 *   k, v               : host descriptors of the two sides (same n_kv_heads, head_dim
 *                        and block_size; bits may differ).
 *   q                  : device float16 [n_seqs][n_qtok][n_q_heads][head_dim].
 *   n_seqs >= 0, n_qtok >= 1, n_q_heads a multiple of n_kv_heads with
 *   (n_q_heads / n_kv_heads) * n_qtok <= TQ_MAX_ROWS_PER_KV_HEAD.
 *   seq_lens           : device int32 [n_seqs], 0 <= len <= max_blocks_per_seq*block_size;
 *                        each length includes the n_qtok new tokens.
 *   block_table        : device int32 [n_seqs][max_blocks_per_seq]; entry p is the
 *                        physical page holding positions [p*block_size, (p+1)*block_size).
 *   softmax_scale      : > 0, or 0 for 1/sqrt(head_dim).
 *   sparse_v_tau       : >= 0.  With p the final normalised softmax weight, position t
 *                        contributes p_t * v_hat_t iff p_t >= tau (no renormalisation);
 *                        0 is dense attention.
 *   out                : device float32 [n_seqs][n_qtok][n_q_heads][head_dim].
 *   workspace          : device scratch of *workspace_bytes bytes, 256-byte aligned;
 *                        NULL queries the size: the required size is written to
 *                        *workspace_bytes and nothing is launched.  Its contents
 *                        need no initialisation (every call writes what it reads:
 *                        the per-chunk partials and, for a large call, the work
 *                        list and item counters of the persistent pass); calls that
 *                        share one workspace must be ordered on the stream.
 * Query token j of a sequence of length len attends to positions t <= len - n_qtok + j;
 * query head h reads KV head h / (n_q_heads / n_kv_heads).  A row that sees no
 * position outputs zeros.
 * The pass runs on the matrix cores with the library's choice of tokens per pass
 * block (tq_decode_attention_ex selects otherwise).  A float16 K side, heads of
 * more than one block and a V side with kept channels are supported by the
 * matrix-core pass (a K side with kept channels: TQ_ERR_UNSUPPORTED).
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
tq_status tq_decode_attention(const tq_cache *k, const tq_cache *v, const void *q,
                              int32_t n_seqs, int32_t n_qtok, int32_t n_q_heads,
                              const int32_t *seq_lens, const int32_t *block_table,
                              int32_t max_blocks_per_seq, float softmax_scale,
                              float sparse_v_tau, float *out, void *workspace,
                              size_t *workspace_bytes, void *stream);

/* Options of one decode call (tq_decode_attention_ex, tq_append_decode_attention).
 * A NULL options pointer, or a zeroed struct, is the default: what
 * tq_decode_attention does.  The kernel and the chunk change the workspace size,
 * so a workspace query must pass the same options as the call it sizes. */
typedef enum tq_decode_kernel {
    TQ_DECODE_KERNEL_DEFAULT = 0,   /* the matrix-core pass */
    TQ_DECODE_KERNEL_MFMA = 1,      /* the matrix-core pass (fp16 MFMA, fp32-level operands) */
    TQ_DECODE_KERNEL_VALU = 2       /* the vector-ALU pass: 128-wide heads, compressed K, V
                                       without kept channels, no fused append
                                       (TQ_ERR_UNSUPPORTED otherwise) */
} tq_decode_kernel;

typedef struct tq_decode_options {
    int32_t  kernel;          /* a tq_decode_kernel value */
    int32_t  chunk;           /* tokens per pass block: 0 = the library's choice, else a multiple
                                 of 256 (matrix-core pass) or 512 (vector-ALU pass), at most
                                 1 << 20 (TQ_ERR_INVALID_ARG otherwise) */
    uint64_t *v_rows_read;    /* NULL, or a device counter: with sparse_v_tau > 0 the gated pass
                                 adds the number of V code rows the sparse rule needs: one per
                                 token and 128-element block of a KV head whose weight some
                                 query row keeps (the pass may read more: with 128-wide heads
                                 it reads the whole 64-token slice of a kept token).  The
                                 caller zeroes it.  Not touched when tau = 0. */
} tq_decode_options;

/* tq_decode_attention with options, and with start / stop events on the dominant
 * kernel: when `events` is not NULL, events[0] and events[1] (hipEvent_t handles
 * created by the caller) mark the start and the end of the execution of the main
 * pass kernel (the one that streams every K code: the dense pass, or the scoring
 * pass when sparse_v_tau > 0), as hipExtLaunchKernelGGL records them.
 *   opts   : host, may be NULL (defaults).
 *   events : host array of two hipEvent_t, may be NULL.
 * Errors: as tq_decode_attention; TQ_ERR_INVALID_ARG for a bad chunk or kernel. */
tq_status tq_decode_attention_ex(const tq_cache *k, const tq_cache *v, const void *q,
                                 int32_t n_seqs, int32_t n_qtok, int32_t n_q_heads,
                                 const int32_t *seq_lens, const int32_t *block_table,
                                 int32_t max_blocks_per_seq, float softmax_scale,
                                 float sparse_v_tau, float *out, void *workspace,
                                 size_t *workspace_bytes, void *stream,
                                 const tq_decode_options *opts, void *const *events);

/* Quantize-on-append and decode attention in one call: the same result as
 * tq_quantize_kv(k, k_new, v, v_new, new_token_stride, n_seqs * n_qtok, slots)
 * followed by tq_decode_attention(k, v, q, ...), where new token j of sequence b
 * (row b * n_qtok + j of k_new / v_new, device float16 [n_seqs * n_qtok][n_kv_heads]
 * [128], tokens new_token_stride elements apart, >= n_kv_heads * 128, a multiple
 * of 8) goes to position seq_lens[b] - n_qtok + j of sequence b, i.e. to the slot
 * that block_table gives that position (positions below 0 are skipped) - the
 * [TQ+ README] backend table's quantize on append, fused into the pass kernel.
 * The pass block whose chunk holds a new position quantizes it, stores its codes
 * and norm, and uses them for this attention from its own copy; the new tokens'
 * slots must not be read by other sequences of the call.  Supported: the
 * matrix-core pass, head_dim 128, K with 2..4 bits, V without kept channels
 * (TQ_ERR_UNSUPPORTED otherwise: use the two calls).  Codes of elements within
 * rounding of a decision boundary may differ from tq_quantize_kv's (both count
 * the boundaries below the rotated value, in float32 with different roundings).
 * opts, events: as in tq_decode_attention_ex (either may be NULL; the kernel must
 * be the matrix-core pass).  Workspace: as tq_decode_attention (query with
 * workspace NULL and the same options).
 * Errors: as tq_decode_attention; TQ_ERR_INVALID_ARG for NULL or misaligned new
 *         rows or a bad stride. */
tq_status tq_append_decode_attention(const tq_cache *k, const void *k_new, const tq_cache *v, const void *v_new,
                                     int64_t new_token_stride, const void *q, int32_t n_seqs, int32_t n_qtok,
                                     int32_t n_q_heads, const int32_t *seq_lens, const int32_t *block_table,
                                     int32_t max_blocks_per_seq, float softmax_scale, float sparse_v_tau,
                                     float *out, void *workspace, size_t *workspace_bytes, void *stream,
                                     const tq_decode_options *opts, void *const *events);

/* Decode attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * result of tq_decode_attention with the same arguments and no workspace argument.
 * The chunk partials go to a fixed device array inside the library of
 * TQ_NOALLOC_SCRATCH_BYTES (32 MiB), one copy per GPU, held until the process
 * ends; its address on the current device is looked up on the first call on that
 * device.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * routine).  Every call on a GPU shares that GPU's array: calls that overlap on
 * one GPU (on different streams, or from several threads) race; calls ordered on
 * one stream do not.  Nothing in the array needs to start at zero (each call
 * writes every partial it reads).
 * Errors: as tq_decode_attention; TQ_ERR_WORKSPACE (nothing launched) when the
 *         call would need more than TQ_NOALLOC_SCRATCH_BYTES of partials (the size
 *         a tq_decode_attention workspace query returns); TQ_ERR_HIP when the
 *         array's address cannot be found. */
#define TQ_NOALLOC_SCRATCH_BYTES (32u << 20)
tq_status tq_decode_attention_noalloc(const tq_cache *k, const tq_cache *v, const void *q,
                                      int32_t n_seqs, int32_t n_qtok, int32_t n_q_heads,
                                      const int32_t *seq_lens, const int32_t *block_table,
                                      int32_t max_blocks_per_seq, float softmax_scale,
                                      float sparse_v_tau, float *out, void *stream);

/* A plain streaming read of n_bytes (a multiple of 16) at src (device, 16-byte
 * aligned): 16-byte nontemporal loads, grid-stride, the words xor-folded; *sink
 * (device uint32) is written only if the fold equals a fixed value, which keeps
 * the loads alive.  Not part of the method: it measures the practical HBM read
 * ceiling that the decode and quantize kernels are compared with.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_HIP. */
tq_status tq_stream_read(const void *src, size_t n_bytes, uint32_t *sink, void *stream);

/* Dequantize cache rows: dst[t][h][:] = x_hat of slot slots[t], head h
 * ([llama-tq]: K needs no dequantization inside attention; this is the explicit
 * inverse for everything else).
 *   c           : host descriptor.
 *   slots       : device int64 [n_tokens]; a slot outside [0, n_blocks*block_size)
 *                 yields a row of zeros.
 *   dst         : device [n_tokens][n_kv_heads][head_dim], float16 if dst_is_fp16 else float32.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP. */
tq_status tq_dequantize(const tq_cache *c, const int64_t *slots, int32_t n_tokens,
                        void *dst, int32_t dst_is_fp16, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
