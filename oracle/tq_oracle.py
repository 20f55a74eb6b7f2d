"""Plain, slow, float64 CPU oracle of the compressed-KV hot path.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): nothing in the product
may import this module, and the product path never falls back to it.

Every step is written as its plain definition in float64 numpy: the Hadamard
matrix is built entry by entry and applied as an explicit matrix product (no
fast transform), encoding counts boundaries, softmax is exp/sum, and so on.  A
library primitive (a matrix product, ``scipy.special.ndtr``) may serve as one
step; there is no blocking, fusion or reordering beyond the definitions.

Sources, cited below by key (page title, then the section / table used):

  [llama-tq]     zingnex thread "llama-tq：让大模型在消费级显卡上跑起10万token长上下文
                 的技术突破", section "KV缓存量化的技术困境与TurboQuant的解决方案"
                 (randomized Hadamard + Lloyd-Max codebook for K; Q.K computed in
                 the Hadamard domain without dequantizing K).
  [TQ+ README]   bittide repost of the "TheTom/llama-cpp-turboquant" README
                 ("llama.cpp + TurboQuant+"): the "量化类型" (quantization types)
                 table and the note under it (Walsh-Hadamard rotation, then
                 codebook quantization on 128-element blocks; turbo2/3/4); the
                 "压缩策略" list (sparse V dequantization gated by the softmax
                 weight); the "后端覆盖" (backend) table (SET_ROWS quantize on
                 append, VEC flash attention for quantized KV).
  [TQ+ article]  zingnex thread "TurboQuant+：面向生产环境的LLM KV缓存与权重量化技术",
                 sections "Walsh-Hadamard变换" and "注意力门控稀疏V解压" (skipped
                 V positions are treated as zero).
  [TQ blog]      intelliparadigm TurboQuant article (weixin_29053577/2214691):
                 section 3.2 (H_random = D x H with D a random +-1 diagonal; fast
                 Hadamard transform in O(d log d)), section 3.3 (Lloyd-Max: assign
                 each point to the nearest centre, recompute centres as means,
                 repeat; separate quantizers for K and V), section 4.1 table
                 (bits per value 3.25 / 4.25 for turbo3 / turbo4).

Readings taken where the pages are silent:

  R1  Hadamard order and scale: Sylvester matrix in natural order,
      H[i, j] = (-1)^popcount(i & j), scaled by 1/sqrt(d) so the rotation is
      orthonormal.
  R2  "H_random = D x H" is read with row vectors, so the signs are applied
      first and the Hadamard second: y = H (s * u) / sqrt(d).
  R3  Per-block scale: the L2 norm of the 128-vector, stored as float32; the
      unit vector is what gets rotated and quantized (32 bits of overhead per
      128 values, i.e. b + 0.25 bits per value, which is what the [TQ blog]
      section 4.1 table prints for turbo3 and turbo4).  A zero vector has norm
      0 and rotated coordinates 0.
  R4  Codebook: the Lloyd-Max quantizer of N(0, sigma^2), sigma = 1/sqrt(128)
      (the coordinate law of a rotated random unit vector), computed in float64
      from a uniform start until it stops moving, made exactly antisymmetric,
      then each centroid rounded to the nearest float16 value.  Decision
      boundaries are the exact midpoints of neighbouring stored centroids
      (exactly representable in float32).
  R4a Data-fitted codebook (the [TQ blog] 3.3 steps on data, with the 5.3
      warm-up advice): the samples are the rotated coordinates of the given
      nonzero vectors; the centres start at the stored Gaussian codebook of R4
      and stop when no sample changes cell; not made antisymmetric; stored like
      R4 (float16 centres, exact midpoints).
  R5  Encoding: code = number of boundaries strictly below y, comparing the
      float64 y with the stored boundaries; a tie goes to the lower code.
  R6  Packing: LSB-first bitstream per 128-block; code i occupies stream bits
      [b*i, b*i + b); stream bit k is bit (k mod 8) of byte k // 8; 16*b bytes.
  R7  Attention: scores scale * q . k_hat with scale 1/sqrt(head_dim) unless given;
      GQA maps query head h to KV head h // (H_q / H_kv); with n_qtok query
      tokens per sequence, query token j sees positions t <= len - n_qtok + j.
  R8  Sparse V: with p the exact, final, normalised softmax weight, position t
      contributes p_t * v_hat_t iff p_t >= tau; skipped positions count as zero
      and the kept weights are not renormalised.  tau = 0 is dense attention.
  R11 A side kept in float16 (the [TQ+ README] usage steps start from f16 K
      with turbo V; the [TQ+ article] deployment advice starts from a light
      asymmetric setting): the row is stored as its 128 float16 values and read
      back exactly; attention scores it as scale * q . k with no rotation.
  R12 Heads wider than one block (the [TQ+ README] types note puts every turbo
      format on 128-element blocks; its Metal row has flash attention for a
      512-wide head): a head of head_dim = 128 * nb elements is nb consecutive
      blocks, elements [128 i, 128 i + 128) forming block i, each quantized on
      its own as in R1-R6 with its own norm and its own sign vector.  The cache
      keeps block i of head j as sub-head nb * j + i; the dequantized head is the
      concatenation of its blocks, and attention is R7 over the whole head.
  R13 V outlier channels (the V family "v3" of [llama-tq], named there only as
      V quantization with outlier-channel separation, its high-quality tier; the
      fourth page's compression principle keeps rare high-magnitude values at 8
      or 16 bits): per KV head a fixed set of k <= 16 channels is kept exactly
      as float16 for every token; the vector with those channels set to zero is
      quantized as R1-R6 (its norm and rotation see zeros there); the
      dequantized vector is the TurboQuant reconstruction with the kept values
      written over those channels.  The channels come from warm-up data (the
      [TQ blog] 5.3 advice): the k with the largest mean square over the head's
      vectors, ties to the lower index, listed in ascending order.
  R14 Non-finite input (the pages say nothing of it): a vector with an inf or
      NaN element has no direction to quantize.  It is stored like the zero
      vector of R3 (every rotated coordinate 0, so every code is that of y = 0,
      2^(b-1) - 1 under R5), with its norm as computed: inf, or NaN when an
      element is NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
from scipy.special import ndtr

D = 128  # elements per block ([TQ+ README] note under the quantization types table)

__all__ = [
    "D", "hadamard_matrix", "sign_vector", "rotate", "unrotate",
    "gaussian_lloyd_max", "lloyd_max_from_samples", "Codebook", "build_codebook", "fit_codebook",
    "codebook_mse", "encode", "near_boundary_mask", "quantize_vectors",
    "pack_codes", "unpack_codes", "dequantize_vectors", "OracleCache",
    "new_cache", "cache_write", "cache_read", "slots_for_sequence", "FP16", "select_outlier_channels",
    "MAX_OUTLIERS",
    "decode_attention_rows", "decode_attention", "bits_per_value",
]


# ---------------------------------------------------------------------------
# Rotation  ([TQ blog] section 3.2; [TQ+ article] "Walsh-Hadamard变换"; R1, R2)
# ---------------------------------------------------------------------------

def hadamard_matrix(d: int = D) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix, natural order (reading R1).

    H[i, j] = (-1)^popcount(i AND j), written entry by entry.
    """
    h = np.empty((d, d), dtype=np.float64)
    for i in range(d):
        for j in range(d):
            h[i, j] = -1.0 if bin(i & j).count("1") % 2 else 1.0
    return h


_H = hadamard_matrix(D)


def sign_vector(sign_words) -> np.ndarray:
    """+-1 diagonal of D from four uint32 words: bit i of word w is element 32w+i; set means -1."""
    w = np.asarray(sign_words, dtype=np.uint32).reshape(4)
    s = np.empty(D, dtype=np.float64)
    for e in range(D):
        s[e] = -1.0 if (int(w[e // 32]) >> (e % 32)) & 1 else 1.0
    return s


def rotate(u: np.ndarray, s: np.ndarray) -> np.ndarray:
    """y = H (s * u) / sqrt(d) for every row of u ([TQ blog] 3.2 read as R2)."""
    u = np.asarray(u, dtype=np.float64)
    return ((u * s) @ _H.T) / math.sqrt(D)


def unrotate(y: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Inverse of rotate: u = s * (H^T y) / sqrt(d)  (the rotation is orthonormal)."""
    y = np.asarray(y, dtype=np.float64)
    return s * (y @ _H) / math.sqrt(D)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook  ([TQ blog] section 3.3; [llama-tq]; R4)
# ---------------------------------------------------------------------------

def _phi(z: np.ndarray) -> np.ndarray:
    out = np.zeros_like(z)
    fin = np.isfinite(z)
    out[fin] = np.exp(-0.5 * z[fin] ** 2) / math.sqrt(2.0 * math.pi)
    return out


def gaussian_lloyd_max(n_levels: int, sigma: float, max_iter: int = 20000,
                       tol: float = 1e-14) -> np.ndarray:
    """Lloyd-Max centroids of N(0, sigma^2), float64, ascending (reading R4).

    The two Lloyd steps of [TQ blog] 3.3 with the data replaced by the density:
      (a) each boundary is the midpoint of its two neighbouring centres
          (nearest-centre assignment);
      (b) each centre is the mean of the density over its cell, which for a
          Gaussian is sigma * (phi(lo) - phi(hi)) / (Phi(hi) - Phi(lo)) on the
          standardised cell [lo, hi].
    Start uniform on [-2 sigma, 2 sigma]; stop when no centre moves by more
    than tol * sigma.  Antisymmetry is imposed after every step.
    """
    if n_levels == 1:
        return np.zeros(1)
    c = np.linspace(-2.0, 2.0, n_levels)  # standardised units
    for _ in range(max_iter):
        b = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-np.inf], b))
        hi = np.concatenate((b, [np.inf]))
        mass = ndtr(hi) - ndtr(lo)
        c_new = (_phi(lo) - _phi(hi)) / mass
        c_new = 0.5 * (c_new - c_new[::-1])
        moved = np.max(np.abs(c_new - c))
        c = c_new
        if moved < tol:
            break
    return c * sigma


def lloyd_max_from_samples(x: np.ndarray, n_levels: int, max_iter: int = 500,
                           init: np.ndarray | None = None) -> np.ndarray:
    """Data-driven Lloyd-Max exactly as [TQ blog] 3.3 lists it.

    Initialise centres, assign each sample to its nearest centre, recompute each
    centre as the mean of its samples, repeat until the assignment is stable.
    """
    x = np.sort(np.asarray(x, dtype=np.float64).ravel())
    if init is None:
        qs = (np.arange(n_levels) + 0.5) / n_levels
        c = np.quantile(x, qs)
    else:
        c = np.asarray(init, dtype=np.float64).copy()
    prev = None
    for _ in range(max_iter):
        assign = np.argmin(np.abs(x[:, None] - c[None, :]), axis=1)
        if prev is not None and np.array_equal(assign, prev):
            break
        prev = assign
        for j in range(n_levels):
            sel = x[assign == j]
            if sel.size:
                c[j] = sel.mean()
    return c


@dataclass
class Codebook:
    bits: int
    centroids: np.ndarray      # float64 holding float16-exact values, ascending
    boundaries: np.ndarray     # float64 holding the exact midpoints (float32-exact)
    mse: float                 # expected squared error for N(0, sigma^2)
    sigma: float
    centroids_f64: np.ndarray = field(repr=False, default=None)  # before float16 rounding

    @property
    def n_levels(self) -> int:
        return 1 << self.bits


def codebook_mse(centroids: np.ndarray, boundaries: np.ndarray, sigma: float) -> float:
    """E[(X - Q(X))^2] for X ~ N(0, sigma^2), integrated cell by cell in closed form.

    On a standardised cell [a, b] with centre c (standardised):
      int (x - c)^2 phi = (1 + c^2)(Phi(b) - Phi(a)) + (a - 2c) phi(a) - (b - 2c) phi(b)
    (with x phi(x) -> 0 at the infinite ends).
    """
    c = np.asarray(centroids, dtype=np.float64) / sigma
    bd = np.asarray(boundaries, dtype=np.float64) / sigma
    lo = np.concatenate(([-np.inf], bd))
    hi = np.concatenate((bd, [np.inf]))
    mass = ndtr(hi) - ndtr(lo)
    a_phi = np.where(np.isfinite(lo), np.nan_to_num(lo, neginf=0.0) * _phi(lo), 0.0)
    b_phi = np.where(np.isfinite(hi), np.nan_to_num(hi, posinf=0.0) * _phi(hi), 0.0)
    per_cell = (1.0 + c * c) * mass + (a_phi - 2.0 * c * _phi(lo)) - (b_phi - 2.0 * c * _phi(hi))
    return float(np.sum(per_cell) * sigma * sigma)


def build_codebook(bits: int, sigma: float = 1.0 / math.sqrt(D)) -> Codebook:
    """Stored codebook of the format (reading R4): float16-exact centres, exact midpoints."""
    if bits not in (1, 2, 3, 4):
        raise ValueError("bits must be 1..4")
    c64 = gaussian_lloyd_max(1 << bits, sigma)
    c16 = c64.astype(np.float16).astype(np.float64)
    # keep exact antisymmetry after rounding (float16 rounding is symmetric, this is a guard)
    c16 = 0.5 * (c16 - c16[::-1])
    b = 0.5 * (c16[:-1] + c16[1:])
    return Codebook(bits=bits, centroids=c16, boundaries=b,
                    mse=codebook_mse(c16, b, sigma), sigma=sigma, centroids_f64=c64)


def fit_codebook(bits: int, vectors: np.ndarray, sign_words, max_iter: int = 200):
    """Data-fitted stored codebook of one side ([TQ blog] 3.3 steps; 5.3 warm-up; R4a).

    Samples: for every nonzero, finite vector x (float16 values, rows of
    [..., n_heads, 128]; the head is the last-but-one index), the 128 rotated
    coordinates y = H (s_head * x / ||x||) / sqrt(128).  Centres start at the
    stored Gaussian codebook of build_codebook(bits) and follow
    lloyd_max_from_samples (nearest centre, then means, until the assignment is
    stable).  Stored as build_codebook stores: centres rounded to float16,
    boundaries the exact midpoints; mse is the mean squared error of the samples.

    Returns (Codebook, centres before rounding, samples).
    """
    sw = np.asarray(sign_words, dtype=np.uint32).reshape(-1, 4)
    x = np.asarray(vectors).astype(np.float64).reshape(-1, sw.shape[0], D)
    ys = []
    for h in range(sw.shape[0]):
        xh = x[:, h, :]
        n = np.sqrt(np.sum(xh * xh, axis=-1))
        ok = np.isfinite(xh).all(axis=-1) & (n > 0)
        u = xh[ok] / n[ok, None]
        ys.append(rotate(u, sign_vector(sw[h])).ravel())
    y = np.concatenate(ys)
    if y.size == 0:
        raise ValueError("no nonzero finite vector")
    init = build_codebook(bits).centroids
    c64 = lloyd_max_from_samples(y, 1 << bits, max_iter=max_iter, init=init)
    c16 = c64.astype(np.float16).astype(np.float64)
    b = 0.5 * (c16[:-1] + c16[1:])
    code = encode(y, b)
    mse = float(np.mean((y - c16[code]) ** 2))
    cb = Codebook(bits=bits, centroids=c16, boundaries=b, mse=mse, sigma=1.0 / math.sqrt(D), centroids_f64=c64)
    return cb, c64, y


def bits_per_value(bits: int) -> float:
    """Stored bits per element: b code bits plus one float32 norm per 128 (reading R3)."""
    return bits + 32.0 / D


# ---------------------------------------------------------------------------
# Quantize one 128-vector  (R3, R5; [llama-tq]; [TQ+ README] types note)
# ---------------------------------------------------------------------------

_CHUNK = 1 << 20   # elements per step, only to bound temporary memory


def encode(y: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    """code = #{j : y > boundary_j} (nearest centre with ties to the lower code, R5)."""
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i in range(0, flat.size, _CHUNK):
        out[i:i + _CHUNK] = np.sum(flat[i:i + _CHUNK, None] > boundaries, axis=-1)
    return out.reshape(y.shape)


def near_boundary_mask(y: np.ndarray, boundaries: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Elements whose rotated value lies within eps of some decision boundary."""
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=bool)
    for i in range(0, flat.size, _CHUNK):
        out[i:i + _CHUNK] = np.any(np.abs(flat[i:i + _CHUNK, None] - boundaries) < eps, axis=-1)
    return out.reshape(y.shape)


def quantize_vectors(x: np.ndarray, s: np.ndarray, cb: Codebook):
    """Quantize rows of x (float16 values, any leading shape, last dim 128).

    Returns (norms float32, codes uint8 [..., 128], y float64 [..., 128]).
      n = ||x||_2 (float64, stored rounded to float32)           R3
      u = x / n   (u = 0 when n = 0, or when x has a non-finite   R3, R14
                   element: then n is inf or NaN)
      y = H (s * u) / sqrt(128)                                   R1, R2
      code_i = #{j : y_i > b_j}                                   R5
    """
    x = np.asarray(x).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        n = np.sqrt(np.sum(x * x, axis=-1))
        has_dir = (n > 0) & np.all(np.isfinite(x), axis=-1)
        safe = np.where(has_dir, n, 1.0)
        u = np.where(has_dir[..., None], x / safe[..., None], 0.0)
    y = rotate(u.reshape(-1, D), s).reshape(u.shape)
    codes = encode(y, cb.boundaries)
    return n.astype(np.float32), codes, y


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """LSB-first bitstream of the 128 codes of each block (reading R6)."""
    codes = np.asarray(codes, dtype=np.uint8)
    lead = codes.shape[:-1]
    flat = codes.reshape(-1, D)
    out = np.zeros((flat.shape[0], 16 * bits), dtype=np.uint8)
    for i in range(D):
        for k in range(bits):
            bit = (flat[:, i] >> k) & 1
            pos = bits * i + k
            out[:, pos // 8] |= (bit << (pos % 8)).astype(np.uint8)
    return out.reshape(*lead, 16 * bits)


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    flat = packed.reshape(-1, 16 * bits)
    out = np.zeros((flat.shape[0], D), dtype=np.uint8)
    for i in range(D):
        for k in range(bits):
            pos = bits * i + k
            bit = (flat[:, pos // 8] >> (pos % 8)) & 1
            out[:, i] |= (bit << k).astype(np.uint8)
    return out.reshape(*lead, D)


def dequantize_vectors(norms: np.ndarray, codes: np.ndarray, s: np.ndarray,
                       cb: Codebook) -> np.ndarray:
    """x_hat = n * R^T c[code]  (the decode side of R3/R4; float64)."""
    c = cb.centroids[np.asarray(codes, dtype=np.int64)]
    u_hat = unrotate(c.reshape(-1, D), s).reshape(c.shape)
    return np.asarray(norms, dtype=np.float64)[..., None] * u_hat


# ---------------------------------------------------------------------------
# Paged cache  ([TQ+ README] backend table: SET_ROWS writes quantized rows)
# ---------------------------------------------------------------------------

@dataclass
class OracleCache:
    bits: int
    n_kv_heads: int
    block_size: int
    n_blocks: int
    codes: np.ndarray   # uint8 [n_blocks, n_sub, block_size, 16*bits]
    norms: np.ndarray   # float32 [n_blocks, n_sub, block_size]
    signs: np.ndarray   # uint32 [n_sub, 4]
    cb: Codebook
    head_dim: int = D   # elements per head; n_sub = n_kv_heads * head_dim / 128 sub-heads (R12)
    n_outliers: int = 0                      # R13: channels per sub-head kept in float16
    outlier_channels: np.ndarray = None      # uint8 [n_sub, n_outliers], ascending
    outliers: np.ndarray = None              # float16 [n_blocks, n_sub, n_outliers, block_size]

    @property
    def blocks_per_head(self) -> int:
        return self.head_dim // D

    @property
    def n_sub(self) -> int:
        return self.n_kv_heads * self.blocks_per_head


FP16 = 16  # bits of a side kept in float16 (R11): rows of 128 float16, no norm, no codebook


MAX_OUTLIERS = 16   # R13: at most this many kept channels per head


def new_cache(bits, n_kv_heads, block_size, n_blocks, signs, cb, head_dim: int = D,
              outlier_channels=None) -> OracleCache:
    """A zeroed paged cache side; bits = FP16 keeps float16 rows (256 bytes each).

    head_dim is a multiple of 128 (R12); signs hold one word quadruple per
    sub-head, [n_kv_heads, head_dim / 128, 4] in any shape of that size.
    outlier_channels (R13, a compressed side): [n_sub, k] distinct channel
    indices per sub-head, k <= 16, kept in float16.
    """
    if head_dim % D != 0 or head_dim < D:
        raise ValueError("head_dim must be a positive multiple of 128")
    n_sub = n_kv_heads * (head_dim // D)
    c = OracleCache(bits, n_kv_heads, block_size, n_blocks,
                    np.zeros((n_blocks, n_sub, block_size, 16 * bits), np.uint8),
                    np.zeros((n_blocks, n_sub, block_size), np.float32),
                    np.asarray(signs, np.uint32).reshape(n_sub, 4), cb, head_dim)
    if outlier_channels is not None:
        idx = np.asarray(outlier_channels, np.int64).reshape(n_sub, -1)
        k = idx.shape[1]
        if bits == FP16 or k > MAX_OUTLIERS or np.any(idx < 0) or np.any(idx >= D):
            raise ValueError("outlier channels: a compressed side, at most 16 channels in [0, 128)")
        if any(len(set(row.tolist())) != k for row in idx):
            raise ValueError("outlier channels of a head must be distinct")
        c.n_outliers = k
        c.outlier_channels = np.sort(idx, axis=1).astype(np.uint8)
        c.outliers = np.zeros((n_blocks, n_sub, k, block_size), np.float16)
    return c


def select_outlier_channels(vectors: np.ndarray, k: int) -> np.ndarray:
    """R13: per head, the k channels with the largest mean square over the given
    vectors [..., n_heads, 128] (float16 values; a vector with a non-finite
    element is skipped), ties to the lower index; returns uint8 [n_heads, k],
    each row ascending."""
    x = np.asarray(vectors).astype(np.float64)
    x = x.reshape(-1, x.shape[-2], D)
    out = np.zeros((x.shape[1], k), np.uint8)
    for h in range(x.shape[1]):
        rows = x[:, h, :]
        rows = rows[np.all(np.isfinite(rows), axis=1)]
        ms = np.mean(rows * rows, axis=0) if len(rows) else np.zeros(D)
        order = sorted(range(D), key=lambda c: (-ms[c], c))
        out[h] = np.sort(order[:k])
    return out


def cache_write(cache: OracleCache, src: np.ndarray, slots: np.ndarray):
    """Quantize src [n_tokens, n_kv_heads, head_dim] (float16) into the cache slots.

    slot = block * block_size + offset; a negative slot skips that token.
    Returns (norms, codes, y) of all rows, per sub-head, for the caller's diagnostics.
    """
    src = np.asarray(src)
    slots = np.asarray(slots, dtype=np.int64)
    n_tok = src.shape[0]
    # R12: element 128 i + e of head j is element e of sub-head nb j + i
    src = src.reshape(n_tok, cache.n_kv_heads, cache.blocks_per_head, D).reshape(n_tok, cache.n_sub, D)
    if cache.bits == FP16:   # R11: the row itself, byte for byte
        rows = np.ascontiguousarray(src.astype(np.float16)).view(np.uint8).reshape(n_tok, cache.n_sub, 2 * D)
        for t in range(n_tok):
            if slots[t] >= 0:
                blk, off = divmod(int(slots[t]), cache.block_size)
                cache.codes[blk, :, off, :] = rows[t]
        return None
    norms = np.zeros((n_tok, cache.n_sub), np.float32)
    codes = np.zeros((n_tok, cache.n_sub, D), np.uint8)
    ys = np.zeros((n_tok, cache.n_sub, D), np.float64)
    kept = None
    if cache.n_outliers:   # R13: the kept channels leave the vector before R3-R6
        idx = cache.outlier_channels.astype(np.int64)
        kept = np.stack([src[:, h, idx[h]] for h in range(cache.n_sub)], axis=1).astype(np.float16)
        src = src.copy()
        for h in range(cache.n_sub):
            src[:, h, idx[h]] = 0
    for h in range(cache.n_sub):
        s = sign_vector(cache.signs[h])
        nh, ch, yh = quantize_vectors(src[:, h, :], s, cache.cb)
        norms[:, h], codes[:, h], ys[:, h] = nh, ch, yh
    packed = pack_codes(codes, cache.bits)
    for t in range(n_tok):
        if slots[t] < 0:
            continue
        blk, off = divmod(int(slots[t]), cache.block_size)
        cache.codes[blk, :, off, :] = packed[t]
        cache.norms[blk, :, off] = norms[t]
        if kept is not None:
            cache.outliers[blk, :, :, off] = kept[t]
    return norms, codes, ys


def slots_for_sequence(block_table_row: np.ndarray, block_size: int, n_tokens: int) -> np.ndarray:
    """Physical slot of logical positions 0..n_tokens-1 of one sequence."""
    t = np.arange(n_tokens, dtype=np.int64)
    return np.asarray(block_table_row, np.int64)[t // block_size] * block_size + t % block_size


def _read_sub(cache: OracleCache, blk: np.ndarray, off: np.ndarray, sub: int) -> np.ndarray:
    """Dequantized float64 128-vectors of one sub-head at the given (page, offset)s."""
    if cache.bits == FP16:   # R11
        return np.ascontiguousarray(cache.codes[blk, sub, off, :]).view(np.float16).astype(np.float64)
    packed = cache.codes[blk, sub, off, :]
    norms = cache.norms[blk, sub, off]
    codes = unpack_codes(packed, cache.bits)
    x = dequantize_vectors(norms, codes, sign_vector(cache.signs[sub]), cache.cb)
    if cache.n_outliers:   # R13: the kept values over their channels
        x[:, cache.outlier_channels[sub].astype(np.int64)] = cache.outliers[blk, sub, :, off].astype(np.float64)
    return x


def cache_read(cache: OracleCache, slots: np.ndarray, head: int) -> np.ndarray:
    """Dequantized float64 vectors [len(slots), head_dim] of one KV head: the
    concatenation of its blocks (R12)."""
    slots = np.asarray(slots, dtype=np.int64)
    blk, off = slots // cache.block_size, slots % cache.block_size
    nb = cache.blocks_per_head
    return np.concatenate([_read_sub(cache, blk, off, nb * head + i) for i in range(nb)], axis=1)


# ---------------------------------------------------------------------------
# Decode attention  ([llama-tq]; [TQ+ README] backend table and sparse V;
#                    [TQ+ article] "注意力门控稀疏V解压"; R7, R8)
# ---------------------------------------------------------------------------

def decode_attention_rows(q_rows: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
                          n_visible: np.ndarray, scale: float, tau: float):
    """Attention of several query rows over one KV head's dequantized tokens.

    q_rows [R, d] float64, k_hat / v_hat [T, d] float64, row r sees the first
    n_visible[r] tokens.  Returns (out [R, d], list of weight vectors p_r).
      s_t = scale * q . k_hat_t ;  p = exp(s - max s) / sum exp(s - max s)
      out = sum_{t : p_t >= tau} p_t v_hat_t     (tau = 0: every t)
    Rows that see no token return zeros.
    """
    out = np.zeros((q_rows.shape[0], v_hat.shape[1]), dtype=np.float64)
    ps = []
    for r in range(q_rows.shape[0]):
        n = int(n_visible[r])
        if n <= 0:
            ps.append(np.zeros(0))
            continue
        s = scale * (k_hat[:n] @ q_rows[r])
        e = np.exp(s - np.max(s))
        p = e / np.sum(e)
        keep = p >= tau
        out[r] = (p * keep) @ v_hat[:n]
        ps.append(p)
    return out, ps


def decode_attention(q: np.ndarray, kc: OracleCache, vc: OracleCache, seq_lens,
                     block_table, n_qtok: int, scale: float = 0.0, tau: float = 0.0,
                     seqs=None, kv_heads=None, return_weights: bool = False):
    """Decode attention over the paged caches, float64.

    q [n_seqs, n_qtok, H_q, head_dim] (float16 values); seq_lens include the n_qtok
    new tokens; block_table [n_seqs, max_blocks].  Returns out with the shape of
    q (float64); only the requested sequences / KV heads are filled (others 0).
    """
    q = np.asarray(q).astype(np.float64)
    n_seqs, _, hq, hd = q.shape
    if hd != kc.head_dim or hd != vc.head_dim:
        raise ValueError("q, K and V must share head_dim")
    hkv = kc.n_kv_heads
    g = hq // hkv
    if scale == 0.0:
        scale = 1.0 / math.sqrt(hd)
    out = np.zeros_like(q)
    weights = {}
    seqs = range(n_seqs) if seqs is None else seqs
    kv_heads = range(hkv) if kv_heads is None else kv_heads
    for b in seqs:
        length = int(seq_lens[b])
        if length <= 0:
            continue
        slots = slots_for_sequence(block_table[b], kc.block_size, length)
        for kv in kv_heads:
            k_hat = cache_read(kc, slots, kv)
            v_hat = cache_read(vc, slots, kv)
            for j in range(n_qtok):
                vis = length - n_qtok + j + 1
                heads = range(kv * g, (kv + 1) * g)
                rows = np.stack([q[b, j, h] for h in heads])
                o, ps = decode_attention_rows(rows, k_hat, v_hat,
                                              np.full(len(rows), vis), scale, tau)
                for idx, h in enumerate(heads):
                    out[b, j, h] = o[idx]
                    if return_weights:
                        weights[(b, j, h)] = ps[idx]
    if return_weights:
        return out, weights
    return out
