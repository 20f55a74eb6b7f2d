"""Seeded synthetic inputs for the compressed-KV hot path.

This module holds only input generation: shapes, value distributions, random
sign words, sequence lengths and page tables.  It contains none of the
method's arithmetic (no rotation, codebook, encoding or attention), and it is
the only module that both the HIP path's tests/benchmark and the CPU oracle
consume.

Every tensor is drawn from its own stream of ``numpy.random.SeedSequence(seed)``
(spawned children, identified by a fixed key), generated in float64 and cast to
float16 on the host, so the GPU and the oracle see identical float16 inputs.

Workloads (the shapes the pages' deployments use; there is no dataset or
model here, so these synthetic tensors stand in for real K/V activations):

  tiny      1 layer, 1 KV head, 1024 tokens, K/V ~ N(0,1) with 4 outlier
            channels x20; K 4-bit, V 3-bit; one query ~ N(0,1); block 256.
  llama8b   Llama-3-8B-shaped decode: 32 q / 8 KV heads, 32768 tokens, batch 1;
            K channel scales lognormal(0,1) per (head, channel), V ~ N(0,1);
            K 4-bit, V 3-bit; block 256, identity page table.
  prefill   32 layers x 8192 tokens x 8 KV heads, K/V ~ Laplace(0,1) with 1% of
            entries x30; K 3-bit, V 2-bit; identity slots.
  longctx   batch 4 x 131072 tokens, 40 q / 4 KV heads; K/V ~ N(0,1) except 64
            planted keys per (sequence, KV head) near an anchor a ~ N(0, I); each
            query head is a + N(0, 0.1^2) (a peaked softmax); K 3-bit, V 2-bit,
            sparse-V threshold 1e-4.
  ragged    64 sequences, lengths uniform in [4096, 65536], 32 q / 8 KV heads,
            4 query tokens per sequence (speculative verify); K 4-bit, V 4-bit;
            256-token pages in a seeded random physical order, table padded -1.
  llama8b_d256, llama8b_d512
            the llama8b decode with heads of 256 / 512 elements (two / four
            128-element blocks, each with its own sign words).
  llama8b_vout
            the llama8b decode whose V has 4 outlier channels x20 (the same 4
            in every head), for a V side that keeps 8 channels in float16.
"""

from __future__ import annotations

from dataclasses import dataclass
from functools import cached_property

import numpy as np

HEAD_DIM = 128

# fixed spawn keys so that adding a stream never shifts another one
_KEY_SIGNS_K, _KEY_SIGNS_V, _KEY_LENS, _KEY_PERM, _KEY_Q, _KEY_KV, _KEY_SCALES, _KEY_OUTL = range(8)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


def random_sign_words(rng: np.random.Generator, n_heads: int) -> np.ndarray:
    """uint32 [n_heads, 4]: 128 independent fair coin flips per head (bit set = -1)."""
    return rng.integers(0, 2**32, size=(n_heads, 4), dtype=np.uint64).astype(np.uint32)


@dataclass
class DecodeWorkload:
    name: str
    n_seqs: int
    n_qtok: int
    n_q_heads: int
    n_kv_heads: int
    k_bits: int
    v_bits: int
    tau: float
    block_size: int
    seq_lens: np.ndarray        # int32 [n_seqs], includes the n_qtok new tokens
    block_table: np.ndarray     # int32 [n_seqs, max_blocks], -1 padded
    n_blocks: int
    kind: str                   # value recipe: tiny | llama8b | normal | longctx
    seed: int = 0
    head_dim: int = HEAD_DIM    # a multiple of 128: head_dim / 128 blocks per head
    v_planted: int = 0          # V channels scaled x20 in every head (at most 4)
    v_kept: int = 0             # channels per head the V side keeps in float16 (0: none)

    @property
    def blocks_per_head(self) -> int:
        return self.head_dim // HEAD_DIM

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @cached_property
    def signs_k(self) -> np.ndarray:
        """uint32 [n_kv_heads * blocks_per_head, 4]: the words of block i of head j in row nb j + i."""
        return random_sign_words(_rng(self.seed, _KEY_SIGNS_K), self.n_kv_heads * self.blocks_per_head)

    @cached_property
    def signs_v(self) -> np.ndarray:
        return random_sign_words(_rng(self.seed, _KEY_SIGNS_V), self.n_kv_heads * self.blocks_per_head)

    @cached_property
    def _k_channel_scales(self) -> np.ndarray:
        # llama8b: sigma_c ~ lognormal(0, 1) per (KV head, channel), fixed across tokens
        return _rng(self.seed, _KEY_SCALES).lognormal(0.0, 1.0, size=(self.n_kv_heads, self.head_dim))

    @cached_property
    def _outlier_channels(self):
        r = _rng(self.seed, _KEY_OUTL)
        return (r.choice(self.head_dim, size=4, replace=False), r.choice(self.head_dim, size=4, replace=False))

    def _anchor_plan(self, seq: int):
        """longctx: per KV head an anchor, 64 planted positions and their noise."""
        r = _rng(self.seed, _KEY_KV, seq, 1)
        length = int(self.seq_lens[seq])
        anchors = r.standard_normal((self.n_kv_heads, self.head_dim))
        pos = np.stack([r.choice(length, size=64, replace=False) for _ in range(self.n_kv_heads)])
        return anchors, pos, r

    def kv_source(self, seq: int):
        """float16 K and V of one sequence: [seq_len, n_kv_heads, head_dim] each."""
        length = int(self.seq_lens[seq])
        r = _rng(self.seed, _KEY_KV, seq, 0)
        shape = (length, self.n_kv_heads, self.head_dim)
        k = r.standard_normal(shape)
        v = r.standard_normal(shape)
        if self.kind == "tiny":
            ko, vo = self._outlier_channels
            k[:, :, ko] *= 20.0
            v[:, :, vo] *= 20.0
        elif self.kind == "llama8b":
            k *= self._k_channel_scales[None, :, :]
        elif self.kind == "longctx":
            anchors, pos, ra = self._anchor_plan(seq)
            for h in range(self.n_kv_heads):
                k[pos[h], h, :] = anchors[h] + 0.1 * ra.standard_normal((64, self.head_dim))
        if self.v_planted:
            v[:, :, self._outlier_channels[1][: self.v_planted]] *= 20.0
        return k.astype(np.float16), v.astype(np.float16)

    def warmup_v(self, n_tokens: int = 1024) -> np.ndarray:
        """float16 V of the first n_tokens positions of sequence 0 (warm-up data)."""
        return self.kv_source(0)[1][:n_tokens]

    def queries(self) -> np.ndarray:
        """float16 [n_seqs, n_qtok, n_q_heads, head_dim]."""
        r = _rng(self.seed, _KEY_Q)
        q = r.standard_normal((self.n_seqs, self.n_qtok, self.n_q_heads, self.head_dim))
        if self.kind == "longctx":
            for b in range(self.n_seqs):
                anchors, _, _ = self._anchor_plan(b)
                for h in range(self.n_q_heads):
                    q[b, :, h, :] = anchors[h // self.group] + 0.1 * q[b, :, h, :]
        return q.astype(np.float16)

    def slots(self, seq: int) -> np.ndarray:
        """int64 physical slot of each logical position of sequence seq."""
        length = int(self.seq_lens[seq])
        t = np.arange(length, dtype=np.int64)
        return self.block_table[seq].astype(np.int64)[t // self.block_size] * self.block_size + t % self.block_size

    @property
    def total_tokens(self) -> int:
        return int(np.sum(self.seq_lens))


def _identity_table(n_seqs: int, length: int, block_size: int):
    nb = -(-length // block_size)
    table = np.arange(n_seqs * nb, dtype=np.int32).reshape(n_seqs, nb)
    return table, n_seqs * nb


def tiny(seed: int = 0) -> DecodeWorkload:
    table, nb = _identity_table(1, 1024, 256)
    return DecodeWorkload("tiny", 1, 1, 1, 1, 4, 3, 0.0, 256,
                          np.array([1024], np.int32), table, nb, "tiny", seed)


def llama8b(seed: int = 0, context: int = 32768) -> DecodeWorkload:
    table, nb = _identity_table(1, context, 256)
    return DecodeWorkload("llama8b", 1, 1, 32, 8, 4, 3, 0.0, 256,
                          np.array([context], np.int32), table, nb, "llama8b", seed)


def llama8b_k16(seed: int = 0, context: int = 32768) -> DecodeWorkload:
    """The Llama-3-8B-shaped decode with K kept in float16 and V at 3 bits."""
    table, nb = _identity_table(1, context, 256)
    return DecodeWorkload("llama8b_k16", 1, 1, 32, 8, 16, 3, 0.0, 256,
                          np.array([context], np.int32), table, nb, "llama8b", seed)


def llama8b_wide(head_dim: int, seed: int = 0, context: int = 32768) -> DecodeWorkload:
    """The Llama-3-8B-shaped decode (heads, context, value recipe, K 4-bit / V 3-bit)
    with heads of head_dim = 256 or 512 elements."""
    table, nb = _identity_table(1, context, 256)
    return DecodeWorkload(f"llama8b_d{head_dim}", 1, 1, 32, 8, 4, 3, 0.0, 256,
                          np.array([context], np.int32), table, nb, "llama8b", seed, head_dim)


def llama8b_vout(seed: int = 0, context: int = 32768) -> DecodeWorkload:
    """The Llama-3-8B-shaped decode (K4 / V3) with 4 planted V outlier channels x20
    and a V side keeping 8 channels per head in float16."""
    table, nb = _identity_table(1, context, 256)
    return DecodeWorkload("llama8b_vout", 1, 1, 32, 8, 4, 3, 0.0, 256,
                          np.array([context], np.int32), table, nb, "llama8b", seed, v_planted=4, v_kept=8)


def longctx(seed: int = 0, context: int = 131072, batch: int = 4) -> DecodeWorkload:
    table, nb = _identity_table(batch, context, 256)
    return DecodeWorkload("longctx", batch, 1, 40, 4, 3, 2, 1e-4, 256,
                          np.full(batch, context, np.int32), table, nb, "longctx", seed)


def ragged(seed: int = 0, n_seqs: int = 64, lo: int = 4096, hi: int = 65536) -> DecodeWorkload:
    bs = 256
    lens = _rng(seed, _KEY_LENS).integers(lo, hi + 1, size=n_seqs).astype(np.int32)
    max_blocks = -(-hi // bs)
    need = -(-lens.astype(np.int64) // bs)
    n_blocks = int(np.sum(need))
    perm = _rng(seed, _KEY_PERM).permutation(n_blocks).astype(np.int32)
    table = np.full((n_seqs, max_blocks), -1, np.int32)
    at = 0
    for b in range(n_seqs):
        table[b, : need[b]] = perm[at: at + need[b]]
        at += need[b]
    return DecodeWorkload("ragged", n_seqs, 4, 32, 8, 4, 4, 0.0, bs, lens, table, n_blocks, "normal", seed)


@dataclass
class PrefillWorkload:
    """32 layers x 8192 tokens x 8 KV heads of Laplace(0,1) K and V, 1% x30."""
    n_layers: int = 32
    n_tokens: int = 8192
    n_kv_heads: int = 8
    k_bits: int = 3
    v_bits: int = 2
    block_size: int = 256
    seed: int = 0

    def signs(self, layer: int):
        return (random_sign_words(_rng(self.seed, _KEY_SIGNS_K, layer), self.n_kv_heads),
                random_sign_words(_rng(self.seed, _KEY_SIGNS_V, layer), self.n_kv_heads))

    def kv_source(self, layer: int, n_tokens: int | None = None):
        n = self.n_tokens if n_tokens is None else n_tokens
        r = _rng(self.seed, _KEY_KV, layer)
        out = []
        for _ in range(2):
            x = r.laplace(0.0, 1.0, size=(n, self.n_kv_heads, HEAD_DIM))
            x *= np.where(r.random(x.shape) < 0.01, 30.0, 1.0)
            out.append(x.astype(np.float16))
        return out[0], out[1]

    @property
    def n_blocks(self) -> int:
        return -(-self.n_tokens // self.block_size)


def prefill(seed: int = 0) -> PrefillWorkload:
    return PrefillWorkload(seed=seed)


def small_decode(seed: int, n_seqs: int, lens, n_qtok: int, n_q_heads: int, n_kv_heads: int,
                 k_bits: int, v_bits: int, tau: float = 0.0, block_size: int = 256,
                 shuffle_pages: bool = True, head_dim: int = HEAD_DIM, v_planted: int = 0,
                 v_kept: int = 0) -> DecodeWorkload:
    """A small ragged, paged workload with N(0,1) K/V/q for parity tests."""
    lens = np.asarray(lens, np.int32)
    max_blocks = max(1, int(-(-int(np.max(lens)) // block_size))) if n_seqs else 1
    need = -(-lens.astype(np.int64) // block_size)
    n_blocks = max(1, int(np.sum(need)))
    perm = (_rng(seed, _KEY_PERM).permutation(n_blocks) if shuffle_pages
            else np.arange(n_blocks)).astype(np.int32)
    table = np.full((max(n_seqs, 1), max_blocks), -1, np.int32)[:n_seqs]
    at = 0
    for b in range(n_seqs):
        table[b, : need[b]] = perm[at: at + need[b]]
        at += need[b]
    return DecodeWorkload("small", n_seqs, n_qtok, n_q_heads, n_kv_heads, k_bits, v_bits, tau,
                          block_size, lens, table, n_blocks, "normal", seed, head_dim, v_planted, v_kept)
