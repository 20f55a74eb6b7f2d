"""GPU parity: the HIP path (called through the C ABI) against the CPU oracle.

Codes must be bit-exact except elements whose rotated value lies within 1e-6 of
a decision boundary (excluded, counted, printed).  Norms within 1e-6 relative.
Attention rows within 1e-3 relative L2 of the float64 oracle computed on the
same cache contents (the cache given to both sides is written by the oracle).
"""

import math
import sys

import numpy as np
import pytest

import oracle as O
from compressed_kv_attention_tq_amd import tq as T
from compressed_kv_attention_tq_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu



def _t():
    import torch
    return torch


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = _t()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T.load_library()
    yield


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# Decode kernels under test: the matrix-core pass with the default chunking, the
# same with 1024-token chunks (several slices per wave, so the next-slice loads
# run), and the vector-ALU pass.
DECODE_KERNELS = {
    "mfma": T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA),
    "mfma-c1024": T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA, chunk=1024),
    "valu": T.DecodeOptions(kernel=T.DECODE_KERNEL_VALU),
}


@pytest.fixture(params=list(DECODE_KERNELS))
def kernel(request, monkeypatch):
    """Every decode call of the test runs with these options (the binding's default)."""
    monkeypatch.setattr(T, "default_options", DECODE_KERNELS[request.param])
    log(f"[decode kernel {request.param}]")
    return request.param


# Oracle results reused across the kernels of one case (keyed by the workload's
# defining parameters; only the last few are kept).
_ORACLE_MEMO = {}


def _wl_key(wl):
    return (wl.name, wl.kind, wl.seed, wl.n_seqs, tuple(int(x) for x in wl.seq_lens), wl.n_qtok, wl.n_q_heads,
            wl.n_kv_heads, wl.k_bits, wl.v_bits, wl.block_size, wl.n_blocks, wl.head_dim, wl.v_planted, wl.v_kept)


def _memo(key, fn):
    if key not in _ORACLE_MEMO:
        while len(_ORACLE_MEMO) >= 4:
            _ORACLE_MEMO.pop(next(iter(_ORACLE_MEMO)))
        _ORACLE_MEMO[key] = fn()
    return _ORACLE_MEMO[key]


# --------------------------------------------------------------------------- quantize

def quantize_and_compare(x16, signs, bits, block_size=16, slot_perm=None, token_pad=0, ocb=None):
    """GPU-quantize x16 [n_tok, n_kv, 128] into a fresh cache and compare with the oracle
    (codebook ocb, an oracle codebook, by default the Gaussian one)."""
    torch = _t()
    n_tok, n_kv, _ = x16.shape
    n_blocks = max(1, -(-n_tok // block_size)) + 1
    slots = np.arange(n_tok, dtype=np.int64) if slot_perm is None else slot_perm
    g = T.Cache.allocate(bits, n_kv, block_size, n_blocks, signs,
                         cb=None if ocb is None else U.tq_codebook_from(ocb))
    g.codes.fill_(0xAB)
    src = np.zeros((n_tok, n_kv * 128 + token_pad), np.float16)
    src[:, : n_kv * 128] = x16.reshape(n_tok, -1)
    src_t = torch.from_numpy(src).cuda()
    view = src_t[:, : n_kv * 128].view(n_tok, n_kv, 128) if token_pad == 0 else \
        torch.as_strided(src_t, (n_tok, n_kv, 128), (n_kv * 128 + token_pad, 128, 1))
    T.tq_quantize_kv(g, view, None, None, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    # [block][head][offset] -> [slot][head]
    codes = g.codes.cpu().numpy().transpose(0, 2, 1, 3).reshape(-1, n_kv, 16 * bits)
    norms = g.norms.cpu().numpy().transpose(0, 2, 1).reshape(-1, n_kv)
    near = 0
    for h in range(n_kv):
        ok = slots >= 0
        near += U.check_codes(codes[slots[ok], h], norms[slots[ok], h], x16[ok, h], signs[h], bits, cb=ocb)
    untouched = np.setdiff1d(np.arange(codes.shape[0]), slots[slots >= 0])
    assert np.all(codes[untouched] == 0xAB), "a skipped or unused slot was written"
    return near


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n_kv,n_tok", [(1, 1), (3, 7), (8, 300), (5, 33), (4, 13), (2, 77), (8, 6), (16, 21),
                                        (12, 9)])
def test_quantize_random(bits, n_kv, n_tok):
    """n_kv dividing 16 takes the matrix-core transform (tiles of 16 vectors: 52, 154,
    48 and 336 vectors leave partial tiles and waves), the others the vector path."""
    rng = np.random.default_rng(100 * bits + n_tok)
    x = (rng.standard_normal((n_tok, n_kv, 128)) * rng.lognormal(0, 1, (1, n_kv, 128))).astype(np.float16)
    signs = W.random_sign_words(rng, n_kv)
    near = quantize_and_compare(x, signs, bits)
    log(f"quantize bits={bits} n_kv={n_kv} n_tok={n_tok}: near-boundary {near}")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_special_vectors_skips_and_strides(bits):
    rng = np.random.default_rng(5)
    n_tok, n_kv = 40, 2
    x = rng.standard_normal((n_tok, n_kv, 128)).astype(np.float16)
    x[0] = 0                                   # zero vectors
    x[1, 0] = np.float16(65504.0)              # largest float16, all coordinates
    x[2, 1, :] = np.float16(6e-8)              # float16 subnormals
    x[3, 0, :] = 0; x[3, 0, 77] = 3.0          # a single spike
    x[4, 1] = np.where(np.arange(128) % 2, 1.0, -1.0).astype(np.float16)
    signs = W.random_sign_words(rng, n_kv)
    perm = rng.permutation(n_tok + 24)[:n_tok].astype(np.int64)
    perm[[5, 9, 17]] = -1                      # skipped tokens
    near = quantize_and_compare(x, signs, bits, block_size=16, slot_perm=perm, token_pad=72)
    log(f"quantize special bits={bits}: near-boundary {near}")


def test_quantize_tiny_workload():
    wl = W.tiny()
    k, v = wl.kv_source(0)
    nk = quantize_and_compare(k, wl.signs_k, wl.k_bits, block_size=256)
    nv = quantize_and_compare(v, wl.signs_v, wl.v_bits, block_size=256)
    log(f"tiny workload: near-boundary K {nk} / {k.size}, V {nv} / {v.size}")


@pytest.mark.parametrize("layer", [0, 31])
def test_quantize_prefill_layer_full(layer):
    """Full 8192 x 8 heads K (3-bit) and V (2-bit) of one prefill layer, both sides in one call."""
    torch = _t()
    wl = W.prefill()
    sk, sv = wl.signs(layer)
    k, v = wl.kv_source(layer)
    kc = T.Cache.allocate(wl.k_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, sk)
    vc = T.Cache.allocate(wl.v_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, sv)
    slots = torch.arange(wl.n_tokens, dtype=torch.int64, device="cuda")
    T.tq_quantize_kv(kc, torch.from_numpy(k).cuda(), vc, torch.from_numpy(v).cuda(), slots)
    torch.cuda.synchronize()
    near = 0
    for cache, x, sg in ((kc, k, sk), (vc, v, sv)):
        codes = cache.codes.cpu().numpy().transpose(0, 2, 1, 3).reshape(wl.n_tokens, wl.n_kv_heads, -1)
        norms = cache.norms.cpu().numpy().transpose(0, 2, 1).reshape(wl.n_tokens, wl.n_kv_heads)
        for h in range(wl.n_kv_heads):
            near += U.check_codes(codes[:, h], norms[:, h], x[:, h], sg[h], cache.bits)
    log(f"prefill layer {layer}: near-boundary {near} of {2 * k.size}")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_with_fitted_codebook(bits):
    """Codebook fitted (by the oracle) on warm-up tokens of a prefill layer; the GPU
    quantizes the next tokens with it, the oracle with the same stored values."""
    wl = W.prefill()
    sk, _ = wl.signs(3)
    k, _ = wl.kv_source(3)
    ocb, _, _ = O.fit_codebook(bits, k[:256], sk)
    assert not np.array_equal(ocb.centroids, O.build_codebook(bits).centroids)
    near = quantize_and_compare(k[256:768], sk, bits, block_size=64, ocb=ocb)
    log(f"fitted {bits}-bit: near-boundary {near}")


@pytest.mark.parametrize("n_kv,n_tok", [(1, 5), (8, 300), (3, 77)])
def test_float16_side_store_and_read(n_kv, n_tok):
    """A float16 side stores each row's bytes in its slot and reads them back exactly."""
    torch = _t()
    rng = np.random.default_rng(n_kv * 1000 + n_tok)
    x = (rng.standard_normal((n_tok, n_kv, 128)) * 8).astype(np.float16)
    bs = 16
    n_blocks = -(-n_tok // bs) + 2
    slots = rng.permutation(n_blocks * bs)[:n_tok].astype(np.int64)
    slots[1::9] = -1
    g = T.Cache.allocate(T.BITS_FP16, n_kv, bs, n_blocks, np.zeros((n_kv, 4), np.uint32))
    g.codes.fill_(0xAB)
    T.tq_quantize_kv(g, torch.from_numpy(x).cuda(), None, None, torch.from_numpy(slots).cuda())
    rows = g.codes.cpu().numpy().transpose(0, 2, 1, 3).reshape(-1, n_kv, 256)
    ok = slots >= 0
    want = np.ascontiguousarray(x).view(np.uint8).reshape(n_tok, n_kv, 256)
    assert np.array_equal(rows[slots[ok]], want[ok])
    untouched = np.setdiff1d(np.arange(rows.shape[0]), slots[ok])
    assert np.all(rows[untouched] == 0xAB)
    rd = torch.from_numpy(slots[ok]).cuda()
    assert np.array_equal(T.tq_dequantize(g, rd, fp16=True).cpu().numpy(), x[ok])
    assert np.array_equal(T.tq_dequantize(g, rd).cpu().numpy(), x[ok].astype(np.float32))


# --------------------------------------------------------------------------- dequantize

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_non_finite_vectors(bits):
    """R14: vectors with a +inf, -inf or NaN element (and an all-inf one) store the
    zero direction with the norm as computed; finite rows of the same call are
    unaffected; dequantize agrees with the oracle NaN for NaN."""
    torch = _t()
    rng = np.random.default_rng(300 + bits)
    n_tok, n_kv = 24, 2
    x = rng.standard_normal((n_tok, n_kv, 128)).astype(np.float16)
    x[0, 0, 5] = np.inf
    x[3, 1, 127] = -np.inf
    x[7, 0, 0] = np.nan
    x[9, 1, :] = np.inf
    x[12, 0, 64] = np.nan
    x[12, 0, 65] = np.inf
    signs = W.random_sign_words(rng, n_kv)
    g = T.Cache.allocate(bits, n_kv, 16, 2, signs)
    slots = np.arange(n_tok, dtype=np.int64)
    T.tq_quantize_kv(g, torch.from_numpy(x).cuda(), None, None, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    codes = g.codes.cpu().numpy().transpose(0, 2, 1, 3).reshape(-1, n_kv, 16 * bits)[:n_tok]
    norms = g.norms.cpu().numpy().transpose(0, 2, 1).reshape(-1, n_kv)[:n_tok]
    cb = O.build_codebook(bits)
    bad = ~np.all(np.isfinite(x.astype(np.float64)), axis=-1)
    for h in range(n_kv):
        on, oc, oy = O.quantize_vectors(x[:, h], O.sign_vector(signs[h]), cb)
        got = O.unpack_codes(codes[:, h], bits)
        b = bad[:, h]
        assert np.array_equal(got[b], oc[b]) and np.all(oc[b] == (1 << (bits - 1)) - 1)
        np.testing.assert_array_equal(norms[b, h], on[b])          # inf == inf, NaN == NaN
        U.check_codes(codes[~b, h], norms[~b, h], x[~b, h], signs[h], bits)
    # dequantize: the oracle's reconstruction of the same stored rows, NaN for NaN
    out = T.tq_dequantize(g, torch.from_numpy(slots).cuda()).cpu().numpy()
    oc_cache = O.new_cache(bits, n_kv, 16, 2, signs, cb)
    O.cache_write(oc_cache, x, slots)
    for h in range(n_kv):
        want = O.cache_read(oc_cache, slots, h)
        b = bad[:, h]
        np.testing.assert_array_equal(np.isnan(out[b, h]), np.isnan(want[b]))
        fin = ~np.isnan(want[b])
        np.testing.assert_array_equal(out[b, h][fin], want[b][fin])   # the +-inf entries
    log(f"quantize non-finite bits={bits}: {int(bad.sum())} rows stored as the zero direction")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequantize_matches_oracle(bits):
    torch = _t()
    wl = W.small_decode(seed=bits, n_seqs=2, lens=[300, 77], n_qtok=1, n_q_heads=3, n_kv_heads=3,
                        k_bits=bits, v_bits=bits, block_size=64)
    oc = U.oracle_cache(wl, 0)
    g = U.gpu_cache_from(oc)
    slots = np.concatenate([wl.slots(0), wl.slots(1)])
    out32 = T.tq_dequantize(g, torch.from_numpy(slots).cuda()).cpu().numpy()
    out16 = T.tq_dequantize(g, torch.from_numpy(slots).cuda(), fp16=True).cpu().numpy()
    for h in range(3):
        want = O.cache_read(oc, slots, h)
        assert np.max(U.row_rel_err(out32[:, h], want)) < 1e-5
        np.testing.assert_allclose(out16[:, h].astype(np.float64), want, rtol=2e-3, atol=1e-4)


# --------------------------------------------------------------------------- decode

def oracle_caches(wl):
    return _memo(("caches",) + _wl_key(wl), lambda: (U.oracle_cache(wl, 0), U.oracle_cache(wl, 1)))


def decode_and_compare(wl, seqs=None, kv_heads=None, tau=None, scale=0.0, gpu_caches=None, q=None,
                       oracle_key=None):
    """Decode on the GPU with oracle-written caches; compare rows of the given seqs."""
    torch = _t()
    tau = wl.tau if tau is None else tau
    if gpu_caches is None:
        ok, ov = oracle_caches(wl)
        gk, gv = U.gpu_cache_from(ok), U.gpu_cache_from(ov)
    else:
        ok, ov, gk, gv = gpu_caches
    q = wl.queries() if q is None else q
    out = T.tq_decode_attention(gk, gv, torch.from_numpy(q).cuda(),
                                torch.from_numpy(wl.seq_lens).cuda(),
                                torch.from_numpy(wl.block_table).cuda(), scale, tau).cpu().numpy()
    key = ("decode",) + _wl_key(wl) + (tau, scale, None if seqs is None else tuple(seqs),
                                       None if kv_heads is None else tuple(kv_heads), oracle_key)
    want, weights = _memo(key, lambda: O.decode_attention(q, ok, ov, wl.seq_lens, wl.block_table, wl.n_qtok,
                                                          scale, tau, seqs=seqs, kv_heads=kv_heads,
                                                          return_weights=True))
    seqs = list(range(wl.n_seqs) if seqs is None else seqs)
    kv_heads = list(range(wl.n_kv_heads) if kv_heads is None else kv_heads)
    heads = [h for kv in kv_heads for h in range(kv * wl.group, (kv + 1) * wl.group)]
    # slack for gate decisions within rounding of tau (|p / tau - 1| < 1e-4): the
    # contribution p v_hat of each such position, per row and per element
    row_slack = np.zeros((len(seqs), wl.n_qtok, len(heads)))
    elem_slack = np.zeros((len(seqs), wl.n_qtok, len(heads), wl.head_dim))
    ambiguous = 0
    if tau > 0:
        for bi, b in enumerate(seqs):
            for j in range(wl.n_qtok):
                for hi, h in enumerate(heads):
                    p = weights.get((b, j, h))
                    if p is None:
                        continue
                    amb = np.abs(p / tau - 1.0) < 1e-4
                    if amb.any():
                        ambiguous += int(amb.sum())
                        slots = O.slots_for_sequence(wl.block_table[b], wl.block_size, len(p))
                        vh = O.cache_read(ov, slots[amb], h // wl.group)
                        row_slack[bi, j, hi] = float(np.sum(p[amb] * np.linalg.norm(vh, axis=1)))
                        elem_slack[bi, j, hi] = np.sum(p[amb][:, None] * np.abs(vh), axis=0)
    got = out[np.ix_(seqs, range(wl.n_qtok), heads)]
    ref = want[np.ix_(seqs, range(wl.n_qtok), heads)]
    worst, worst_e = U.assert_attention_close(got, ref, (row_slack, elem_slack), what=f"decode {wl.name}")
    log(f"decode {wl.name}: worst row rel err {worst:.2e}, worst element error / bound {worst_e:.2e}, "
        f"ambiguous gate decisions {ambiguous}")
    return out, want


def _gate_slack(wl, ov, weights, tau):
    """Per-row and per-element slack for gate decisions within rounding of tau, over
    every row of the workload (zeros when tau = 0)."""
    rs = np.zeros((wl.n_seqs, wl.n_qtok, wl.n_q_heads))
    es = np.zeros((wl.n_seqs, wl.n_qtok, wl.n_q_heads, wl.head_dim))
    if tau <= 0:
        return rs, es
    for (b, j, h), p in weights.items():
        amb = np.abs(p / tau - 1.0) < 1e-4
        if amb.any():
            slots = O.slots_for_sequence(wl.block_table[b], wl.block_size, len(p))
            vh = O.cache_read(ov, slots[amb], h // wl.group)
            rs[b, j, h] = float(np.sum(p[amb] * np.linalg.norm(vh, axis=1)))
            es[b, j, h] = np.sum(p[amb][:, None] * np.abs(vh), axis=0)
    return rs, es


def test_decode_tiny_workload(kernel):
    decode_and_compare(W.tiny())


@pytest.mark.parametrize("case", [
    # n_seqs, lens, n_qtok, n_q_heads, n_kv, kb, vb, block_size
    (1, [1], 1, 1, 1, 4, 3, 256),
    (3, [1000, 1, 257], 1, 8, 2, 4, 3, 256),
    (2, [700, 1300], 1, 6, 3, 3, 2, 64),
    (2, [255, 513], 2, 8, 4, 2, 4, 100),
    (3, [40, 3, 2], 4, 4, 1, 4, 4, 16),
    (2, [900, 600], 1, 20, 2, 3, 3, 128),
    (2, [1500, 77], 4, 32, 8, 4, 4, 256),
    (2, [333, 1024], 3, 4, 1, 2, 2, 32),
    (1, [4097], 1, 16, 16, 4, 2, 256),
], ids=lambda c: f"s{c[0]}-q{c[2]}-h{c[3]}/{c[4]}-b{c[5]}{c[6]}-bs{c[7]}")
def test_decode_small_cases(case, kernel):
    n_seqs, lens, n_qtok, hq, hkv, kb, vb, bs = case
    wl = W.small_decode(seed=sum(lens), n_seqs=n_seqs, lens=lens, n_qtok=n_qtok, n_q_heads=hq,
                        n_kv_heads=hkv, k_bits=kb, v_bits=vb, block_size=bs)
    decode_and_compare(wl)


def test_decode_rows_with_no_visible_token_are_zero(kernel):
    wl = W.small_decode(seed=3, n_seqs=2, lens=[2, 0], n_qtok=4, n_q_heads=2, n_kv_heads=1, k_bits=4,
                        v_bits=3, block_size=16)
    out, want = decode_and_compare(wl)
    assert np.all(out[0, :2] == 0) and np.all(out[1] == 0)


def test_decode_with_fitted_codebooks(kernel):
    """K and V codebooks fitted (oracle) on the first 512 positions of sequence 0."""
    wl = W.small_decode(seed=31, n_seqs=2, lens=[1800, 640], n_qtok=2, n_q_heads=8, n_kv_heads=2, k_bits=4,
                        v_bits=3, block_size=256)
    k0, v0 = wl.kv_source(0)

    def build():
        ckb, _, _ = O.fit_codebook(wl.k_bits, k0[:512], wl.signs_k)
        cvb, _, _ = O.fit_codebook(wl.v_bits, v0[:512], wl.signs_v)
        return U.oracle_cache(wl, 0, cb=ckb), U.oracle_cache(wl, 1, cb=cvb)

    ok, ov = _memo(("fitted",) + _wl_key(wl), build)
    decode_and_compare(wl, gpu_caches=(ok, ov, U.gpu_cache_from(ok), U.gpu_cache_from(ov)), oracle_key="fitted")


def _skip_valu_for_fp16_k(kernel):
    if kernel == "valu":
        pytest.skip("float16 K runs on the matrix-core pass only (the vector-ALU pass rejects it)")


@pytest.mark.parametrize("case", [
    # (n_seqs, lens, n_qtok, n_q_heads, n_kv_heads, v_bits, block_size)
    (1, [700], 1, 4, 1, 3, 256),
    (2, [1000, 33], 1, 32, 8, 2, 256),
    (2, [300, 129], 4, 16, 4, 4, 64),
    (3, [77, 5, 260], 2, 8, 1, 3, 16),
])
def test_decode_float16_k(case, kernel):
    """K kept in float16, V compressed ([TQ+ README] f16 K with turbo V)."""
    _skip_valu_for_fp16_k(kernel)
    n_seqs, lens, n_qtok, hq, hkv, vb, bs = case
    wl = W.small_decode(seed=sum(lens) + vb, n_seqs=n_seqs, lens=lens, n_qtok=n_qtok, n_q_heads=hq,
                        n_kv_heads=hkv, k_bits=T.BITS_FP16, v_bits=vb, block_size=bs)
    decode_and_compare(wl)


@pytest.mark.parametrize("tau", [1e-4, 3e-2, 1.5])
def test_decode_float16_k_sparse(tau, kernel):
    _skip_valu_for_fp16_k(kernel)
    wl = W.small_decode(seed=41, n_seqs=2, lens=[2500, 700], n_qtok=2, n_q_heads=8, n_kv_heads=2,
                        k_bits=T.BITS_FP16, v_bits=2, tau=tau, block_size=256)
    out, _ = decode_and_compare(wl)
    if tau > 1:
        assert np.all(out == 0)


def test_decode_float16_k_llama8b_full(kernel):
    """The Llama-3-8B-shaped decode (32768 tokens, 32 / 8 heads) with float16 K and 3-bit V."""
    _skip_valu_for_fp16_k(kernel)
    decode_and_compare(W.llama8b_k16())


def test_decode_custom_scale(kernel):
    wl = W.small_decode(seed=8, n_seqs=1, lens=[800], n_qtok=1, n_q_heads=4, n_kv_heads=2, k_bits=4,
                        v_bits=4, block_size=256)
    decode_and_compare(wl, scale=0.3)


@pytest.mark.parametrize("tau", [1e-4, 1e-3, 3e-2, 0.5, 1.5])
def test_decode_sparse_small(tau, kernel):
    wl = W.small_decode(seed=11, n_seqs=2, lens=[3000, 900], n_qtok=2, n_q_heads=8, n_kv_heads=2, k_bits=3,
                        v_bits=2, tau=tau, block_size=256)
    out, _ = decode_and_compare(wl)
    if tau > 1:
        assert np.all(out == 0)


@pytest.mark.parametrize("tau", [0.0, 1e-3])
def test_decode_many_chunks(tau, monkeypatch):
    """More chunks per row than the merge takes in one round of loads (a 40000-token
    sequence in 256-token chunks: 157 of them), next to a 700-token sequence (3): the
    merge's first round is loaded before the lengths are read, clamped to the chunks
    the workspace holds, and drops the chunks past each sequence's own."""
    monkeypatch.setattr(T, "default_options", T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA, chunk=256))
    wl = W.small_decode(seed=23, n_seqs=2, lens=[40000, 700], n_qtok=1, n_q_heads=4, n_kv_heads=1, k_bits=4,
                        v_bits=3, tau=tau, block_size=256)
    decode_and_compare(wl)


@pytest.mark.parametrize("tau", [0.0, 1e-3])
@pytest.mark.parametrize("case", [(2048, 1, 4, 2, 128), (1280, 4, 32, 8, 128), (1024, 1, 8, 1, 256)],
                         ids=["8slots-rows2", "5slots-rows16", "4slots-d256"])
def test_decode_merge_few_slots(tau, case, monkeypatch):
    """The merge for at most 8 chunk slots (8 outputs per block, every slot of a
    column in one round): lengths ending in every chunk of a 256-token-chunk table,
    on chunk edges and one token past them, an empty sequence, 2 and 16 rows per KV
    head, and two 128-element blocks per head; the output count is not a multiple of
    8 for the first case (9 sequences x 4 heads)."""
    cap, n_qtok, hq, n_kv, d = case
    monkeypatch.setattr(T, "default_options", T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA, chunk=256))
    lens = [0, 1, 256, 257, 700, cap // 2 + 3, cap - 256, cap - 1, cap]
    wl = W.small_decode(seed=31 + cap + d, n_seqs=len(lens), lens=lens, n_qtok=n_qtok, n_q_heads=hq,
                        n_kv_heads=n_kv, k_bits=4, v_bits=3, tau=tau, block_size=256,
                        head_dim=d)
    decode_and_compare(wl)


def _persistent_workload(seed, tau, n_qtok, n_q_heads, block_size):
    """48 ragged sequences (empty, single-token, chunk-edge and ~3000-token ones), 8 KV
    heads: in 256-token chunks that is 48 x 8 x 12 = 4608 (chunk, unit) items, more
    than any GPU holds blocks at once, so the matrix-core passes run persistent and
    take their items from the work list; about half the items are empty."""
    rng = np.random.default_rng(seed)
    lens = [0, 1, 255, 256, 257, 512, 3072, 3000] + [int(x) for x in rng.integers(0, 3073, 40)]
    return W.small_decode(seed=seed, n_seqs=len(lens), lens=lens, n_qtok=n_qtok, n_q_heads=n_q_heads,
                          n_kv_heads=8, k_bits=4, v_bits=3, tau=tau, block_size=block_size)


@pytest.mark.parametrize("tau", [0.0, 1e-3])
@pytest.mark.parametrize("shape", [(1, 32, 256), (4, 32, 64), (2, 64, 100)],
                         ids=["q1-rows4-bs256", "q4-rows16-bs64", "q2-rows16-bs100"])
def test_decode_persistent_work_list(tau, shape, monkeypatch):
    n_qtok, hq, bs = shape
    monkeypatch.setattr(T, "default_options", T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA, chunk=256))
    wl = _persistent_workload(400 + n_qtok + bs, tau, n_qtok, hq, bs)
    decode_and_compare(wl)


def _paired_workload(seed, tau, n_qtok):
    """64 sequences of a 262144-token page table (2 KV heads): at the library's chunk
    choice that is 2048 (chunk, unit) items of 16384 tokens, so the chunk is halved
    and the work list pairs chunks (items of 16384 tokens, then the odd last 8192-token
    chunks).  Most sequences are short; three are long enough for pairs (one with an
    odd chunk count, one ending on a chunk edge)."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, 1200, 61)] + [40000, 24576, 17000]
    wl = W.small_decode(seed=seed, n_seqs=len(lens), lens=lens, n_qtok=n_qtok, n_q_heads=8, n_kv_heads=2,
                        k_bits=4, v_bits=3, tau=tau, block_size=256)
    table = np.full((wl.n_seqs, 1024), -1, np.int32)
    table[:, : wl.block_table.shape[1]] = wl.block_table
    wl.block_table = table
    return wl


@pytest.mark.parametrize("tau", [0.0, 1e-3])
@pytest.mark.parametrize("n_qtok", [1, 4])
def test_decode_persistent_paired_items(tau, n_qtok, monkeypatch):
    monkeypatch.setattr(T, "default_options", T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA))
    decode_and_compare(_paired_workload(500 + n_qtok, tau, n_qtok))


@pytest.mark.parametrize("tau", [0.0, 1e-3])
def test_append_decode_persistent_work_list(tau, monkeypatch):
    monkeypatch.setattr(T, "default_options", T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA, chunk=256))
    wl = _persistent_workload(411, tau, 2, 32, 256)
    append_and_compare(wl)


@pytest.mark.parametrize("variant", ["large-q", "small-q"])
def test_decode_extreme_magnitudes(variant, kernel):
    """Queries scaled far from unit size (K norms scaled back for large ones, so the
    scores keep their spread) and V norms spread over eight decades."""
    wl = W.small_decode(seed=17, n_seqs=2, lens=[1200, 333], n_qtok=2, n_q_heads=8, n_kv_heads=2, k_bits=4,
                        v_bits=3, block_size=64)
    qs = 300.0 if variant == "large-q" else 1e-3

    def build():
        ok, ov = U.oracle_cache(wl, 0), U.oracle_cache(wl, 1)
        f = np.random.default_rng(99).choice([3e4, 1.0, 1e-3], size=ov.norms.shape, p=[0.05, 0.5, 0.45])
        ov.norms = (ov.norms * f).astype(np.float32)
        if variant == "large-q":
            ok.norms = (ok.norms / qs).astype(np.float32)
        return ok, ov

    ok, ov = _memo(("extreme", variant) + _wl_key(wl), build)
    q = (wl.queries().astype(np.float64) * qs).astype(np.float16)
    decode_and_compare(wl, gpu_caches=(ok, ov, U.gpu_cache_from(ok), U.gpu_cache_from(ov)), q=q,
                       oracle_key=variant)


def test_decode_sparse_peaked_small(kernel):
    wl = W.longctx(context=8192, batch=2)
    decode_and_compare(wl)


def test_decode_llama8b_full(kernel):
    """Llama-3-8B-shaped decode (32 q / 8 KV heads, 32K context, K4/V3), every row."""
    decode_and_compare(W.llama8b())


def _mixed_caches(wl, sampled):
    """Device caches whose sampled sequences hold oracle-written pages and whose
    other sequences hold GPU-quantized N(0,1) data (torch RNG); only sampled rows
    are compared, and they depend only on their own pages."""
    torch = _t()
    gk = T.Cache.allocate(wl.k_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, wl.signs_k)
    gv = T.Cache.allocate(wl.v_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, wl.signs_v)
    gen = torch.Generator(device="cuda").manual_seed(1234)
    for b in range(wl.n_seqs):
        if b in sampled:
            continue
        n = int(wl.seq_lens[b])
        kx = torch.randn((n, wl.n_kv_heads, 128), generator=gen, device="cuda").half()
        vx = torch.randn((n, wl.n_kv_heads, 128), generator=gen, device="cuda").half()
        T.tq_quantize_kv(gk, kx, gv, vx, torch.from_numpy(wl.slots(b)).cuda())
    ok, ov = _memo(("mixed", tuple(sampled)) + _wl_key(wl),
                   lambda: (U.oracle_cache(wl, 0, seqs=sampled), U.oracle_cache(wl, 1, seqs=sampled)))
    blocks = np.concatenate([wl.block_table[b][: -(-int(wl.seq_lens[b]) // wl.block_size)] for b in sampled])
    U.upload_blocks(ok, gk, blocks)
    U.upload_blocks(ov, gv, blocks)
    torch.cuda.synchronize()
    return ok, ov, gk, gv


def test_decode_longctx_sampled(kernel):
    """4 x 128K sparse decode (40 q / 4 KV heads, K3/V2, tau 1e-4): sequence 0 checked, all heads."""
    wl = W.longctx()
    caches = _mixed_caches(wl, [0])
    decode_and_compare(wl, seqs=[0], gpu_caches=caches)


def test_decode_ragged_sampled(kernel):
    """64 ragged sequences 4K-64K, 4 query tokens, paged: shortest and longest sequence checked."""
    wl = W.ragged()
    sampled = [int(np.argmin(wl.seq_lens)), int(np.argmax(wl.seq_lens))]
    caches = _mixed_caches(wl, sampled)
    decode_and_compare(wl, seqs=sampled, gpu_caches=caches)


def test_end_to_end_tiny_against_oracle_pipeline(kernel):
    """GPU quantize + GPU decode vs oracle quantize + oracle decode (codes equal away from
    boundaries, so the outputs agree to the attention tolerance unless a boundary code flipped)."""
    torch = _t()
    wl = W.tiny()
    k, v = wl.kv_source(0)
    gk = T.Cache.allocate(wl.k_bits, 1, wl.block_size, wl.n_blocks, wl.signs_k)
    gv = T.Cache.allocate(wl.v_bits, 1, wl.block_size, wl.n_blocks, wl.signs_v)
    T.tq_quantize_kv(gk, torch.from_numpy(k).cuda(), gv, torch.from_numpy(v).cuda(),
                     torch.from_numpy(wl.slots(0)).cuda())
    q = wl.queries()
    out = T.tq_decode_attention(gk, gv, torch.from_numpy(q).cuda(), torch.from_numpy(wl.seq_lens).cuda(),
                                torch.from_numpy(wl.block_table).cuda()).cpu().numpy()
    ok, ov = U.oracle_cache(wl, 0), U.oracle_cache(wl, 1)
    # codes: the oracle's away from boundaries
    k, v = wl.kv_source(0)
    kc, vc = gk.codes.cpu().numpy()[:, 0], gv.codes.cpu().numpy()[:, 0]
    slots = wl.slots(0)
    U.check_codes(kc.reshape(-1, kc.shape[-1])[slots], gk.norms.cpu().numpy()[:, 0].reshape(-1)[slots], k[:, 0],
                  wl.signs_k[0], wl.k_bits)
    U.check_codes(vc.reshape(-1, vc.shape[-1])[slots], gv.norms.cpu().numpy()[:, 0].reshape(-1)[slots], v[:, 0],
                  wl.signs_v[0], wl.v_bits)
    # attention: the oracle over the GPU-written cache, to the stated bar
    ref = O.decode_attention(q, U.oracle_cache_from_gpu(gk, ok), U.oracle_cache_from_gpu(gv, ov), wl.seq_lens,
                             wl.block_table, 1)
    worst, worst_e = U.assert_attention_close(out, ref, what="end-to-end tiny")
    # statistics only: the oracle pipeline (oracle codes) and the codes that differ
    flips = int(np.sum(gk.codes.cpu().numpy() != ok.codes) + np.sum(gv.codes.cpu().numpy() != ov.codes))
    want = O.decode_attention(q, ok, ov, wl.seq_lens, wl.block_table, 1)
    log(f"end-to-end tiny: vs the oracle on the GPU cache {worst:.2e} (element / bound {worst_e:.2e}); "
        f"vs the oracle pipeline {float(U.row_rel_err(out[0, 0, 0], want[0, 0, 0])):.2e} (statistic), "
        f"differing code bytes {flips}")


def test_graph_replay_matches_eager(kernel):
    """Quantize-append + decode captured in a HIP graph: every replay equals the eager result."""
    torch = _t()
    wl = W.small_decode(seed=21, n_seqs=2, lens=[1500, 700], n_qtok=2, n_q_heads=8, n_kv_heads=2, k_bits=4,
                        v_bits=3, block_size=64)
    ok, ov = U.oracle_cache(wl, 0), U.oracle_cache(wl, 1)
    gk, gv = U.gpu_cache_from(ok), U.gpu_cache_from(ov)
    q = torch.from_numpy(wl.queries()).cuda()
    lens = torch.from_numpy(wl.seq_lens).cuda()
    table = torch.from_numpy(wl.block_table).cuda()
    new_slots = torch.from_numpy(np.concatenate([wl.slots(b)[-2:] for b in range(2)])).cuda()
    gen = torch.Generator(device="cuda").manual_seed(5)
    knew = torch.randn((4, 2, 128), generator=gen, device="cuda").half()
    vnew = torch.randn((4, 2, 128), generator=gen, device="cuda").half()
    out = torch.zeros((2, 2, 8, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(T.decode_workspace_bytes(gk, gv, 2, 2, 8, wl.block_table.shape[1]), dtype=torch.uint8,
                     device="cuda")

    def step():
        T.tq_quantize_kv(gk, knew, gv, vnew, new_slots)
        T.tq_decode_attention(gk, gv, q, lens, table, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    codes_eager = gk.codes.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from eager"
        assert torch.equal(gk.codes, codes_eager)


@pytest.mark.parametrize("tau", [0.0, 1e-3])
def test_graph_replay_fused_append_matches_eager(tau, monkeypatch):
    """The fused append + decode call captured in a HIP graph (as the benchmark
    replays it): every replay equals the eager result, output and cache rows."""
    monkeypatch.setattr(T, "default_options", None)
    torch = _t()
    wl = W.small_decode(seed=22, n_seqs=2, lens=[1500, 700], n_qtok=2, n_q_heads=8, n_kv_heads=2, k_bits=4,
                        v_bits=3, tau=tau, block_size=64)
    ok, ov = U.oracle_cache(wl, 0), U.oracle_cache(wl, 1)
    gk, gv = U.gpu_cache_from(ok), U.gpu_cache_from(ov)
    q = torch.from_numpy(wl.queries()).cuda()
    lens = torch.from_numpy(wl.seq_lens).cuda()
    table = torch.from_numpy(wl.block_table).cuda()
    gen = torch.Generator(device="cuda").manual_seed(6)
    knew = torch.randn((4, 2, 128), generator=gen, device="cuda").half()
    vnew = torch.randn((4, 2, 128), generator=gen, device="cuda").half()
    out = torch.zeros((2, 2, 8, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(T.decode_workspace_bytes(gk, gv, 2, 2, 8, wl.block_table.shape[1], tau), dtype=torch.uint8,
                     device="cuda")

    def step():
        T.tq_append_decode_attention(gk, knew, gv, vnew, q, lens, table, 0.0, tau, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    kc, vc, kn, vn = gk.codes.clone(), gv.codes.clone(), gk.norms.clone(), gv.norms.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from eager"
        assert torch.equal(gk.codes, kc) and torch.equal(gv.codes, vc)
        assert torch.equal(gk.norms, kn) and torch.equal(gv.norms, vn)


# ------------------------------------------------- heads of 256 / 512 elements (R12)

def _skip_valu_for_wide_heads(kernel):
    if kernel == "valu":
        pytest.skip("heads of several blocks run on the matrix-core pass only (the vector-ALU pass rejects them)")


@pytest.mark.parametrize("n_kv", [3, 2, 8])
@pytest.mark.parametrize("head_dim", [256, 512])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_wide_heads(bits, head_dim, n_kv):
    """Every 128-slice of every head is quantized with its own sign words (R12),
    from a padded token stride and into shuffled slots.  (Sub-heads dividing 16 take
    the matrix-core transform: 2 KV heads, and 8 of 256 elements; 3 KV heads and 8
    of 512 elements the vector path.)"""
    torch = _t()
    rng = np.random.default_rng(7 * bits + head_dim + (0 if n_kv == 3 else 1000 * n_kv))
    nb, n_tok, bs, pad = head_dim // 128, 90, 16, 24
    x = (rng.standard_normal((n_tok, n_kv, head_dim)) * rng.lognormal(0, 1, (1, n_kv, head_dim))).astype(np.float16)
    signs = W.random_sign_words(rng, n_kv * nb)
    n_blocks = -(-n_tok // bs) + 1
    slots = rng.permutation(n_blocks * bs)[:n_tok].astype(np.int64)
    slots[5] = -1
    g = T.Cache.allocate(bits, n_kv, bs, n_blocks, signs, head_dim=head_dim)
    g.codes.fill_(0xAB)
    src = np.zeros((n_tok, n_kv * head_dim + pad), np.float16)
    src[:, : n_kv * head_dim] = x.reshape(n_tok, -1)
    src_t = torch.from_numpy(src).cuda()
    view = torch.as_strided(src_t, (n_tok, n_kv, head_dim), (n_kv * head_dim + pad, head_dim, 1))
    T.tq_quantize_kv(g, view, None, None, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    codes = g.codes.cpu().numpy().transpose(0, 2, 1, 3).reshape(-1, n_kv * nb, 16 * bits)
    norms = g.norms.cpu().numpy().transpose(0, 2, 1).reshape(-1, n_kv * nb)
    ok = slots >= 0
    near = 0
    for h in range(n_kv):
        for i in range(nb):
            sub = nb * h + i
            near += U.check_codes(codes[slots[ok], sub], norms[slots[ok], sub], x[ok, h, 128 * i:128 * (i + 1)],
                                  signs[sub], bits)
    untouched = np.setdiff1d(np.arange(codes.shape[0]), slots[ok])
    assert np.all(codes[untouched] == 0xAB), "a skipped or unused slot was written"
    # the dequantized heads: every block, in order
    oc = O.new_cache(bits, n_kv, bs, n_blocks, signs, O.build_codebook(bits), head_dim=head_dim)
    O.cache_write(oc, x, slots)
    rd = torch.from_numpy(slots[ok]).cuda()
    got = T.tq_dequantize(g, rd).cpu().numpy()
    assert got.shape == (int(ok.sum()), n_kv, head_dim)
    for h in range(n_kv):
        want = O.cache_read(oc, slots[ok], h)
        err = U.row_rel_err(got[:, h], want)
        assert np.max(err) < 1e-4, f"dequantize head {h}: {np.max(err)} (near-boundary codes {near})"
    log(f"quantize head_dim={head_dim} n_kv={n_kv} bits={bits}: near-boundary {near}")


@pytest.mark.parametrize("case", [
    # (n_seqs, lens, n_qtok, n_q_heads, n_kv_heads, k_bits, v_bits, block_size, head_dim)
    (1, [700], 1, 4, 1, 4, 3, 256, 256),
    (2, [1000, 33], 1, 16, 8, 3, 2, 256, 256),
    (2, [300, 129], 4, 16, 4, 4, 4, 64, 256),
    (2, [1500, 600], 1, 8, 2, 4, 3, 100, 512),
    (3, [77, 5, 260], 2, 8, 1, 2, 3, 16, 512),
    (1, [4097], 3, 6, 2, 3, 3, 256, 512),
    (2, [900, 70], 1, 8, 2, T.BITS_FP16, 3, 256, 256),
    (2, [513, 64], 2, 8, 2, T.BITS_FP16, 4, 64, 512),
], ids=lambda c: f"d{c[8]}-s{c[0]}-q{c[2]}-h{c[3]}/{c[4]}-b{c[5]}{c[6]}-bs{c[7]}")
def test_decode_wide_heads(case, kernel):
    """Heads of 256 / 512 elements: 1-16 rows per KV head, whole and partial slices,
    contiguous and paged layouts, K compressed or float16."""
    _skip_valu_for_wide_heads(kernel)
    n_seqs, lens, n_qtok, hq, hkv, kb, vb, bs, hd = case
    wl = W.small_decode(seed=sum(lens) + hd, n_seqs=n_seqs, lens=lens, n_qtok=n_qtok, n_q_heads=hq,
                        n_kv_heads=hkv, k_bits=kb, v_bits=vb, block_size=bs, head_dim=hd)
    decode_and_compare(wl)


@pytest.mark.parametrize("head_dim", [256, 512])
@pytest.mark.parametrize("tau", [1e-4, 3e-2, 1.5])
def test_decode_wide_heads_sparse(tau, head_dim, kernel):
    """Sparse V with heads of several blocks (the waves of a group share each gate
    decision; groups decide apart)."""
    _skip_valu_for_wide_heads(kernel)
    wl = W.small_decode(seed=53 + head_dim, n_seqs=2, lens=[2500, 700], n_qtok=2, n_q_heads=8, n_kv_heads=2,
                        k_bits=4, v_bits=2, tau=tau, block_size=256, head_dim=head_dim)
    out, _ = decode_and_compare(wl)
    if tau > 1:
        assert np.all(out == 0)


def test_decode_wide_heads_rows_with_no_visible_token_are_zero(kernel):
    _skip_valu_for_wide_heads(kernel)
    wl = W.small_decode(seed=4, n_seqs=2, lens=[2, 0], n_qtok=4, n_q_heads=2, n_kv_heads=1, k_bits=4,
                        v_bits=3, block_size=16, head_dim=512)
    out, _ = decode_and_compare(wl)
    assert np.all(out[0, :2] == 0) and np.all(out[1] == 0)


def _sampled_head_caches(wl, heads):
    """Device caches of the whole workload whose sampled KV heads hold oracle-written
    codes (other heads zero), and the oracle caches of the sampled heads alone."""
    torch = _t()
    nb = wl.blocks_per_head
    sub = np.concatenate([np.arange(nb * h, nb * (h + 1)) for h in heads])

    def build():
        caches = []
        for side, bits, signs in ((0, wl.k_bits, wl.signs_k), (1, wl.v_bits, wl.signs_v)):
            c = O.new_cache(bits, len(heads), wl.block_size, wl.n_blocks, signs[sub],
                            None if bits == O.FP16 else O.build_codebook(bits), head_dim=wl.head_dim)
            for b in range(wl.n_seqs):
                k, v = wl.kv_source(b)
                O.cache_write(c, (k if side == 0 else v)[:, heads], wl.slots(b))
            caches.append(c)
        return caches

    ok, ov = _memo(("heads", tuple(heads)) + _wl_key(wl), build)
    gk = T.Cache.allocate(wl.k_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, wl.signs_k, head_dim=wl.head_dim)
    gv = T.Cache.allocate(wl.v_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, wl.signs_v, head_dim=wl.head_dim)
    idx = torch.as_tensor(sub, device="cuda")
    for oc, g in ((ok, gk), (ov, gv)):
        g.codes.index_copy_(1, idx, torch.from_numpy(oc.codes).cuda())
        g.norms.index_copy_(1, idx, torch.from_numpy(oc.norms).cuda())
    torch.cuda.synchronize()
    return ok, ov, gk, gv


@pytest.mark.parametrize("head_dim,heads", [(256, [0, 5]), (512, [2, 7])])
def test_decode_wide_heads_llama8b_sampled(head_dim, heads, kernel):
    """The Llama-3-8B-shaped decode (32768 tokens, 32 / 8 heads, K4 / V3) with heads of
    256 / 512 elements, at full size: every row of two KV heads checked."""
    _skip_valu_for_wide_heads(kernel)
    torch = _t()
    wl = W.llama8b_wide(head_dim)
    ok, ov, gk, gv = _sampled_head_caches(wl, heads)
    q = wl.queries()
    out = T.tq_decode_attention(gk, gv, torch.from_numpy(q).cuda(), torch.from_numpy(wl.seq_lens).cuda(),
                                torch.from_numpy(wl.block_table).cuda()).cpu().numpy()
    qh = np.concatenate([np.arange(h * wl.group, (h + 1) * wl.group) for h in heads])
    want = _memo(("heads-out", tuple(heads)) + _wl_key(wl),
                 lambda: O.decode_attention(q[:, :, qh], ok, ov, wl.seq_lens, wl.block_table, wl.n_qtok))
    worst, worst_e = U.assert_attention_close(out[:, :, qh], want, what=f"decode {wl.name} heads {heads}")
    log(f"decode {wl.name} heads {heads}: worst row rel err {worst:.2e}, element error / bound {worst_e:.2e}")


# ----------------------------------------------------------- kept V channels (R13)

def _skip_valu_for_kept(kernel):
    if kernel == "valu":
        pytest.skip("kept V channels run on the matrix-core pass only (the vector-ALU pass rejects them)")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n_kv,k", [(1, 1), (3, 5), (8, 16)])
def test_quantize_kept_channels(bits, n_kv, k):
    """The kept channels are stored exactly, slot-major per page; the codes and norms
    are those of the vector with those channels zeroed; skipped and unused slots are
    untouched; dequantize puts the kept values back."""
    torch = _t()
    rng = np.random.default_rng(11 * bits + 7 * k + n_kv)
    n_tok, bs, pad = 77, 16, 40
    x = rng.standard_normal((n_tok, n_kv, 128))
    x[:, :, rng.choice(128, size=min(k, 4), replace=False)] *= 20
    x = x.astype(np.float16)
    signs = W.random_sign_words(rng, n_kv)
    idx = O.select_outlier_channels(x, k)
    n_blocks = -(-n_tok // bs) + 1
    slots = rng.permutation(n_blocks * bs)[:n_tok].astype(np.int64)
    slots[3] = -1
    g = T.Cache.allocate(bits, n_kv, bs, n_blocks, signs, outlier_channels=idx)
    g.codes.fill_(0xAB)
    g.outliers.fill_(7)
    src = np.zeros((n_tok, n_kv * 128 + pad), np.float16)
    src[:, : n_kv * 128] = x.reshape(n_tok, -1)
    view = torch.as_strided(torch.from_numpy(src).cuda(), (n_tok, n_kv, 128), (n_kv * 128 + pad, 128, 1))
    T.tq_quantize_kv(None, None, g, view, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ok = slots >= 0
    oc = O.new_cache(bits, n_kv, bs, n_blocks, signs, O.build_codebook(bits), outlier_channels=idx)
    O.cache_write(oc, x, slots)
    kept = g.outliers.cpu().numpy()          # [n_blocks, n_kv, k, bs]
    blk, off = slots[ok] // bs, slots[ok] % bs
    np.testing.assert_array_equal(kept[blk, :, :, off], oc.outliers[blk, :, :, off])
    codes = g.codes.cpu().numpy().transpose(0, 2, 1, 3).reshape(-1, n_kv, 16 * bits)
    norms = g.norms.cpu().numpy().transpose(0, 2, 1).reshape(-1, n_kv)
    near = 0
    for h in range(n_kv):
        z = x[:, h].copy()
        z[:, idx[h].astype(np.int64)] = 0
        near += U.check_codes(codes[slots[ok], h], norms[slots[ok], h], z[ok], signs[h], bits)
    untouched = np.setdiff1d(np.arange(n_blocks * bs), slots[ok])
    assert np.all(codes[untouched] == 0xAB)
    ub, uo = untouched // bs, untouched % bs
    assert np.all(kept[ub, :, :, uo] == np.float16(7))
    rd = torch.from_numpy(slots[ok]).cuda()
    got32 = T.tq_dequantize(g, rd).cpu().numpy()
    got16 = T.tq_dequantize(g, rd, fp16=True).cpu().numpy()
    for h in range(n_kv):
        want = O.cache_read(oc, slots[ok], h)
        ch = idx[h].astype(np.int64)
        np.testing.assert_array_equal(got32[:, h][:, ch], want[:, ch])
        np.testing.assert_array_equal(got16[:, h][:, ch].astype(np.float64), want[:, ch])
        assert np.max(U.row_rel_err(got32[:, h], want)) < 1e-5
    log(f"quantize kept channels bits={bits} n_kv={n_kv} k={k}: near-boundary {near}")


@pytest.mark.parametrize("case", [
    # (n_seqs, lens, n_qtok, n_q_heads, n_kv_heads, k_bits, v_bits, block_size, kept)
    (1, [700], 1, 4, 1, 4, 3, 256, 8),
    (2, [1000, 33], 1, 32, 8, 3, 2, 256, 16),
    (2, [300, 129], 4, 16, 4, 4, 4, 64, 4),
    (3, [77, 5, 260], 2, 8, 1, 2, 3, 16, 1),
    (2, [1500, 600], 1, 8, 2, 4, 2, 100, 5),
    (1, [4097], 3, 6, 2, 3, 3, 256, 16),
    (2, [900, 70], 1, 8, 2, T.BITS_FP16, 3, 256, 8),
], ids=lambda c: f"s{c[0]}-q{c[2]}-h{c[3]}/{c[4]}-b{c[5]}{c[6]}-bs{c[7]}-k{c[8]}")
def test_decode_kept_channels(case, kernel):
    """V keeping 1-16 channels in float16 (4 planted x20): 1-16 rows per KV head,
    contiguous and paged layouts, ragged tails, K compressed or float16."""
    _skip_valu_for_kept(kernel)
    n_seqs, lens, n_qtok, hq, hkv, kb, vb, bs, kept = case
    wl = W.small_decode(seed=sum(lens) + 3 * kept, n_seqs=n_seqs, lens=lens, n_qtok=n_qtok, n_q_heads=hq,
                        n_kv_heads=hkv, k_bits=kb, v_bits=vb, block_size=bs, v_planted=4, v_kept=kept)
    decode_and_compare(wl)


@pytest.mark.parametrize("tau", [1e-4, 3e-2, 1.5])
def test_decode_kept_channels_sparse(tau, kernel):
    _skip_valu_for_kept(kernel)
    wl = W.small_decode(seed=61, n_seqs=2, lens=[2500, 700], n_qtok=2, n_q_heads=8, n_kv_heads=2,
                        k_bits=4, v_bits=2, tau=tau, block_size=256, v_planted=4, v_kept=8)
    out, _ = decode_and_compare(wl)
    if tau > 1:
        assert np.all(out == 0)


def test_decode_kept_channels_llama8b_full(kernel):
    """The Llama-3-8B-shaped decode (32768 tokens, 32 / 8 heads, K4 / V3) with 4 V
    outlier channels x20 and 8 kept channels per head: every row."""
    _skip_valu_for_kept(kernel)
    decode_and_compare(W.llama8b_vout())


def test_end_to_end_kept_channels(kernel):
    """GPU selection, GPU quantize and GPU decode against the oracle pipeline on the
    same float16 inputs (channels selected by both sides from the same warm-up data)."""
    _skip_valu_for_kept(kernel)
    torch = _t()
    wl = W.small_decode(seed=71, n_seqs=2, lens=[900, 257], n_qtok=1, n_q_heads=8, n_kv_heads=2, k_bits=4,
                        v_bits=3, block_size=64, v_planted=4, v_kept=6)
    gidx = T.tq_select_outlier_channels(wl.warmup_v(), wl.v_kept)
    oidx = O.select_outlier_channels(wl.warmup_v(), wl.v_kept)
    assert np.array_equal(gidx[:, : wl.v_kept], oidx)
    gk = T.Cache.allocate(wl.k_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, wl.signs_k)
    gv = T.Cache.allocate(wl.v_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, wl.signs_v,
                          outlier_channels=gidx[:, : wl.v_kept])
    for b in range(wl.n_seqs):
        k, v = wl.kv_source(b)
        T.tq_quantize_kv(gk, torch.from_numpy(k).cuda(), gv, torch.from_numpy(v).cuda(),
                         torch.from_numpy(wl.slots(b)).cuda())
    q = wl.queries()
    out = T.tq_decode_attention(gk, gv, torch.from_numpy(q).cuda(), torch.from_numpy(wl.seq_lens).cuda(),
                                torch.from_numpy(wl.block_table).cuda()).cpu().numpy()
    ok, ov = oracle_caches(wl)
    assert np.array_equal(gv.outliers.cpu().numpy(), ov.outliers)
    # attention: the oracle over the GPU-written cache, to the stated bar
    ref = O.decode_attention(q, U.oracle_cache_from_gpu(gk, ok), U.oracle_cache_from_gpu(gv, ov), wl.seq_lens,
                             wl.block_table, wl.n_qtok)
    worst, worst_e = U.assert_attention_close(out, ref, what="end-to-end kept channels")
    # statistics only: the oracle pipeline and the code bytes that differ from it
    flips = int(np.sum(gk.codes.cpu().numpy() != ok.codes) + np.sum(gv.codes.cpu().numpy() != ov.codes))
    want = O.decode_attention(q, ok, ov, wl.seq_lens, wl.block_table, wl.n_qtok)
    log(f"end-to-end kept channels: vs the oracle on the GPU cache {worst:.2e} (element / bound {worst_e:.2e}); "
        f"vs the oracle pipeline {float(np.max(U.row_rel_err(out, want))):.2e} (statistic), "
        f"differing code bytes {flips}")


# ----------------------------------------------------------- fused append + decode

def _old_context_cache(wl, side):
    """Oracle cache of every position but each sequence's last n_qtok (the context
    before the new tokens)."""
    bits = wl.k_bits if side == 0 else wl.v_bits
    signs = wl.signs_k if side == 0 else wl.signs_v
    c = O.new_cache(bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, signs, O.build_codebook(bits))
    for b in range(wl.n_seqs):
        n_old = int(wl.seq_lens[b]) - wl.n_qtok
        if n_old <= 0:
            continue
        k, v = wl.kv_source(b)
        O.cache_write(c, (k if side == 0 else v)[:n_old], wl.slots(b)[:n_old])
    return c


def append_and_compare(wl, tau=None):
    """tq_append_decode_attention on caches holding the old context, against (a) the
    oracle pipeline (oracle-quantized new tokens, oracle attention) and (b) the two
    calls tq_quantize_kv + tq_decode_attention on the same caches."""
    torch = _t()
    tau = wl.tau if tau is None else tau
    ok_old, ov_old = _memo(("old",) + _wl_key(wl), lambda: (_old_context_cache(wl, 0), _old_context_cache(wl, 1)))
    ok, ov = oracle_caches(wl)
    n_new = wl.n_seqs * wl.n_qtok
    k_new = np.zeros((n_new, wl.n_kv_heads, 128), np.float16)
    v_new = np.zeros((n_new, wl.n_kv_heads, 128), np.float16)
    slots = np.full(n_new, -1, np.int64)
    for b in range(wl.n_seqs):
        length = int(wl.seq_lens[b])
        if length == 0:
            continue
        k, v = wl.kv_source(b)
        sl = wl.slots(b)
        for j in range(wl.n_qtok):
            p = length - wl.n_qtok + j
            if p >= 0:
                k_new[b * wl.n_qtok + j], v_new[b * wl.n_qtok + j] = k[p], v[p]
                slots[b * wl.n_qtok + j] = sl[p]
    q = torch.from_numpy(wl.queries()).cuda()
    lens = torch.from_numpy(wl.seq_lens).cuda()
    table = torch.from_numpy(wl.block_table).cuda()
    kn, vn = torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda()
    # (b) the two calls
    gk2, gv2 = U.gpu_cache_from(ok_old), U.gpu_cache_from(ov_old)
    T.tq_quantize_kv(gk2, kn, gv2, vn, torch.from_numpy(slots).cuda())
    out2 = T.tq_decode_attention(gk2, gv2, q, lens, table, 0.0, tau).cpu().numpy()
    # the fused call
    gk, gv = U.gpu_cache_from(ok_old), U.gpu_cache_from(ov_old)
    out = T.tq_append_decode_attention(gk, kn, gv, vn, q, lens, table, 0.0, tau).cpu().numpy()
    torch.cuda.synchronize()
    # the new rows: codes as the oracle's (away from boundaries), norms, untouched elsewhere
    kc, vc = gk.codes.cpu().numpy(), gv.codes.cpu().numpy()
    knm, vnm = gk.norms.cpu().numpy(), gv.norms.cpu().numpy()
    m = slots >= 0
    blk, off = slots[m] // wl.block_size, slots[m] % wl.block_size
    near = 0
    for h in range(wl.n_kv_heads):
        near += U.check_codes(kc[blk, h, off], knm[blk, h, off], k_new[m, h], wl.signs_k[h], wl.k_bits)
        near += U.check_codes(vc[blk, h, off], vnm[blk, h, off], v_new[m, h], wl.signs_v[h], wl.v_bits)
    old = np.ones(kc.shape[:3], bool)
    old[blk, :, off] = False
    assert np.array_equal(kc[old], ok_old.codes[old]) and np.array_equal(vc[old], ov_old.codes[old])
    # attention: the oracle over the cache each GPU path wrote (the attention
    # arithmetic alone, to the stated bar), for the fused call and the two calls
    q_np = wl.queries()
    for name, o_gpu, gk_, gv_ in (("fused", out, gk, gv), ("two calls", out2, gk2, gv2)):
        okg, ovg = U.oracle_cache_from_gpu(gk_, ok_old), U.oracle_cache_from_gpu(gv_, ov_old)
        ref, weights = O.decode_attention(q_np, okg, ovg, wl.seq_lens, wl.block_table, wl.n_qtok, 0.0, tau,
                                          return_weights=True)
        worst, worst_e = U.assert_attention_close(o_gpu, ref, _gate_slack(wl, ovg, weights, tau),
                                                  what=f"append+decode {wl.name} ({name})")
        log(f"append+decode {wl.name} ({name}): vs the oracle on its cache: worst row rel err {worst:.2e}, "
            f"element error / bound {worst_e:.2e}")
    # statistics only: codes unlike the oracle's (elements within rounding of a
    # boundary) and the whole-pipeline difference they make
    flips = int(np.sum(kc != ok.codes) + np.sum(vc != ov.codes))
    want = _memo(("decode-app", tau) + _wl_key(wl),
                 lambda: O.decode_attention(q_np, ok, ov, wl.seq_lens, wl.block_table, wl.n_qtok, 0.0, tau))
    log(f"append+decode {wl.name}: near-boundary {near}, code bytes unlike the oracle's {flips}, "
        f"vs the oracle pipeline: worst row rel err {float(np.max(U.row_rel_err(out, want))):.2e} (statistic)")
    return out


@pytest.mark.parametrize("case", [
    # (n_seqs, lens, n_qtok, n_q_heads, n_kv_heads, k_bits, v_bits, block_size)
    (1, [700], 1, 4, 1, 4, 3, 256),
    (1, [258], 4, 4, 1, 4, 3, 64),            # the new positions cross a 256-token chunk
    (3, [1000, 2, 257], 4, 8, 2, 3, 2, 16),   # a sequence shorter than n_qtok
    (2, [1500, 600], 2, 16, 2, 4, 4, 100),    # 16 rows per KV head
    (2, [513, 64], 3, 6, 2, 2, 3, 64),
    (3, [300, 0, 5], 2, 4, 1, 4, 3, 64),      # an empty sequence between two others
    (1, [32768], 1, 32, 8, 4, 3, 256),        # the Llama-3-8B decode shape
], ids=lambda c: f"s{c[0]}-q{c[2]}-h{c[3]}/{c[4]}-b{c[5]}{c[6]}-bs{c[7]}")
def test_append_decode(case, kernel):
    if kernel == "valu":
        pytest.skip("the fused append runs on the matrix-core pass only (the vector-ALU pass rejects it)")
    n_seqs, lens, n_qtok, hq, hkv, kb, vb, bs = case
    wl = W.small_decode(seed=sum(lens) + 5 * n_qtok, n_seqs=n_seqs, lens=lens, n_qtok=n_qtok, n_q_heads=hq,
                        n_kv_heads=hkv, k_bits=kb, v_bits=vb, block_size=bs)
    append_and_compare(wl)


@pytest.mark.parametrize("tau", [1e-4, 3e-2])
def test_append_decode_sparse(tau, kernel):
    if kernel == "valu":
        pytest.skip("the fused append runs on the matrix-core pass only (the vector-ALU pass rejects it)")
    wl = W.small_decode(seed=83, n_seqs=2, lens=[2500, 700], n_qtok=2, n_q_heads=8, n_kv_heads=2, k_bits=4,
                        v_bits=2, tau=tau, block_size=256)
    append_and_compare(wl)
