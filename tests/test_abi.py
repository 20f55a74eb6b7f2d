"""C-ABI contract tests that need no GPU: the library loads, exports every
function include/tq.h declares, builds the same codebook as the oracle, and
rejects invalid arguments on the host before launching anything."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle as O
from compressed_kv_attention_tq_amd import tq as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(T.LIB_PATH), reason="libtq.so not built")


def header_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = T.load_library()
    names = header_functions()
    assert set(names) == set(T.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in [(0, "TQ_OK"), (1, "TQ_ERR_INVALID_ARG"), (2, "TQ_ERR_UNSUPPORTED"),
                       (3, "TQ_ERR_WORKSPACE"), (4, "TQ_ERR_HIP")]:
        assert T.status_string(code) == name


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_oracle_bit_exact(bits):
    cb = T.tq_build_codebook(bits)
    ref = O.build_codebook(bits)
    assert cb.bits == bits and cb.n_levels == 1 << bits
    assert np.array_equal(cb.centroid_array, ref.centroids.astype(np.float32))
    assert np.array_equal(cb.boundary_array, ref.boundaries.astype(np.float32))
    assert math.isclose(cb.mse, ref.mse, rel_tol=1e-9)
    assert list(cb.centroids[cb.n_levels:]) == [0.0] * (16 - cb.n_levels)


def test_codebook_other_sigma_scales():
    a = T.tq_build_codebook(3, 1.0)
    b = T.tq_build_codebook(3, 0.5)
    ref = O.build_codebook(3, 0.5)
    assert np.array_equal(b.centroid_array, ref.centroids.astype(np.float32))
    assert np.allclose(a.centroid_array * 0.5, b.centroid_array, rtol=1e-3)


def test_codebook_rejects_bad_arguments():
    lib = T.load_library()
    cb = T.TQCodebook()
    assert lib.tq_build_codebook(0, 0.1, ctypes.byref(cb)) == T.TQ_ERR_UNSUPPORTED
    assert lib.tq_build_codebook(5, 0.1, ctypes.byref(cb)) == T.TQ_ERR_UNSUPPORTED
    assert lib.tq_build_codebook(2, 0.0, ctypes.byref(cb)) == T.TQ_ERR_INVALID_ARG
    assert lib.tq_build_codebook(2, -1.0, ctypes.byref(cb)) == T.TQ_ERR_INVALID_ARG
    assert lib.tq_build_codebook(2, float("nan"), ctypes.byref(cb)) == T.TQ_ERR_INVALID_ARG
    assert lib.tq_build_codebook(2, 0.1, None) == T.TQ_ERR_INVALID_ARG


FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced: every call below fails validation


def fake_cache(bits=4, n_kv=2, block_size=256, n_blocks=4, head_dim=128):
    d = T.TQCache()
    d.bits, d.n_kv_heads, d.head_dim, d.block_size, d.n_blocks = bits, n_kv, head_dim, block_size, n_blocks
    d.codes, d.norms, d.signs = FAKE, FAKE + 0x100000, FAKE + 0x200000
    if 1 <= bits <= 4:
        d.cb = T.tq_build_codebook(bits)
    return d


VALU = T.DecodeOptions(kernel=T.DECODE_KERNEL_VALU)


def decode_call(k=None, v=None, n_seqs=1, n_qtok=1, n_q_heads=2, max_blocks=4, scale=0.0, tau=0.0,
                ws=None, ws_bytes=None, q=FAKE, out=FAKE, options=None):
    """tq_decode_attention (options None) or tq_decode_attention_ex with the options."""
    lib = T.load_library()
    k = fake_cache() if k is None else k
    v = fake_cache(bits=3) if v is None else v
    size = ctypes.c_size_t(0 if ws_bytes is None else ws_bytes)
    if options is None:
        st = lib.tq_decode_attention(ctypes.byref(k), ctypes.byref(v), q, n_seqs, n_qtok, n_q_heads, FAKE, FAKE,
                                     max_blocks, scale, tau, out, ws, ctypes.byref(size), None)
    else:
        st = lib.tq_decode_attention_ex(ctypes.byref(k), ctypes.byref(v), q, n_seqs, n_qtok, n_q_heads, FAKE,
                                        FAKE, max_blocks, scale, tau, out, ws, ctypes.byref(size), None,
                                        ctypes.byref(options.c()), None)
    return st, size.value


def test_decode_options():
    """The kernel and the chunk are arguments: the workspace follows them, bad values
    are rejected, and a zeroed options struct is the default call."""
    _, dflt = decode_call()
    assert decode_call(options=T.DecodeOptions()) == (T.TQ_OK, dflt)
    assert decode_call(options=T.DecodeOptions(kernel=T.DECODE_KERNEL_MFMA)) == (T.TQ_OK, dflt)
    st, valu = decode_call(options=VALU)
    assert st == T.TQ_OK and valu != dflt            # the vector-ALU pass keeps rotated queries too
    _, big = decode_call(max_blocks=64, options=T.DecodeOptions(chunk=256))
    _, small = decode_call(max_blocks=64, options=T.DecodeOptions(chunk=1024))
    assert big > small                               # more chunks, more partials
    for bad in (T.DecodeOptions(kernel=3), T.DecodeOptions(kernel=-1), T.DecodeOptions(chunk=100),
                T.DecodeOptions(chunk=-256), T.DecodeOptions(chunk=1 << 21),
                T.DecodeOptions(kernel=T.DECODE_KERNEL_VALU, chunk=256)):   # the ALU pass's unit is 512
        assert decode_call(options=bad)[0] == T.TQ_ERR_INVALID_ARG, bad


def test_decode_workspace_query():
    st, size = decode_call()
    assert st == T.TQ_OK and size > 0 and size % 256 == 0
    st, size_sparse = decode_call(tau=1e-4)
    assert st == T.TQ_OK and size_sparse > size
    st, size0 = decode_call(n_seqs=0)
    assert st == T.TQ_OK and size0 == 0
    st, big = decode_call(n_seqs=8, max_blocks=64)
    assert big > size


def test_decode_validation_errors():
    assert decode_call(k=fake_cache(head_dim=64))[0] == T.TQ_ERR_UNSUPPORTED
    assert decode_call(k=fake_cache(bits=5))[0] == T.TQ_ERR_UNSUPPORTED
    assert decode_call(v=fake_cache(bits=3, n_kv=4))[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(v=fake_cache(bits=3, block_size=128))[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(n_q_heads=3)[0] == T.TQ_ERR_INVALID_ARG         # not a multiple of n_kv
    assert decode_call(n_q_heads=2 * 17)[0] == T.TQ_ERR_UNSUPPORTED    # 17 rows per KV head
    assert decode_call(n_q_heads=2 * 4, n_qtok=5)[0] == T.TQ_ERR_UNSUPPORTED
    assert decode_call(n_qtok=0)[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(n_seqs=-1)[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(max_blocks=0)[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(tau=-1.0)[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(tau=float("nan"))[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(scale=-0.1)[0] == T.TQ_ERR_INVALID_ARG
    bad_cb = fake_cache()
    bad_cb.cb.bits = 3
    assert decode_call(k=bad_cb)[0] == T.TQ_ERR_INVALID_ARG
    null_codes = fake_cache()
    null_codes.codes = None
    assert decode_call(k=null_codes)[0] == T.TQ_ERR_INVALID_ARG
    misaligned = fake_cache()
    misaligned.codes = FAKE + 4
    assert decode_call(k=misaligned)[0] == T.TQ_ERR_INVALID_ARG
    _, need = decode_call()
    assert decode_call(ws=FAKE, ws_bytes=need - 1)[0] == T.TQ_ERR_WORKSPACE
    assert decode_call(ws=FAKE + 16, ws_bytes=need)[0] == T.TQ_ERR_INVALID_ARG   # not 256-aligned
    assert decode_call(ws=FAKE, ws_bytes=need, q=None)[0] == T.TQ_ERR_INVALID_ARG
    assert decode_call(ws=FAKE, ws_bytes=need, out=None)[0] == T.TQ_ERR_INVALID_ARG
    lib = T.load_library()
    k, v = fake_cache(), fake_cache(bits=3)
    assert lib.tq_decode_attention(ctypes.byref(k), ctypes.byref(v), FAKE, 1, 1, 2, FAKE, FAKE, 4, 0.0, 0.0,
                                   FAKE, None, None, None) == T.TQ_ERR_INVALID_ARG


def test_decode_wide_heads_validation():
    """Heads of 256 / 512 elements: both sides alike; the workspace holds nb
    accumulators per row; only the matrix-core pass takes them."""
    _, size128 = decode_call()
    for hd in (256, 512):
        st, size = decode_call(k=fake_cache(head_dim=hd), v=fake_cache(bits=3, head_dim=hd))
        assert st == T.TQ_OK and size > size128
        assert decode_call(k=fake_cache(head_dim=hd))[0] == T.TQ_ERR_INVALID_ARG   # V is 128 wide
    assert decode_call(k=fake_cache(head_dim=384), v=fake_cache(bits=3, head_dim=384))[0] == T.TQ_ERR_UNSUPPORTED
    assert decode_call(k=fake_cache(head_dim=256), v=fake_cache(bits=3, head_dim=256), options=VALU)[0] == \
        T.TQ_ERR_UNSUPPORTED
    assert decode_call(options=VALU)[0] == T.TQ_OK


def test_quantize_validation_errors():
    lib = T.load_library()
    k, v = fake_cache(), fake_cache(bits=3)
    call = lambda kk, ks, vv, vs, stride=256, n=4, slots=FAKE: lib.tq_quantize_kv(
        ctypes.byref(kk) if kk is not None else None, ks, ctypes.byref(vv) if vv is not None else None, vs,
        stride, n, slots, None)
    assert call(k, FAKE, v, FAKE, n=-1) == T.TQ_ERR_INVALID_ARG
    assert call(k, None, v, FAKE) == T.TQ_ERR_INVALID_ARG
    assert call(k, FAKE + 2, v, FAKE) == T.TQ_ERR_INVALID_ARG          # src not 16-byte aligned
    assert call(k, FAKE, v, FAKE, stride=255) == T.TQ_ERR_INVALID_ARG   # < n_kv * 128
    assert call(k, FAKE, v, FAKE, stride=260) == T.TQ_ERR_INVALID_ARG   # not a multiple of 8
    assert call(k, FAKE, v, FAKE, slots=None) == T.TQ_ERR_INVALID_ARG
    assert call(k, FAKE, fake_cache(bits=3, n_kv=4), FAKE, stride=512) == T.TQ_ERR_INVALID_ARG
    assert call(fake_cache(head_dim=96), FAKE, None, None) == T.TQ_ERR_UNSUPPORTED
    assert call(fake_cache(head_dim=384), FAKE, None, None) == T.TQ_ERR_UNSUPPORTED
    # heads of 256: both sides alike, and the token stride covers n_kv * 256 elements
    assert call(fake_cache(head_dim=256), FAKE, v, FAKE, stride=512) == T.TQ_ERR_INVALID_ARG
    assert call(fake_cache(head_dim=256), FAKE, None, None, stride=511 - 7) == T.TQ_ERR_INVALID_ARG
    assert call(fake_cache(bits=1), FAKE, None, None) == T.TQ_ERR_UNSUPPORTED
    assert call(fake_cache(block_size=1 << 20, n_blocks=1 << 12), FAKE, None, None) == T.TQ_ERR_UNSUPPORTED
    # no-ops: nothing to do, nothing launched
    assert call(k, FAKE, v, FAKE, n=0) == T.TQ_OK
    assert call(None, None, None, None) == T.TQ_OK


def test_dequantize_validation_errors():
    lib = T.load_library()
    c = fake_cache()
    assert lib.tq_dequantize(ctypes.byref(c), FAKE, -1, FAKE, 0, None) == T.TQ_ERR_INVALID_ARG
    assert lib.tq_dequantize(ctypes.byref(c), None, 4, FAKE, 0, None) == T.TQ_ERR_INVALID_ARG
    assert lib.tq_dequantize(ctypes.byref(c), FAKE, 4, None, 0, None) == T.TQ_ERR_INVALID_ARG
    assert lib.tq_dequantize(ctypes.byref(c), FAKE, 4, FAKE + 8, 0, None) == T.TQ_ERR_INVALID_ARG
    assert lib.tq_dequantize(ctypes.byref(fake_cache(head_dim=384)), FAKE, 4, FAKE, 0, None) == T.TQ_ERR_UNSUPPORTED
    assert lib.tq_dequantize(ctypes.byref(c), FAKE, 0, FAKE, 0, None) == T.TQ_OK
    assert lib.tq_dequantize(None, FAKE, 4, FAKE, 0, None) == T.TQ_ERR_INVALID_ARG


def _fit_inputs(kind, bits, seed):
    rng = np.random.default_rng(seed)
    if kind == "gauss":
        x = rng.standard_normal((96, 4, 128))
    elif kind == "laplace":
        x = rng.laplace(size=(96, 4, 128)) * np.where(rng.random((96, 4, 128)) < 0.01, 30.0, 1.0)
    else:  # channel scales, fixed across tokens (the K recipe of the 8B-shaped workload)
        x = rng.standard_normal((96, 4, 128)) * np.exp(rng.standard_normal((1, 4, 128)))
    x[3, 1] = 0.0   # a zero vector (skipped)
    sw = rng.integers(0, 2 ** 32, size=(4, 4), dtype=np.uint64).astype(np.uint32)
    return x.astype(np.float16), sw


@pytest.mark.parametrize("kind", ["gauss", "laplace", "channels"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fit_codebook_matches_oracle(bits, kind):
    """Library fit (host) = oracle fit; a stored centre may differ by one float16 ulp
    only where the unrounded centre sits at a rounding midpoint."""
    x, sw = _fit_inputs(kind, bits, 100 + bits)
    cb = T.tq_fit_codebook(bits, x, sw)
    ref, c64, _ = O.fit_codebook(bits, x, sw)
    got = cb.centroid_array.astype(np.float64)
    diff = got != ref.centroids
    if diff.any():
        ulp = np.spacing(np.abs(ref.centroids).astype(np.float16)).astype(np.float64)
        frac = np.abs(c64 - ref.centroids) / ulp
        assert np.all(np.abs(frac[diff] - 0.5) < 1e-6)
    else:
        assert np.array_equal(cb.boundary_array.astype(np.float64), ref.boundaries)
    assert cb.n_levels == 1 << bits and cb.bits == bits
    assert math.isclose(cb.sigma, 1.0 / math.sqrt(128), rel_tol=1e-7)
    assert math.isclose(cb.mse, ref.mse, rel_tol=1e-6)


def test_fit_codebook_rejects_bad_arguments():
    lib = T.load_library()
    cb = T.TQCodebook()
    x = np.ones((4, 128), np.float16)
    sw = np.zeros((1, 4), np.uint32)
    ok = lambda bits, n, h, it, v=x, s=sw, out=ctypes.byref(cb): lib.tq_fit_codebook(
        bits, v.ctypes.data if v is not None else None, n, h, s.ctypes.data if s is not None else None, it, out)
    assert ok(3, 4, 1, 10) == T.TQ_OK
    assert ok(0, 4, 1, 10) == T.TQ_ERR_UNSUPPORTED
    assert ok(5, 4, 1, 10) == T.TQ_ERR_UNSUPPORTED
    assert ok(3, 0, 1, 10) == T.TQ_ERR_INVALID_ARG
    assert ok(3, 4, 0, 10) == T.TQ_ERR_INVALID_ARG
    assert ok(3, 4, 1, 0) == T.TQ_ERR_INVALID_ARG
    assert ok(3, 4, 1, 10, v=None) == T.TQ_ERR_INVALID_ARG
    assert ok(3, 4, 1, 10, s=None) == T.TQ_ERR_INVALID_ARG
    assert ok(3, 4, 1, 10, out=None) == T.TQ_ERR_INVALID_ARG
    z = np.zeros((4, 128), np.float16)
    assert ok(3, 4, 1, 10, v=z) == T.TQ_ERR_INVALID_ARG     # no nonzero vector


def test_float16_side_validation():
    """A float16 side needs no norms, signs or codebook; only K may be float16 in
    decode, and only with the matrix-core pass."""
    k16 = fake_cache(bits=T.BITS_FP16)
    k16.norms, k16.signs = None, None
    st, need = decode_call(k=k16)
    assert st == T.TQ_OK and need > 0
    assert decode_call(k=k16, tau=1e-3)[0] == T.TQ_OK
    assert decode_call(v=fake_cache(bits=T.BITS_FP16))[0] == T.TQ_ERR_UNSUPPORTED
    assert decode_call(k=fake_cache(bits=8))[0] == T.TQ_ERR_UNSUPPORTED
    assert decode_call(k=k16, options=VALU)[0] == T.TQ_ERR_UNSUPPORTED
    # a compressed side still needs its norms, signs and codebook
    k4 = fake_cache()
    k4.norms = None
    assert decode_call(k=k4)[0] == T.TQ_ERR_INVALID_ARG
    # quantize / dequantize accept a float16 side with no norms or signs
    lib = T.load_library()
    assert lib.tq_quantize_kv(ctypes.byref(k16), FAKE, None, None, 2 * 128, 0, None, None) == T.TQ_OK
    assert lib.tq_dequantize(ctypes.byref(k16), FAKE, 0, FAKE, 0, None) == T.TQ_OK


# ------------------------------------------------------------------ kept V channels

def test_select_outlier_channels_matches_oracle():
    """tq_select_outlier_channels (host) against the oracle's selection: planted
    channels, non-finite vectors skipped, k from 1 to 16, several heads."""
    rng = np.random.default_rng(77)
    x = rng.standard_normal((300, 5, 128)) * rng.lognormal(0, 0.5, (1, 5, 128))
    x[:, 2, [3, 70, 71]] *= 25
    x = x.astype(np.float16)
    x[7, 1, 9] = np.float16(np.inf)
    x[8, 4, 100] = np.float16(np.nan)
    for k in (1, 5, 16):
        got = T.tq_select_outlier_channels(x, k)
        want = O.select_outlier_channels(x, k)
        assert np.array_equal(got[:, :k], want) and not got[:, k:].any(), k
    assert set(T.tq_select_outlier_channels(x, 3)[2, :3]) == {3, 70, 71}


def test_select_outlier_channels_rejects_bad_arguments():
    lib = T.load_library()
    v = np.zeros((4, 128), np.float16)
    out = np.zeros((4, 16), np.uint8)
    call = lambda vec, n, h, k, o: lib.tq_select_outlier_channels(vec, n, h, k, o)
    assert call(None, 4, 1, 2, out.ctypes.data) == T.TQ_ERR_INVALID_ARG
    assert call(v.ctypes.data, 4, 1, 2, None) == T.TQ_ERR_INVALID_ARG
    assert call(v.ctypes.data, 0, 1, 2, out.ctypes.data) == T.TQ_ERR_INVALID_ARG
    assert call(v.ctypes.data, 4, 0, 2, out.ctypes.data) == T.TQ_ERR_INVALID_ARG
    assert call(v.ctypes.data, 4, 1, 0, out.ctypes.data) == T.TQ_ERR_INVALID_ARG
    assert call(v.ctypes.data, 4, 1, 17, out.ctypes.data) == T.TQ_ERR_INVALID_ARG
    assert call(v.ctypes.data, 4, 2, 16, out.ctypes.data) == T.TQ_OK


def _kept(c, k=4, channels=FAKE + 0x300000, values=FAKE + 0x400000):
    c.n_outliers, c.outlier_channels, c.outliers = k, channels, values
    return c


def test_kept_channel_validation():
    lib = T.load_library()
    q_call = lambda kk: lib.tq_quantize_kv(ctypes.byref(kk), FAKE, None, None, 256, 4, FAKE, None)
    assert q_call(_kept(fake_cache(), k=17)) == T.TQ_ERR_INVALID_ARG
    assert q_call(_kept(fake_cache(), k=-1)) == T.TQ_ERR_INVALID_ARG
    assert q_call(_kept(fake_cache(bits=T.BITS_FP16))) == T.TQ_ERR_UNSUPPORTED
    assert q_call(_kept(fake_cache(head_dim=256))) == T.TQ_ERR_UNSUPPORTED
    assert q_call(_kept(fake_cache(), channels=None)) == T.TQ_ERR_INVALID_ARG
    assert q_call(_kept(fake_cache(), channels=FAKE + 8)) == T.TQ_ERR_INVALID_ARG    # not 16-byte aligned
    assert q_call(_kept(fake_cache(), values=None)) == T.TQ_ERR_INVALID_ARG
    assert q_call(_kept(fake_cache(), values=FAKE + 2)) == T.TQ_ERR_INVALID_ARG      # not 8-byte aligned
    assert lib.tq_quantize_kv(ctypes.byref(_kept(fake_cache())), FAKE, None, None, 256, 0, FAKE, None) == T.TQ_OK
    # decode: kept channels on V only, on the matrix-core pass; the partials grow
    _, plain = decode_call()
    st, size = decode_call(v=_kept(fake_cache(bits=3)))
    assert st == T.TQ_OK and size > plain
    assert decode_call(k=_kept(fake_cache()))[0] == T.TQ_ERR_UNSUPPORTED
    assert decode_call(v=_kept(fake_cache(bits=3)), options=VALU)[0] == T.TQ_ERR_UNSUPPORTED


# ------------------------------------------------------------- fused append + decode

def test_append_decode_validation():
    """tq_append_decode_attention: the decode checks plus the new rows; only the
    matrix-core pass with 128-wide heads, compressed K and V without kept channels."""
    lib = T.load_library()

    def call(k=None, v=None, k_new=FAKE, v_new=FAKE, stride=256, ws=None, ws_bytes=0, options=None):
        k = fake_cache() if k is None else k
        v = fake_cache(bits=3) if v is None else v
        size = ctypes.c_size_t(ws_bytes)
        return lib.tq_append_decode_attention(ctypes.byref(k), k_new, ctypes.byref(v), v_new, stride, FAKE, 1, 1,
                                              2, FAKE, FAKE, 4, 0.0, 0.0, FAKE, ws, ctypes.byref(size), None,
                                              None if options is None else ctypes.byref(options.c()),
                                              None), size.value
    st, size = call()
    assert st == T.TQ_OK and size == decode_call()[1]          # workspace query, as decode
    assert call(k_new=None)[0] == T.TQ_ERR_INVALID_ARG
    assert call(v_new=FAKE + 8)[0] == T.TQ_ERR_INVALID_ARG      # not 16-byte aligned
    assert call(stride=255)[0] == T.TQ_ERR_INVALID_ARG          # < n_kv * 128
    assert call(stride=260)[0] == T.TQ_ERR_INVALID_ARG          # not a multiple of 8
    assert call(k=fake_cache(bits=T.BITS_FP16))[0] == T.TQ_ERR_UNSUPPORTED
    assert call(v=_kept(fake_cache(bits=3)))[0] == T.TQ_ERR_UNSUPPORTED
    assert call(k=fake_cache(head_dim=256), v=fake_cache(bits=3, head_dim=256), stride=512)[0] == \
        T.TQ_ERR_UNSUPPORTED
    assert call(options=VALU)[0] == T.TQ_ERR_UNSUPPORTED
    assert call(options=T.DecodeOptions(chunk=1024))[0] == T.TQ_OK


def test_decode_noalloc_host_checks():
    """tq_decode_attention_noalloc validates like tq_decode_attention and refuses,
    before touching a device, a call whose partials exceed its fixed array."""
    lib = T.load_library()
    k, v = fake_cache(), fake_cache(bits=3)
    call = lambda n_seqs=1, max_blocks=4, n_q_heads=2, kk=k: lib.tq_decode_attention_noalloc(
        ctypes.byref(kk), ctypes.byref(v), FAKE, n_seqs, 1, n_q_heads, FAKE, FAKE, max_blocks, 0.0, 0.0, FAKE, None)
    assert call(n_q_heads=3) == T.TQ_ERR_INVALID_ARG
    assert call(kk=fake_cache(head_dim=64)) == T.TQ_ERR_UNSUPPORTED
    assert call(n_seqs=0) == T.TQ_OK                                      # nothing to do
    n_seqs, max_blocks = 256, 4096
    _, need = decode_call(n_seqs=n_seqs, max_blocks=max_blocks)
    assert need > T.NOALLOC_SCRATCH_BYTES
    assert call(n_seqs=n_seqs, max_blocks=max_blocks) == T.TQ_ERR_WORKSPACE


def test_library_shares_torchs_hip_runtime():
    """Loading the library before anything imports torch still leaves one HIP
    runtime in the process (torch's), so torch's streams and memory are the
    library's own."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from compressed_kv_attention_tq_amd import tq as T\n"
            "T.load_library()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1", out.stdout
