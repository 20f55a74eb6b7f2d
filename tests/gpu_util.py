"""Helpers for the GPU parity tests: oracle caches, upload, comparisons.

Every expected value comes from the oracle; GPU results are only compared.
"""

import numpy as np

import oracle as O
from compressed_kv_attention_tq_amd import tq as T


def torch():
    import torch as _t
    return _t


def tq_codebook_from(ocb):
    """The library's codebook struct holding an oracle codebook's stored values."""
    cb = T.TQCodebook()
    cb.bits = ocb.bits
    cb.n_levels = 1 << ocb.bits
    for j, c in enumerate(ocb.centroids):
        cb.centroids[j] = float(c)
    for j, b in enumerate(ocb.boundaries):
        cb.boundaries[j] = float(b)
    cb.sigma = float(ocb.sigma)
    cb.mse = float(ocb.mse)
    return cb


def oracle_kept_channels(wl):
    """The V side's kept channels of a workload (oracle selection on its warm-up V), or None."""
    if not wl.v_kept:
        return None
    return O.select_outlier_channels(wl.warmup_v(), wl.v_kept)


def oracle_cache(wl, side, seqs=None, n_blocks=None, cb=None):
    """Quantize the workload's K (side 0) or V (side 1) with the oracle into pages
    (with codebook cb, by default the Gaussian one; V keeps the workload's kept channels)."""
    bits = wl.k_bits if side == 0 else wl.v_bits
    signs = wl.signs_k if side == 0 else wl.signs_v
    if bits != O.FP16:
        cb = O.build_codebook(bits) if cb is None else cb
    kept = oracle_kept_channels(wl) if side == 1 else None
    c = O.new_cache(bits, wl.n_kv_heads, wl.block_size, n_blocks or wl.n_blocks, signs, cb, head_dim=wl.head_dim,
                    outlier_channels=kept)
    for b in (range(wl.n_seqs) if seqs is None else seqs):
        if int(wl.seq_lens[b]) == 0:
            continue
        k, v = wl.kv_source(b)
        O.cache_write(c, k if side == 0 else v, wl.slots(b))
    return c


def gpu_cache_from(oc, device="cuda"):
    """A device cache holding exactly the oracle cache's codes, norms and codebook."""
    t = torch()
    g = T.Cache.allocate(oc.bits, oc.n_kv_heads, oc.block_size, oc.n_blocks, oc.signs, device,
                         cb=None if oc.bits == O.FP16 else tq_codebook_from(oc.cb), head_dim=oc.head_dim,
                         outlier_channels=oc.outlier_channels if oc.n_outliers else None)
    g.codes.copy_(t.from_numpy(oc.codes))
    g.norms.copy_(t.from_numpy(oc.norms))
    if oc.n_outliers:
        g.outliers.copy_(t.from_numpy(oc.outliers))
    return g


def upload_blocks(oc, g, blocks):
    """Overwrite the given pages of a device cache with the oracle's pages."""
    t = torch()
    idx = t.as_tensor(np.asarray(blocks, np.int64), device=g.codes.device)
    g.codes.index_copy_(0, idx, t.from_numpy(oc.codes[blocks]).to(g.codes.device))
    g.norms.index_copy_(0, idx, t.from_numpy(oc.norms[blocks]).to(g.norms.device))
    if oc.n_outliers:
        g.outliers.index_copy_(0, idx, t.from_numpy(oc.outliers[blocks]).to(g.outliers.device))


def oracle_cache_from_gpu(g, like):
    """An oracle cache holding what a device cache holds (codes, norms, kept values),
    with the signs, codebook and kept-channel list of the oracle cache `like`: the
    oracle's attention over it checks the attention arithmetic alone, whatever codes
    the GPU wrote."""
    c = O.new_cache(like.bits, like.n_kv_heads, like.block_size, like.n_blocks, like.signs, like.cb,
                    head_dim=like.head_dim,
                    outlier_channels=like.outlier_channels if like.n_outliers else None)
    c.codes[...] = g.codes.cpu().numpy()
    c.norms[...] = g.norms.cpu().numpy()
    if like.n_outliers:
        c.outliers[...] = g.outliers.cpu().numpy()
    return c


ELEM_TOL = 1e-3


def assert_attention_close(got, want, slack=None, what=""):
    """Attention outputs [..., d] against the oracle's, row by row and element by element.

    Per row: ||got - want|| <= 1e-3 ||want|| (+ slack).  Per element:
    |got_i - want_i| <= 1e-3 max(|want_i|, ||want|| / sqrt(d)) (+ slack_i).  A row
    whose oracle output is zero must be zero within 1e-6 (+ slack).  slack: None, or
    (row slack [...], element slack [..., d]) for gate decisions within rounding of
    tau.  Returns the worst per-row relative error and the worst element error
    relative to its bound."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = want.shape[-1]
    rs = np.zeros(want.shape[:-1]) if slack is None else np.asarray(slack[0], np.float64)
    es = np.zeros(want.shape) if slack is None else np.asarray(slack[1], np.float64)
    den = np.linalg.norm(want, axis=-1)
    err = np.linalg.norm(got - want, axis=-1)
    zero = den == 0
    bad = zero & (err > 1e-6 + rs)
    assert not bad.any(), f"{what}: {int(bad.sum())} rows should be zero (worst |got| {float(err[bad].max()):.3e})"
    bad = ~zero & (err > ELEM_TOL * den + rs)
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows beyond 1e-3 relative L2 "
                           f"(worst {float((err / np.where(zero, 1.0, den))[bad].max()):.3e})")
    bound = ELEM_TOL * np.maximum(np.abs(want), (den / np.sqrt(d))[..., None])
    eerr = np.abs(got - want)
    ebad = ~zero[..., None] & (eerr > bound + es)
    assert not ebad.any(), (f"{what}: {int(ebad.sum())} elements beyond 1e-3 max(|want_i|, ||want||/sqrt(d)) "
                            f"(worst ratio {float((eerr / np.maximum(bound, 1e-300))[ebad].max()):.3e})")
    rel = np.where(zero, 0.0, err / np.where(zero, 1.0, den))
    eratio = np.where(zero[..., None], 0.0, eerr / np.maximum(bound, 1e-300))
    return float(rel.max()) if rel.size else 0.0, float(eratio.max()) if eratio.size else 0.0


def row_rel_err(got, want):
    """Per-row ||got - want|| / ||want|| over the last axis (rows with ||want|| = 0 use 1)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.linalg.norm(got - want, axis=-1)
    den = np.linalg.norm(want, axis=-1)
    return num / np.where(den > 0, den, 1.0)


def check_codes(gpu_packed, gpu_norms, x16, signs_words, bits, eps=1e-6, cb=None):
    """Compare GPU-written packed codes / norms of rows x16 [n, 128] against the oracle
    (codebook cb, by default the Gaussian one).

    Returns the number of elements excluded as within eps of a decision boundary.
    Codes must match bit-exactly elsewhere; norms within 1e-6 relative.
    """
    cb = O.build_codebook(bits) if cb is None else cb
    s = O.sign_vector(signs_words)
    n, codes, y = O.quantize_vectors(x16, s, cb)
    got = O.unpack_codes(gpu_packed, bits)
    near = O.near_boundary_mask(y, cb.boundaries, eps)
    bad = (got != codes) & ~near
    assert not bad.any(), f"{int(bad.sum())} code mismatches away from boundaries"
    nf = n.astype(np.float64)
    gn = np.asarray(gpu_norms, np.float64)
    assert np.all(np.abs(gn - nf) <= 1e-6 * np.maximum(nf, 1e-30)), "norm mismatch"
    return int(near.sum())
