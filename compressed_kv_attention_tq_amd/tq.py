"""Python binding of libtq (include/tq.h): argument marshalling only.

Every step of the hot path runs in the HIP kernels of libtq.so.  PyTorch is
used for device memory and the current stream.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

Names follow the C ABI: tq_build_codebook, tq_quantize_kv,
tq_decode_attention, tq_dequantize.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

HEAD_DIM = 128   # elements per block; a head is 1, 2 or 4 blocks (head_dim 128, 256, 512)
BITS_FP16 = 16   # a cache side kept in float16 (TQ_BITS_FP16)
MAX_LEVELS = 16
MAX_ROWS_PER_KV_HEAD = 16
MAX_OUTLIERS = 16   # kept channels per head (TQ_MAX_OUTLIERS)

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_HIP = range(5)
EXPORTS = ("tq_status_string", "tq_build_codebook", "tq_fit_codebook", "tq_select_outlier_channels",
           "tq_quantize_kv", "tq_decode_attention", "tq_decode_attention_ex", "tq_append_decode_attention",
           "tq_decode_attention_noalloc", "tq_dequantize", "tq_stream_read")
NOALLOC_SCRATCH_BYTES = 32 << 20   # TQ_NOALLOC_SCRATCH_BYTES
DECODE_KERNEL_DEFAULT, DECODE_KERNEL_MFMA, DECODE_KERNEL_VALU = 0, 1, 2   # tq_decode_kernel


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)}")


class TQCodebook(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32),
        ("n_levels", ctypes.c_int32),
        ("centroids", ctypes.c_float * MAX_LEVELS),
        ("boundaries", ctypes.c_float * (MAX_LEVELS - 1)),
        ("sigma", ctypes.c_float),
        ("mse", ctypes.c_double),
    ]

    @property
    def centroid_array(self) -> np.ndarray:
        return np.array(self.centroids[: self.n_levels], dtype=np.float32)

    @property
    def boundary_array(self) -> np.ndarray:
        return np.array(self.boundaries[: self.n_levels - 1], dtype=np.float32)


class TQCache(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_blocks", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("norms", ctypes.c_void_p),
        ("signs", ctypes.c_void_p),
        ("cb", TQCodebook),
        ("n_outliers", ctypes.c_int32),
        ("outlier_channels", ctypes.c_void_p),
        ("outliers", ctypes.c_void_p),
    ]


class TQDecodeOptions(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("v_rows_read", ctypes.c_void_p),
    ]


@dataclass
class DecodeOptions:
    """tq_decode_options: the decode kernel (DECODE_KERNEL_*), the tokens per pass
    block (0 = the library's choice) and an optional device counter (a torch int64
    tensor of one element, zeroed by the caller) of the V rows the sparse gated
    pass reads."""
    kernel: int = DECODE_KERNEL_DEFAULT
    chunk: int = 0
    v_rows_read: object = None

    def c(self) -> TQDecodeOptions:
        o = TQDecodeOptions()
        o.kernel = self.kernel
        o.chunk = self.chunk
        o.v_rows_read = None if self.v_rows_read is None else _dev_ptr(self.v_rows_read, "v_rows_read").value
        return o


# Options used by the decode calls that are given none.  The library reads no
# process state; this is the binding's own default, which the tests replace to
# run every decode call of a test on another kernel variant.  None = defaults.
default_options: DecodeOptions | None = None


def _opts(options):
    o = default_options if options is None else options
    return None if o is None else ctypes.byref(o.c())


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libtq.so (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libtq.so not built at {path}; run __graft_entry__.build()")
    # torch first: its wheel carries its own HIP runtime (soname libamdhip64.so.7),
    # which libtq's dependency then resolves to.  Loaded the other way round, the
    # process would hold two HIP runtimes and torch's streams and memory would be
    # foreign to the library's launches.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_status_string.argtypes = [ctypes.c_int]
    lib.tq_build_codebook.restype = ctypes.c_int
    lib.tq_build_codebook.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.POINTER(TQCodebook)]
    lib.tq_fit_codebook.restype = ctypes.c_int
    lib.tq_fit_codebook.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(TQCodebook)]
    lib.tq_select_outlier_channels.restype = ctypes.c_int
    lib.tq_select_outlier_channels.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_void_p]
    lib.tq_quantize_kv.restype = ctypes.c_int
    lib.tq_quantize_kv.argtypes = [ctypes.POINTER(TQCache), ctypes.c_void_p, ctypes.POINTER(TQCache),
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.tq_decode_attention.restype = ctypes.c_int
    lib.tq_decode_attention.argtypes = [ctypes.POINTER(TQCache), ctypes.POINTER(TQCache), ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                        ctypes.c_void_p]
    lib.tq_decode_attention_ex.restype = ctypes.c_int
    lib.tq_decode_attention_ex.argtypes = lib.tq_decode_attention.argtypes + [ctypes.c_void_p, ctypes.c_void_p]
    lib.tq_append_decode_attention.restype = ctypes.c_int
    lib.tq_append_decode_attention.argtypes = [ctypes.POINTER(TQCache), ctypes.c_void_p, ctypes.POINTER(TQCache),
                                               ctypes.c_void_p, ctypes.c_int64] + \
        lib.tq_decode_attention.argtypes[2:] + [ctypes.c_void_p, ctypes.c_void_p]
    lib.tq_decode_attention_noalloc.restype = ctypes.c_int
    lib.tq_decode_attention_noalloc.argtypes = lib.tq_decode_attention.argtypes[:12] + [ctypes.c_void_p]
    lib.tq_stream_read.restype = ctypes.c_int
    lib.tq_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.tq_dequantize.restype = ctypes.c_int
    lib.tq_dequantize.argtypes = [ctypes.POINTER(TQCache), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_int32, ctypes.c_void_p]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().tq_status_string(status).decode()


def _check(status: int, what: str):
    if status != TQ_OK:
        raise TQError(status, what)


def tq_build_codebook(bits: int, sigma: float = 1.0 / math.sqrt(HEAD_DIM)) -> TQCodebook:
    cb = TQCodebook()
    _check(load_library().tq_build_codebook(bits, sigma, ctypes.byref(cb)), "tq_build_codebook")
    return cb


def tq_fit_codebook(bits: int, vectors, sign_words, max_iter: int = 200) -> TQCodebook:
    """Data-fitted codebook of one side from host float16 vectors [..., n_heads, 128]
    (the last-but-one axis is the head, whose signs are sign_words[head])."""
    v = np.ascontiguousarray(np.asarray(vectors, dtype=np.float16))
    if v.ndim < 2 or v.shape[-1] != HEAD_DIM:
        raise ValueError("vectors must be [..., 128] float16")
    sw = np.ascontiguousarray(np.asarray(sign_words, dtype=np.uint32).reshape(-1, 4))
    n_heads = sw.shape[0]
    if v.ndim >= 3 and v.shape[-2] != n_heads:
        raise ValueError("vectors [..., n_heads, 128] must match sign_words [n_heads, 4]")
    cb = TQCodebook()
    _check(load_library().tq_fit_codebook(bits, v.ctypes.data, v.size // HEAD_DIM, n_heads, sw.ctypes.data,
                                          max_iter, ctypes.byref(cb)), "tq_fit_codebook")
    return cb


def tq_select_outlier_channels(vectors, k: int) -> np.ndarray:
    """Kept channels per head from host float16 vectors [..., n_heads, 128]: uint8
    [n_heads, 16], the k channels of largest mean square (ascending), then zeros."""
    v = np.ascontiguousarray(np.asarray(vectors, dtype=np.float16))
    if v.ndim < 2 or v.shape[-1] != HEAD_DIM:
        raise ValueError("vectors must be [..., n_heads, 128] float16")
    n_heads = v.shape[-2]
    out = np.zeros((n_heads, 16), np.uint8)
    _check(load_library().tq_select_outlier_channels(v.ctypes.data, v.size // HEAD_DIM, n_heads, k,
                                                     out.ctypes.data), "tq_select_outlier_channels")
    return out


# ---------------------------------------------------------------------------- caches

def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, what: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class Cache:
    """One side (K or V) of a paged compressed cache, device memory owned by torch.
    A head of head_dim = 128 nb elements is nb sub-heads of 128 (block i of head j
    is sub-head nb j + i)."""
    bits: int
    n_kv_heads: int
    block_size: int
    n_blocks: int
    codes: object      # torch.uint8 [n_blocks, n_kv_heads * nb, block_size, 16*bits]
    norms: object      # torch.float32 [n_blocks, n_kv_heads * nb, block_size]
    signs: object      # torch.int32 (bit pattern of uint32) [n_kv_heads * nb, 4]
    cb: TQCodebook
    head_dim: int = HEAD_DIM
    n_outliers: int = 0
    outlier_channels: object = None   # torch.uint8 [n_kv_heads, 16] (kept channels, ascending)
    outliers: object = None           # torch.float16 [n_blocks, n_kv_heads, n_outliers, block_size]

    @classmethod
    def allocate(cls, bits, n_kv_heads, block_size, n_blocks, sign_words, device="cuda", cb=None,
                 head_dim=HEAD_DIM, outlier_channels=None):
        """outlier_channels: None, or [n_kv_heads, k] (k <= 16) channels per head kept in
        float16 (a 16-wide row as tq_select_outlier_channels returns needs k given via
        a [n_kv_heads, k] slice)."""
        torch = _torch()
        if head_dim not in (HEAD_DIM, 2 * HEAD_DIM, 4 * HEAD_DIM):
            raise ValueError("head_dim must be 128, 256 or 512")
        n_sub = n_kv_heads * (head_dim // HEAD_DIM)
        codes = torch.zeros((n_blocks, n_sub, block_size, 16 * bits), dtype=torch.uint8, device=device)
        norms = torch.zeros((n_blocks, n_sub, block_size), dtype=torch.float32, device=device)
        sw = np.ascontiguousarray(np.asarray(sign_words, dtype=np.uint32).reshape(n_sub, 4))
        signs = torch.from_numpy(sw.view(np.int32)).to(device)
        if bits == BITS_FP16:
            cb = TQCodebook()   # a float16 side has no codebook
        c = cls(bits, n_kv_heads, block_size, n_blocks, codes, norms, signs,
                tq_build_codebook(bits) if cb is None else cb, head_dim)
        if outlier_channels is not None:
            idx = np.asarray(outlier_channels, dtype=np.int64).reshape(n_kv_heads, -1)
            k = idx.shape[1]
            if not 1 <= k <= MAX_OUTLIERS:
                raise ValueError(f"1..{MAX_OUTLIERS} kept channels per head")
            rows = np.zeros((n_kv_heads, 16), np.uint8)
            rows[:, :k] = np.sort(idx, axis=1)
            c.n_outliers = k
            c.outlier_channels = torch.from_numpy(rows).to(device)
            c.outliers = torch.zeros((n_blocks, n_kv_heads, k, block_size), dtype=torch.float16, device=device)
        return c

    def desc(self) -> TQCache:
        d = TQCache()
        d.bits = self.bits
        d.n_kv_heads = self.n_kv_heads
        d.head_dim = self.head_dim
        d.block_size = self.block_size
        d.n_blocks = self.n_blocks
        d.codes = _dev_ptr(self.codes, "codes").value
        d.norms = _dev_ptr(self.norms, "norms").value
        d.signs = _dev_ptr(self.signs, "signs").value
        d.cb = self.cb
        d.n_outliers = self.n_outliers
        if self.n_outliers:
            d.outlier_channels = _dev_ptr(self.outlier_channels, "outlier_channels").value
            d.outliers = _dev_ptr(self.outliers, "outliers").value
        return d


def tq_quantize_kv(k_cache: Cache | None, k_src, v_cache: Cache | None, v_src, slot_mapping, stream=None):
    """Quantize-on-append: k_src / v_src float16 [n_tokens, n_kv_heads, head_dim] (token
    stride taken from the tensor), slot_mapping int64 [n_tokens] (negative = skip)."""
    torch = _torch()
    src = k_src if k_src is not None else v_src
    if src is None:
        return
    n_tokens = src.shape[0]
    stride = src.stride(0)
    for t, c, name in ((k_src, k_cache, "k_src"), (v_src, v_cache, "v_src")):
        if t is None:
            continue
        hd = c.head_dim if c is not None else HEAD_DIM
        if t.dtype != torch.float16 or not t.is_cuda or t.dim() != 3 or t.shape[2] != hd:
            raise ValueError(f"{name} must be a float16 device tensor [n_tokens, n_kv_heads, {hd}]")
        if t.stride(2) != 1 or t.stride(1) != hd or t.stride(0) != stride or t.shape[0] != n_tokens:
            raise ValueError(f"{name}: heads must be contiguous and both sides share one token stride")
    kd = ctypes.byref(k_cache.desc()) if k_cache is not None else None
    vd = ctypes.byref(v_cache.desc()) if v_cache is not None else None
    st = load_library().tq_quantize_kv(
        kd, ctypes.c_void_p(k_src.data_ptr()) if k_src is not None else None,
        vd, ctypes.c_void_p(v_src.data_ptr()) if v_src is not None else None,
        stride, n_tokens, _dev_ptr(slot_mapping, "slot_mapping", torch.int64), _stream_ptr(stream))
    _check(st, "tq_quantize_kv")


def decode_workspace_bytes(k_cache: Cache, v_cache: Cache, n_seqs, n_qtok, n_q_heads, max_blocks_per_seq,
                           tau=0.0, options: DecodeOptions | None = None) -> int:
    """The workspace size of a decode call with these shapes and options."""
    size = ctypes.c_size_t(0)
    st = load_library().tq_decode_attention_ex(ctypes.byref(k_cache.desc()), ctypes.byref(v_cache.desc()), None,
                                               n_seqs, n_qtok, n_q_heads, None, None, max_blocks_per_seq,
                                               0.0, float(tau), None, None, ctypes.byref(size), None,
                                               _opts(options), None)
    _check(st, "tq_decode_attention (workspace query)")
    return size.value


def tq_decode_attention(k_cache: Cache, v_cache: Cache, q, seq_lens, block_table, softmax_scale=0.0,
                        sparse_v_tau=0.0, out=None, workspace=None, stream=None, events=None,
                        options: DecodeOptions | None = None):
    """q float16 [n_seqs, n_qtok, n_q_heads, head_dim]; seq_lens int32 [n_seqs];
    block_table int32 [n_seqs, max_blocks].  Returns float32 out like q.
    events: optional pair of raw hipEvent_t handles (ctypes.c_void_p or int) recorded
    around the main pass kernel; options: DecodeOptions (tq_decode_attention_ex)."""
    torch = _torch()
    n_seqs, n_qtok, n_q_heads, hd = q.shape
    if hd != k_cache.head_dim:
        raise ValueError(f"q has head_dim {hd}, the cache {k_cache.head_dim}")
    max_blocks = block_table.shape[1]
    need = decode_workspace_bytes(k_cache, v_cache, n_seqs, n_qtok, n_q_heads, max_blocks, sparse_v_tau, options)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((n_seqs, n_qtok, n_q_heads, hd), dtype=torch.float32, device=q.device)
    size = ctypes.c_size_t(workspace.numel())
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * 2)(*[e.value if isinstance(e, ctypes.c_void_p) else e for e in events])
    st = load_library().tq_decode_attention_ex(
        ctypes.byref(k_cache.desc()), ctypes.byref(v_cache.desc()), _dev_ptr(q, "q", torch.float16),
        n_seqs, n_qtok, n_q_heads, _dev_ptr(seq_lens, "seq_lens", torch.int32),
        _dev_ptr(block_table, "block_table", torch.int32), max_blocks, float(softmax_scale),
        float(sparse_v_tau), _dev_ptr(out, "out", torch.float32), _dev_ptr(workspace, "workspace"),
        ctypes.byref(size), _stream_ptr(stream), _opts(options), ev)
    _check(st, "tq_decode_attention")
    return out


def tq_append_decode_attention(k_cache: Cache, k_new, v_cache: Cache, v_new, q, seq_lens, block_table,
                               softmax_scale=0.0, sparse_v_tau=0.0, out=None, workspace=None, stream=None,
                               events=None, options: DecodeOptions | None = None):
    """Quantize-on-append of the new tokens and decode attention in one call (the
    fused pass): k_new / v_new float16 [n_seqs * n_qtok, n_kv_heads, 128] (token
    stride from the tensor), token j of sequence b going to position
    seq_lens[b] - n_qtok + j; the rest as tq_decode_attention."""
    torch = _torch()
    n_seqs, n_qtok, n_q_heads, hd = q.shape
    if hd != k_cache.head_dim:
        raise ValueError(f"q has head_dim {hd}, the cache {k_cache.head_dim}")
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if t.dtype != torch.float16 or not t.is_cuda or t.dim() != 3 or t.shape[0] != n_seqs * n_qtok:
            raise ValueError(f"{name} must be a float16 device tensor [n_seqs * n_qtok, n_kv_heads, 128]")
        if t.stride(2) != 1 or t.stride(1) != HEAD_DIM or t.stride(0) != k_new.stride(0):
            raise ValueError(f"{name}: heads must be contiguous and both share one token stride")
    max_blocks = block_table.shape[1]
    need = decode_workspace_bytes(k_cache, v_cache, n_seqs, n_qtok, n_q_heads, max_blocks, sparse_v_tau, options)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((n_seqs, n_qtok, n_q_heads, hd), dtype=torch.float32, device=q.device)
    size = ctypes.c_size_t(workspace.numel())
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * 2)(*[e.value if isinstance(e, ctypes.c_void_p) else e for e in events])
    st = load_library().tq_append_decode_attention(
        ctypes.byref(k_cache.desc()), ctypes.c_void_p(k_new.data_ptr()), ctypes.byref(v_cache.desc()),
        ctypes.c_void_p(v_new.data_ptr()), k_new.stride(0), _dev_ptr(q, "q", torch.float16), n_seqs, n_qtok,
        n_q_heads, _dev_ptr(seq_lens, "seq_lens", torch.int32), _dev_ptr(block_table, "block_table", torch.int32),
        max_blocks, float(softmax_scale), float(sparse_v_tau), _dev_ptr(out, "out", torch.float32),
        _dev_ptr(workspace, "workspace"), ctypes.byref(size), _stream_ptr(stream), _opts(options), ev)
    _check(st, "tq_append_decode_attention")
    return out


def tq_decode_attention_noalloc(k_cache: Cache, v_cache: Cache, q, seq_lens, block_table, softmax_scale=0.0,
                                sparse_v_tau=0.0, out=None, stream=None):
    """tq_decode_attention with the library's fixed scratch array in place of a
    workspace (the C call allocates nothing; `out` is allocated here if not given)."""
    torch = _torch()
    n_seqs, n_qtok, n_q_heads, hd = q.shape
    if hd != k_cache.head_dim:
        raise ValueError(f"q has head_dim {hd}, the cache {k_cache.head_dim}")
    if out is None:
        out = torch.empty((n_seqs, n_qtok, n_q_heads, hd), dtype=torch.float32, device=q.device)
    st = load_library().tq_decode_attention_noalloc(
        ctypes.byref(k_cache.desc()), ctypes.byref(v_cache.desc()), _dev_ptr(q, "q", torch.float16),
        n_seqs, n_qtok, n_q_heads, _dev_ptr(seq_lens, "seq_lens", torch.int32),
        _dev_ptr(block_table, "block_table", torch.int32), block_table.shape[1], float(softmax_scale),
        float(sparse_v_tau), _dev_ptr(out, "out", torch.float32), _stream_ptr(stream))
    _check(st, "tq_decode_attention_noalloc")
    return out


def tq_dequantize(cache: Cache, slots, fp16=False, out=None, stream=None):
    """Dequantized rows [n_tokens, n_kv_heads, head_dim] of the given slots (int64)."""
    torch = _torch()
    n = slots.shape[0]
    if out is None:
        out = torch.empty((n, cache.n_kv_heads, cache.head_dim), dtype=torch.float16 if fp16 else torch.float32,
                          device=slots.device)
    st = load_library().tq_dequantize(ctypes.byref(cache.desc()), _dev_ptr(slots, "slots", torch.int64), n,
                                      _dev_ptr(out, "out"), 1 if fp16 else 0, _stream_ptr(stream))
    _check(st, "tq_dequantize")
    return out


def tq_stream_read(src, sink, stream=None):
    """Read every byte of the contiguous device tensor src once (the streaming
    ceiling kernel); sink: a device int32 tensor of one element."""
    torch = _torch()
    _check(load_library().tq_stream_read(_dev_ptr(src, "src"), src.numel() * src.element_size(),
                                         _dev_ptr(sink, "sink", torch.int32), _stream_ptr(stream)),
           "tq_stream_read")
