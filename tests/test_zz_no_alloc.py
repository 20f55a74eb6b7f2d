"""tq_decode_attention_noalloc (the decode call for callers that cannot allocate)
against tq_decode_attention, through the C ABI: two calls in a row, the second
with a smaller input, each equal to the workspace call's output bit for bit (the
same kernels and partial layout), and within the attention bar of the oracle."""

import numpy as np
import pytest

import oracle as O
from compressed_kv_attention_tq_amd import tq as T
from compressed_kv_attention_tq_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T.load_library()


def _case(wl, tau):
    import torch
    ok, ov = U.oracle_cache(wl, 0), U.oracle_cache(wl, 1)
    gk, gv = U.gpu_cache_from(ok), U.gpu_cache_from(ov)
    q = torch.from_numpy(wl.queries()).cuda()
    lens = torch.from_numpy(wl.seq_lens).cuda()
    table = torch.from_numpy(wl.block_table).cuda()
    # the no-allocation call first (nothing else has touched the scratch array yet
    # in a fresh process), then the workspace call
    got = T.tq_decode_attention_noalloc(gk, gv, q, lens, table, 0.0, tau).cpu().numpy()
    ref = T.tq_decode_attention(gk, gv, q, lens, table, 0.0, tau).cpu().numpy()
    assert np.array_equal(got, ref, equal_nan=True), float(np.max(np.abs(got - ref)))
    want = O.decode_attention(wl.queries(), ok, ov, wl.seq_lens, wl.block_table, wl.n_qtok, 0.0, tau)
    if tau == 0:
        U.assert_attention_close(got, want, what="noalloc")
    return got


@pytest.mark.parametrize("tau", [0.0, 1e-3])
def test_noalloc_equals_workspace_call_twice(tau):
    big = W.small_decode(seed=91, n_seqs=3, lens=[3000, 700, 1500], n_qtok=2, n_q_heads=8, n_kv_heads=2,
                         k_bits=4, v_bits=3, tau=tau, block_size=64)
    small = W.small_decode(seed=92, n_seqs=2, lens=[300, 65], n_qtok=1, n_q_heads=4, n_kv_heads=1,
                           k_bits=3, v_bits=2, tau=tau, block_size=32)
    _case(big, tau)
    _case(small, tau)


def test_noalloc_rejects_more_than_the_scratch():
    """A call whose partials exceed the array returns TQ_ERR_WORKSPACE and launches nothing."""
    import torch
    wl = W.small_decode(seed=93, n_seqs=1, lens=[10], n_qtok=4, n_q_heads=16, n_kv_heads=4, k_bits=4, v_bits=4)
    gk = T.Cache.allocate(4, 4, 256, 4, wl.signs_k)
    gv = T.Cache.allocate(4, 4, 256, 4, wl.signs_v)
    n_seqs, max_blocks = 64, 4096   # 64 x 4 x 1M-token tables: far more partials than 32 MiB
    q = torch.zeros((n_seqs, 4, 16, 128), dtype=torch.float16, device="cuda")
    lens = torch.zeros(n_seqs, dtype=torch.int32, device="cuda")
    table = torch.zeros((n_seqs, max_blocks), dtype=torch.int32, device="cuda")
    need = T.decode_workspace_bytes(gk, gv, n_seqs, 4, 16, max_blocks)
    assert need > T.NOALLOC_SCRATCH_BYTES
    with pytest.raises(T.TQError) as e:
        T.tq_decode_attention_noalloc(gk, gv, q, lens, table)
    assert e.value.status == T.TQ_ERR_WORKSPACE
