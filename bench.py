"""Benchmark of the compressed-KV hot path on one MI355X.

A step is one pass of the whole hot path over one batch: quantize-on-append of
the new tokens' K and V into the paged compressed cache and decode attention of
the new query tokens over the whole cache, in one call
(tq_append_decode_attention, the append fused into the decode pass) where that
is supported, else tq_quantize_kv then tq_decode_attention.  The default workload is the Llama-3-8B-shaped decode:
1 sequence of 32768 tokens, 32 query / 8 KV heads, d = 128, K 4-bit, V 3-bit.

The cache is replicated R times (R x 31.5 MB > the 256 MB last-level cache)
and step i works on replica i mod R, so every step streams its cache from HBM.
`value` = algorithmic bytes of a step / time of a step (inputs resident in HBM).
The second half of the metric, quantize throughput, is measured on the prefill
workload (32 layers x 8192 tokens x 8 KV heads, K 3-bit, V 2-bit): one call per
layer, the 32 calls replayed from a HIP graph (and, reported beside it, launched
back to back from the host).

python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload llama8b]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from compressed_kv_attention_tq_amd import tq as T  # noqa: E402
from compressed_kv_attention_tq_amd import workloads as W  # noqa: E402

METRIC = "compressed-KV decode attention HBM GB/s (% of peak) + quantize Mtok/s"
HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20
KERNEL_SOURCES = ["tq_decode.hip", "tq_decode_mfma.hip", "tq_decode_common.h", "tq_device.h", "tq_quant.hip",
                  "tq_internal.h", "tq_api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cache_bytes_per_token_head(bits):
    return 256 if bits == 16 else 16 * bits + 4   # a float16 side: the row, no norm


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "compressed_kv_attention_tq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_key):
    """HBM bytes per launch from a committed PMC record of the same kernel sources, else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    r = rec.get(kernel_key)
    if not r or r.get("source_hash") != source_hash():
        return None
    return r.get("bytes_per_launch")


class HipEvents:
    """Raw hipEvent_t pairs (the library records them on the launch stream itself)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0 and self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def handles(self, i):
        return self.pairs[i]

    def times_ms(self):
        """Elapsed time of every pair (ms); the events are destroyed."""
        out = []
        for a, b in self.pairs:
            ms = self.ct.c_float()
            assert self.hip.hipEventSynchronize(b) == 0
            assert self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) == 0
            out.append(ms.value)
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        return np.array(out)


def decode_workload(name):
    return {"llama8b": W.llama8b, "llama8b_k16": W.llama8b_k16, "longctx": W.longctx, "ragged": W.ragged,
            "tiny": W.tiny, "llama8b_d256": lambda: W.llama8b_wide(256),
            "llama8b_d512": lambda: W.llama8b_wide(512), "llama8b_vout": W.llama8b_vout}[name]()


def gen_kv_device(wl, b, torch, gen):
    """K/V of sequence b: the workload's own seeded numpy recipe, except the ragged
    workload (2.2 M tokens), whose N(0,1) K/V come from a seeded device generator."""
    if wl.kind == "normal":
        n = int(wl.seq_lens[b])
        k = torch.randn((n, wl.n_kv_heads, wl.head_dim), generator=gen, device="cuda").half()
        v = torch.randn((n, wl.n_kv_heads, wl.head_dim), generator=gen, device="cuda").half()
        return k, v
    k, v = wl.kv_source(b)
    return torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()


def run_decode(args, torch):
    wl = decode_workload(args.workload)
    kb, vb, hd, hb = wl.k_bits, wl.v_bits, wl.head_dim, wl.blocks_per_head
    kept_b = 2 * wl.v_kept   # kept V channels: float16 each
    per_tok = hb * (cache_bytes_per_token_head(kb) + cache_bytes_per_token_head(vb)) + kept_b   # one token-head
    cache_bytes = wl.total_tokens * wl.n_kv_heads * per_tok
    reps = args.replicas or min(64, max(1, math.ceil(1.5 * LLC_BYTES / cache_bytes)))
    log(f"[bench] workload {wl.name}: {wl.n_seqs} seqs, {wl.total_tokens} tokens, cache {cache_bytes / 1e6:.1f} MB, "
        f"{reps} replicas")

    nb = wl.n_blocks
    kc = T.Cache.allocate(kb, wl.n_kv_heads, wl.block_size, nb * reps, wl.signs_k, head_dim=hd)
    kept_idx = None
    if wl.v_kept:   # the V side's kept channels, selected on warm-up V by the library
        kept_idx = T.tq_select_outlier_channels(wl.warmup_v(), wl.v_kept)[:, : wl.v_kept]
    vc = T.Cache.allocate(vb, wl.n_kv_heads, wl.block_size, nb * reps, wl.signs_v, head_dim=hd,
                          outlier_channels=kept_idx)
    gen = torch.Generator(device="cuda").manual_seed(0)
    tables = []
    for r in range(reps):
        t = wl.block_table.copy()
        t[t >= 0] += r * nb
        tables.append(torch.from_numpy(t).cuda())
    for b in range(wl.n_seqs):
        if int(wl.seq_lens[b]) == 0:
            continue
        k, v = gen_kv_device(wl, b, torch, gen)
        for r in range(reps):
            slots = torch.from_numpy(wl.slots(b) + r * nb * wl.block_size).cuda()
            T.tq_quantize_kv(kc, k, vc, v, slots)
        del k, v
    torch.cuda.synchronize()
    log("[bench] caches filled")

    # the new tokens of each step: the last n_qtok positions of every sequence
    q = torch.from_numpy(wl.queries()).cuda()
    n_new = wl.n_seqs * wl.n_qtok
    k_new = torch.randn((n_new, wl.n_kv_heads, hd), generator=gen, device="cuda").half()
    v_new = torch.randn((n_new, wl.n_kv_heads, hd), generator=gen, device="cuda").half()
    new_slots = []
    for r in range(reps):
        s = []
        for b in range(wl.n_seqs):
            sl = wl.slots(b) + r * nb * wl.block_size
            s.extend(sl[-wl.n_qtok:].tolist() if len(sl) >= wl.n_qtok else [-1] * wl.n_qtok)
        new_slots.append(torch.tensor(s, dtype=torch.int64, device="cuda"))
    lens = torch.from_numpy(wl.seq_lens).cuda()
    out = torch.empty((wl.n_seqs, wl.n_qtok, wl.n_q_heads, hd), dtype=torch.float32, device="cuda")
    ws_bytes = T.decode_workspace_bytes(kc, vc, wl.n_seqs, wl.n_qtok, wl.n_q_heads, wl.block_table.shape[1],
                                        wl.tau)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    # the append fused into the pass (tq_append_decode_attention) where it is supported
    fused = not args.separate_append and kb != 16 and wl.head_dim == 128 and not wl.v_kept and \
        os.environ.get("TQ_DECODE_KERNEL", "mfma") != "valu"

    def step(i, events=None):
        r = i % reps
        if fused:
            T.tq_append_decode_attention(kc, k_new, vc, v_new, q, lens, tables[r], 0.0, wl.tau, out=out,
                                         workspace=ws, events=events)
        else:
            T.tq_quantize_kv(kc, k_new, vc, v_new, new_slots[r])
            T.tq_decode_attention(kc, vc, q, lens, tables[r], 0.0, wl.tau, out=out, workspace=ws, events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # eager steps; the library launches the dominant kernel with start / stop events
    # (hipExtLaunchKernelGGL), which time that kernel's execution
    evs = HipEvents(args.steps)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(args.warmup + i, events=evs.handles(i))
    t1.record()
    torch.cuda.synchronize()
    ms_step_eager = t0.elapsed_time(t1) / args.steps
    pass_times = evs.times_ms()
    pass_ms = float(np.mean(pass_times))
    log(f"[bench] pass kernel by events over {len(pass_times)} launches: mean {pass_ms * 1e3:.1f} us, "
        f"p10 / p50 / p90 {np.percentile(pass_times, 10) * 1e3:.1f} / {np.median(pass_times) * 1e3:.1f} / "
        f"{np.percentile(pass_times, 90) * 1e3:.1f} us")
    # the same steps replayed from a HIP graph (one graph = one step on every replica)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for r in range(reps):
            step(r)
    for _ in range(max(1, args.warmup // reps)):
        graph.replay()
    torch.cuda.synchronize()
    n_replay = max(1, -(-args.steps // reps))
    t0.record()
    for _ in range(n_replay):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / (n_replay * reps)

    # algorithmic bytes
    if wl.tau > 0:
        kept = 64 * wl.n_seqs * wl.n_kv_heads          # planted positions kept per (seq, KV head)
        cache_step = hb * (wl.total_tokens * wl.n_kv_heads * cache_bytes_per_token_head(kb) +
                           kept * cache_bytes_per_token_head(vb)) + kept * kept_b
        pass_bytes = hb * wl.total_tokens * wl.n_kv_heads * cache_bytes_per_token_head(kb)
    else:
        cache_step = cache_bytes
        pass_bytes = cache_bytes
    qo = wl.n_seqs * wl.n_qtok * wl.n_q_heads * hd * (2 + 4)
    meta = wl.n_seqs * 4 + wl.block_table.size * 4
    append = n_new * wl.n_kv_heads * (2 * 2 * hd + per_tok) + n_new * 8
    step_bytes = cache_step + qo + meta + append
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = pass_bytes / (pass_ms * 1e-3) / 1e9
    log(f"[bench] {ms_step * 1e3:.1f} us/step (graph), {ms_step_eager * 1e3:.1f} us/step (eager), "
        f"pass kernel {pass_ms * 1e3:.1f} us, "
        f"step {value:.0f} GB/s, pass {achieved:.0f} GB/s")
    mfma = os.environ.get("TQ_DECODE_KERNEL", "mfma") != "valu"
    kernel = "tq_decode_mfma_kernel" if mfma else "tq_decode_pass_kernel"
    kernel_key = f"{kernel}:{wl.name}"
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": pmc_traffic(kernel_key),
            "kernel": kernel + (" (scoring pass)" if wl.tau > 0 else ""), "bytes_per_launch": pass_bytes,
            "avg_launch_us": round(pass_ms * 1e3, 2),
            "median_launch_us": round(float(np.median(pass_times)) * 1e3, 2),
            "p10_launch_us": round(float(np.percentile(pass_times, 10)) * 1e3, 2),
            "p90_launch_us": round(float(np.percentile(pass_times, 90)) * 1e3, 2)}
    cfg = {"workload": f"{wl.name}: {wl.n_seqs} seq x {int(wl.seq_lens.max())} tokens, "
                       f"{wl.n_q_heads} q / {wl.n_kv_heads} KV heads, d={hd}, K{kb}/V{vb}"
                       f"{f' ({wl.v_kept} V channels kept in float16)' if wl.v_kept else ''}, "
                       f"{wl.n_qtok} query token(s), tau={wl.tau}, page {wl.block_size}",
           "global_batch": wl.n_seqs, "seq_len": int(wl.seq_lens.max()), "replicas": reps,
           "launch": "HIP graph replay", "ms_per_step_eager": round(ms_step_eager, 5),
           "append": ("fused into the pass (tq_append_decode_attention)" if fused
                      else "tq_quantize_kv, then tq_decode_attention"),
           "decode_kernel": ("matrix-core pass (fp16 MFMA, hi/lo-split fp32 operands, fp32 accumulate)"
                             if mfma else "vector-ALU pass (fp32)"),
           "parallelism": "single GPU"}
    return wl, value, ms_step, roof, cfg, step_bytes


def run_quantize(args, torch):
    """Prefill quantize: 32 layers x 8192 tokens x 8 KV heads, K3/V2, one call per layer."""
    wl = W.prefill()
    gen = torch.Generator(device="cuda").manual_seed(1)
    n = wl.n_tokens
    srcs, caches = [], []
    for layer in range(wl.n_layers):
        xs = []
        for _ in range(2):       # Laplace(0,1) = sign * Exp(1); 1% of entries x30
            e = torch.empty((n, wl.n_kv_heads, 128), device="cuda").exponential_(generator=gen)
            sgn = torch.randint(0, 2, e.shape, device="cuda", generator=gen) * 2 - 1
            big = torch.rand(e.shape, device="cuda", generator=gen) < 0.01
            xs.append((e * sgn * torch.where(big, 30.0, 1.0)).half())
        srcs.append(xs)
        sk, sv = wl.signs(layer)
        caches.append((T.Cache.allocate(wl.k_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, sk),
                       T.Cache.allocate(wl.v_bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, sv)))
    slots = torch.arange(n, dtype=torch.int64, device="cuda")

    def one_pass(events=None):
        for layer in range(wl.n_layers):
            if events is not None:
                events[layer][0].record()
            T.tq_quantize_kv(caches[layer][0], srcs[layer][0], caches[layer][1], srcs[layer][1], slots)
            if events is not None:
                events[layer][1].record()

    for _ in range(2):
        one_pass()
    torch.cuda.synchronize()
    reps = max(1, args.quantize_reps)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # 32 calls back to back, launched from the host
    t0.record()
    for r in range(reps):
        one_pass()
    t1.record()
    torch.cuda.synchronize()
    pass_ms_eager = t0.elapsed_time(t1) / reps
    # the kernel alone: events around every call (one more pass)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(wl.n_layers)]
    one_pass(evs)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    # the 32 calls replayed from a HIP graph
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for r in range(reps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    pass_ms = t0.elapsed_time(t1) / reps
    vec_per_call = 2 * n * wl.n_kv_heads
    bytes_per_call = n * wl.n_kv_heads * (2 * 256 + cache_bytes_per_token_head(wl.k_bits)
                                          + cache_bytes_per_token_head(wl.v_bits)) + n * 8
    mtok = n * wl.n_layers / (pass_ms * 1e-3) / 1e6
    # per launch: the graph replays the 32 kernels back to back (no host gap),
    # so its time / 32 is the kernel's own time per call
    launch_ms = pass_ms / wl.n_layers
    achieved = bytes_per_call / (launch_ms * 1e-3) / 1e9
    log(f"[bench] quantize: {pass_ms * 1e3:.1f} us / 32 layers (graph), {pass_ms_eager * 1e3:.1f} us (eager), "
        f"{kern_ms * 1e3:.2f} us/kernel, {mtok:.0f} M token-layers/s, {achieved:.0f} GB/s")
    return {"workload": "prefill: 32 layers x 8192 tokens x 8 KV heads, d=128, K3/V2 (Laplace, 1% x30)",
            "value": round(mtok, 1), "unit": "M token-layers/s", "launch": "HIP graph replay of the 32 calls",
            "ms_per_32_layers": round(pass_ms, 4), "ms_per_32_layers_eager": round(pass_ms_eager, 4),
            "value_eager": round(n * wl.n_layers / (pass_ms_eager * 1e-3) / 1e6, 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": pmc_traffic("tq_quantize_kernel:prefill"),
                         "kernel": "tq_quantize_kernel", "bytes_per_launch": bytes_per_call,
                         "vectors_per_launch": vec_per_call, "avg_launch_us": round(launch_ms * 1e3, 2),
                         "avg_launch_us_events": round(kern_ms * 1e3, 2)}}


def run_codebook_fit(torch):
    """Data-fitted codebooks (tq_fit_codebook) on the prefill data: fitted on the first
    1024 tokens of layer 0, measured on the other 7168 through the GPU quantize and
    dequantize kernels (relative MSE of the reconstruction), against the Gaussian
    codebooks; plus the host fit time and the quantize kernel time with each."""
    wl = W.prefill()
    sk, sv = wl.signs(0)
    k, v = wl.kv_source(0)
    warm, n = 1024, wl.n_tokens
    res = {"warmup_tokens": warm, "held_out_tokens": n - warm, "fit_ms": {}, "rel_mse": {}, "quantize_us": {}}
    for side, x, sg, bits in (("k", k, sk, wl.k_bits), ("v", v, sv, wl.v_bits)):
        t = time.perf_counter()
        fitted = T.tq_fit_codebook(bits, x[:warm], sg)
        res["fit_ms"][side] = round((time.perf_counter() - t) * 1e3, 1)
        xs = torch.from_numpy(x[warm:]).cuda()
        slots = torch.arange(n - warm, dtype=torch.int64, device="cuda")
        ref = xs.float()
        res["rel_mse"][side], res["quantize_us"][side] = {}, {}
        for name, cb in (("gaussian", None), ("fitted", fitted)):
            c = T.Cache.allocate(bits, wl.n_kv_heads, wl.block_size, -(-(n - warm) // wl.block_size), sg, cb=cb)
            T.tq_quantize_kv(c, xs, None, None, slots)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                T.tq_quantize_kv(c, xs, None, None, slots)
            e1.record()
            torch.cuda.synchronize()
            xh = T.tq_dequantize(c, slots)
            err = float(((xh - ref) ** 2).sum() / (ref ** 2).sum())
            res["rel_mse"][side][name] = round(err, 6)
            res["quantize_us"][side][name] = round(e0.elapsed_time(e1) * 100.0, 2)
    log(f"[bench] fitted codebooks: {res}")
    return res


def cpu_baseline(wl, budget_s=12.0):
    """The oracle (unchanged) on a bounded sample of the same decode step: for the KV
    heads of sequence 0 in turn (cycling), quantize-append the new token and decode its
    query rows over the whole context, until budget_s seconds are spent.  GB/s of
    algorithmic bytes processed."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    b = 0
    length = int(wl.seq_lens[b])
    k, v = wl.kv_source(b)
    slots = wl.slots(b)
    q = wl.queries()
    hb = wl.blocks_per_head
    per_tok = hb * (cache_bytes_per_token_head(wl.k_bits) + cache_bytes_per_token_head(wl.v_bits)) + 2 * wl.v_kept
    lens1, table1 = wl.seq_lens[:1], wl.block_table[:1]
    kept = O.select_outlier_channels(wl.warmup_v(), wl.v_kept) if wl.v_kept else None
    prepared = []
    for kv in range(wl.n_kv_heads):   # the context before the new tokens (not timed)
        kcache = O.new_cache(wl.k_bits, 1, wl.block_size, wl.n_blocks, wl.signs_k[kv * hb:(kv + 1) * hb],
                             None if wl.k_bits == 16 else O.build_codebook(wl.k_bits), head_dim=wl.head_dim)
        vcache = O.new_cache(wl.v_bits, 1, wl.block_size, wl.n_blocks, wl.signs_v[kv * hb:(kv + 1) * hb],
                             O.build_codebook(wl.v_bits), head_dim=wl.head_dim,
                             outlier_channels=None if kept is None else kept[kv:kv + 1])
        O.cache_write(kcache, k[:-wl.n_qtok, kv:kv + 1], slots[:-wl.n_qtok])
        O.cache_write(vcache, v[:-wl.n_qtok, kv:kv + 1], slots[:-wl.n_qtok])
        prepared.append((kcache, vcache, q[:1, :, kv * wl.group:(kv + 1) * wl.group]))
    done_bytes, spent, units = 0, 0.0, 0
    while spent < budget_s:
        kv = units % wl.n_kv_heads
        kcache, vcache, qh = prepared[kv]
        t0 = time.perf_counter()
        O.cache_write(kcache, k[-wl.n_qtok:, kv:kv + 1], slots[-wl.n_qtok:])
        O.cache_write(vcache, v[-wl.n_qtok:, kv:kv + 1], slots[-wl.n_qtok:])
        O.decode_attention(qh, kcache, vcache, lens1, table1, wl.n_qtok, 0.0, wl.tau)
        spent += time.perf_counter() - t0
        units += 1
        done_bytes += length * per_tok + wl.n_qtok * (2 * 2 * wl.head_dim + per_tok) + qh.size * 6
    gbs = done_bytes / spent / 1e9
    log(f"[bench] cpu oracle: {units} (KV head, step) units of seq 0 in {spent:.1f} s -> {gbs:.4f} GB/s, "
        f"{cores} threads")
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{wl.name}: sequence 0, {units} single-KV-head steps (append + decode of "
                      f"{wl.group * wl.n_qtok} query rows over {length} tokens each), {spent:.1f} s",
            "host": {"cpu_model": cpu_model, "nproc": os.cpu_count()}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "llama8b_k16", "llama8b_d256", "llama8b_d512", "llama8b_vout", "longctx",
                             "ragged", "tiny"])
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--separate-append", action="store_true",
                    help="append with tq_quantize_kv and decode with tq_decode_attention (two calls)")
    ap.add_argument("--quantize-reps", type=int, default=5)
    ap.add_argument("--no-quantize", action="store_true")
    ap.add_argument("--quantize-only", action="store_true", help="only the prefill quantize measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device copies of 256 MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the hot path does not shard across GPUs here)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    T.load_library()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 256 << 20, "copies": 5}), flush=True)
        return

    if args.quantize_only:
        print(json.dumps({"quantize": run_quantize(args, torch), "codebook_fit": run_codebook_fit(torch)}),
              flush=True)
        return
    wl, value, ms_step, roof, cfg, step_bytes = run_decode(args, torch)
    quant = None if args.no_quantize else run_quantize(args, torch)
    fitted = None if args.no_quantize else run_codebook_fit(torch)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": cfg, "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step_bytes": step_bytes,
        # per step: the query tokens answered and the KV token-heads scanned (each
        # sequence's KV heads over its whole context), each per second
        "query_tokens_per_s": round(wl.n_seqs * wl.n_qtok / (ms_step * 1e-3), 1),
        "kv_token_heads_per_s": round(wl.total_tokens * wl.n_kv_heads / (ms_step * 1e-3), 1),
        "roofline": roof, "cpu_baseline": cpu, "quantize": quant, "codebook_fit": fitted,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
