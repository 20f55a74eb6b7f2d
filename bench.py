"""Benchmark of the compressed-KV hot path on one MI355X.

A step is one pass of the whole hot path over one batch: quantize-on-append of
the new tokens' K and V into the paged compressed cache and decode attention of
the new query tokens over the whole cache, in one call
(tq_append_decode_attention: the append fused into the decode pass).

The headline is the largest single-GPU workload, the ragged batched verify
decode: 64 sequences of 4K-64K tokens, 32 query / 8 KV heads, d = 128, 4 query
tokens per sequence, K 4-bit / V 4-bit, 256-token pages in random physical
order (about 2.4 GB of compressed cache per step).  `value` = algorithmic bytes
of a step / time of a step, with the cache resident in HBM.

The same line carries sub-records, each with its own roofline and CPU baseline:
  llama8b   Llama-3-8B-shaped decode, 1 x 32768 tokens, 32 / 8 heads, K4 / V3
  longctx   4 x 131072 tokens, 40 / 4 heads, K3 / V2, sparse V at tau = 1e-4
  tiny      1 x 1024 tokens, 1 / 1 head, K4 / V3 (latency-bound, reported only)
  quantize  prefill: 32 layers x 8192 tokens x 8 KV heads, K3 / V2 (tq_quantize_kv)

Caches smaller than 1.5 x the 256 MB last-level cache are replicated and step i
works on replica i mod R, so every step streams its cache from HBM.  The
dominant kernel of each workload is timed by HIP events recorded around its own
launch on its own stream (tq_decode_attention_ex / tq_append_decode_attention
events), steps by a HIP graph replay.  A device copy of the same bytes gives the
practical streaming ceiling beside the 8 TB/s peak.

CPU baseline: the float64 oracle (oracle/), unchanged, on the host cores: one
process, then one process per core over independent units (a (sequence, KV
head) decode step, or a (layer, side) quantize); see cpu_baseline().

python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload all|ragged|llama8b|...]
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
# the sources each measured kernel is built from (its traffic record is tied to them)
KERNEL_SOURCES = {
    "tq_decode_mfma_kernel": ["tq_decode.hip", "tq_decode_mfma.hip", "tq_decode_common.h", "tq_device.h",
                              "tq_internal.h", "tq_api.cpp"],
    "tq_quantize_kernel": ["tq_quant.hip", "tq_device.h", "tq_internal.h", "tq_api.cpp"],
}
PMC_RECORD = os.path.join(ROOT, "profiles", "pmc_traffic.json")
DECODE_DTYPE = "fp16 hi/lo-split operands (fp32-level), fp32 accumulate"
DECODE_WORKLOADS = ["llama8b", "llama8b_k16", "llama8b_d256", "llama8b_d512", "llama8b_vout", "longctx", "ragged",
                    "tiny"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cache_bytes_per_token_head(bits):
    return 256 if bits == 16 else 16 * bits + 4   # a float16 side: the row, no norm


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "compressed_kv_attention_tq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 PMC record
    (profiles/pmc_traffic.json: FETCH_SIZE and WRITE_SIZE scaled by the copy
    calibration) of exactly these kernel sources, else None."""
    if not os.path.exists(PMC_RECORD):
        return None
    with open(PMC_RECORD) as f:
        rec = json.load(f)
    r = rec.get(kernel_key)
    if not r or r.get("source_hash") != source_hash(kernel_key.split(":")[0]):
        return None
    return r.get("bytes_per_launch")


# rocprofv3 FETCH_SIZE counts half of the bytes a plain device copy reads, WRITE_SIZE
# all it writes (profiles/copy_calibration_pmc.md)
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def record_traffic(kernel_key, fetch_csv, write_csv):
    """Write the HBM bytes per launch of one kernel into the traffic record, from two
    rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; counter_collection.csv, KiB
    per dispatch): the mean over that kernel's dispatches, scaled as above.  Of the
    instantiations of the kernel in the run (the scoring and the gated pass of a
    sparse decode are both the matrix-core kernel) the one that fetches the most is
    taken: the dominant kernel the bench's roofline is about."""
    import csv
    kernel = kernel_key.split(":")[0]

    def per_name(path, counter):
        tot = {}   # kernel name -> dispatch -> KiB
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                if row.get("Counter_Name") != counter or kernel not in name:
                    continue
                d = row.get("Dispatch_Id") or row.get("Correlation_Id")
                tot.setdefault(name, {})
                tot[name][d] = tot[name].get(d, 0.0) + float(row["Counter_Value"])
        if not tot:
            raise SystemExit(f"no {counter} rows for {kernel} in {path}")
        return {n: (sum(v.values()) / len(v), len(v)) for n, v in tot.items()}

    fetch = per_name(fetch_csv, "FETCH_SIZE")
    name = max(fetch, key=lambda n: fetch[n][0])
    write = per_name(write_csv, "WRITE_SIZE")
    if name not in write:
        raise SystemExit(f"{name} has no WRITE_SIZE rows in {write_csv}")
    (fetch_kib, nf), (write_kib, nw) = fetch[name], write[name]
    fetch_b = FETCH_SCALE * fetch_kib * 1024
    write_b = WRITE_SCALE * write_kib * 1024
    rec = {}
    if os.path.exists(PMC_RECORD):
        with open(PMC_RECORD) as f:
            rec = json.load(f)
    fetch_i, write_i = int(round(fetch_b)), int(round(write_b))
    rec[kernel_key] = {"bytes_per_launch": fetch_i + write_i, "fetch_bytes": fetch_i,
                       "write_bytes": write_i, "source_hash": source_hash(kernel),
                       "kernel_name": name[:160],
                       "dispatches": [nf, nw], "fetch_kib_per_dispatch": round(fetch_kib, 1),
                       "write_kib_per_dispatch": round(write_kib, 1)}
    with open(PMC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps({kernel_key: rec[kernel_key]}))


def host_info():
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": cpu_model, "nproc": os.cpu_count(), "usable_cpus": usable}


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


def describe(wl):
    return (f"{wl.name}: {wl.n_seqs} seq x {int(wl.seq_lens.max())} tokens (total {wl.total_tokens}), "
            f"{wl.n_q_heads} q / {wl.n_kv_heads} KV heads, d={wl.head_dim}, K{wl.k_bits}/V{wl.v_bits}"
            f"{f' ({wl.v_kept} V channels kept in float16)' if wl.v_kept else ''}, "
            f"{wl.n_qtok} query token(s), tau={wl.tau}, page {wl.block_size}")


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


def copy_ceiling(torch, nbytes):
    """Practical streaming rates for nbytes, one launch per buffer: the library's
    plain streaming read (tq_stream_read) and a device-to-device copy (read + write),
    each timed by events over buffers totalling > 1.5 x the last-level cache.
    Returns GB/s of the bytes each moves."""
    n = max(4, (nbytes // 16) * 4)
    reps = max(1, math.ceil(1.5 * LLC_BYTES / (4 * n)))
    srcs = [torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(reps)]
    dsts = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(reps)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rounds = max(3, 20 // reps)
    res = {}
    for name, fn, moved in (("read", lambda i: T.tq_stream_read(srcs[i], sink), 4 * n),
                            ("copy", lambda i: dsts[i].copy_(srcs[i]), 8 * n)):
        for i in range(reps):
            fn(i)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(rounds):
            for i in range(reps):
                fn(i)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / (rounds * reps) * 1e-3
        res[name] = round(moved / t / 1e9, 1)
    del srcs, dsts, sink
    torch.cuda.empty_cache()
    return res


def run_decode(args, torch, name):
    """One decode workload: fill the caches (GPU quantize), time the fused append +
    decode step (events on the pass kernel, graph replay for the step)."""
    wl = decode_workload(name)
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
    base_opts = T.DecodeOptions(chunk=args.chunk)
    ws_bytes = T.decode_workspace_bytes(kc, vc, wl.n_seqs, wl.n_qtok, wl.n_q_heads, wl.block_table.shape[1],
                                        wl.tau, options=base_opts)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    # the append fused into the pass (tq_append_decode_attention) where it is supported
    fused = not args.separate_append and kb != 16 and wl.head_dim == 128 and not wl.v_kept

    def step(i, events=None, options=None):
        r = i % reps
        options = options or base_opts
        if fused:
            T.tq_append_decode_attention(kc, k_new, vc, v_new, q, lens, tables[r], 0.0, wl.tau, out=out,
                                         workspace=ws, events=events, options=options)
        else:
            T.tq_quantize_kv(kc, k_new, vc, v_new, new_slots[r])
            T.tq_decode_attention(kc, vc, q, lens, tables[r], 0.0, wl.tau, out=out, workspace=ws, events=events,
                                  options=options)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # sparse V: the V rows the gated pass reads, counted on the device (one step)
    v_rows = None
    if wl.tau > 0:
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        step(0, options=T.DecodeOptions(chunk=args.chunk, v_rows_read=cnt))
        torch.cuda.synchronize()
        v_rows = int(cnt.item())
    # eager steps; the library launches the dominant kernel with start / stop events
    # (hipExtLaunchKernelGGL), which time that kernel's execution on its own stream
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
    del graph

    # algorithmic bytes
    if wl.tau > 0:
        cache_step = hb * wl.total_tokens * wl.n_kv_heads * cache_bytes_per_token_head(kb) + \
            v_rows * (cache_bytes_per_token_head(vb) + (kept_b if wl.v_kept else 0))
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
    del kc, vc, ws, tables
    torch.cuda.empty_cache()
    ceiling = copy_ceiling(torch, pass_bytes)
    log(f"[bench] {ms_step * 1e3:.1f} us/step (graph), {ms_step_eager * 1e3:.1f} us/step (eager), "
        f"pass kernel {pass_ms * 1e3:.1f} us, step {value:.0f} GB/s, pass {achieved:.0f} GB/s, "
        f"streaming ceiling {ceiling}")
    kernel = "tq_decode_mfma_kernel"
    best = ceiling["read"]
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": pmc_traffic(f"{kernel}:{wl.name}"),
            "traffic_source": "committed rocprofv3 PMC record of these kernel sources (profiles/pmc_traffic.json); "
                              "null when the sources changed since",
            "kernel": kernel + (" (scoring pass: every K code; V in the gated pass)" if wl.tau > 0 else ""),
            "bytes_per_launch": pass_bytes, "avg_launch_us": round(pass_ms * 1e3, 2),
            "median_launch_us": round(float(np.median(pass_times)) * 1e3, 2),
            "p10_launch_us": round(float(np.percentile(pass_times, 10)) * 1e3, 2),
            "p90_launch_us": round(float(np.percentile(pass_times, 90)) * 1e3, 2),
            "streaming_ceiling_gbs": ceiling, "frac_of_read_ceiling": round(achieved / best, 4)}
    rec = {"workload": describe(wl), "value": round(value, 2), "unit": "GB/s", "ms_per_step": round(ms_step, 5),
           "ms_per_step_eager": round(ms_step_eager, 5), "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
           "step_bytes": step_bytes, "replicas": reps, "launch": "HIP graph replay",
           "append": ("fused into the pass (tq_append_decode_attention)" if fused
                      else "tq_quantize_kv, then tq_decode_attention"),
           "decode_kernel": "matrix-core pass (fp16 MFMA, hi/lo-split fp32 operands, fp32 accumulate)",
           "dtype": DECODE_DTYPE,
           # per step: the query tokens answered and the KV token-heads scanned
           "query_tokens_per_s": round(wl.n_seqs * wl.n_qtok / (ms_step * 1e-3), 1),
           "kv_token_heads_per_s": round(wl.total_tokens * wl.n_kv_heads / (ms_step * 1e-3), 1),
           "roofline": roof}
    if v_rows is not None:
        rec["sparse_v"] = {"v_rows_read": v_rows, "per_seq_kv_head": round(v_rows / (wl.n_seqs * wl.n_kv_heads), 1),
                           "counted_by": "the gated pass (tq_decode_options.v_rows_read)"}
    return wl, rec


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
    # the kernel alone: events around every call on the launch stream (one more pass)
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
    del srcs, caches, graph
    torch.cuda.empty_cache()
    ceiling = copy_ceiling(torch, bytes_per_call)
    log(f"[bench] quantize: {pass_ms * 1e3:.1f} us / 32 layers (graph), {pass_ms_eager * 1e3:.1f} us (eager), "
        f"{kern_ms * 1e3:.2f} us/kernel by events, {mtok:.0f} M token-layers/s, {achieved:.0f} GB/s")
    return {"workload": "prefill: 32 layers x 8192 tokens x 8 KV heads, d=128, K3/V2 (Laplace, 1% x30)",
            "value": round(mtok, 1), "unit": "M token-layers/s", "launch": "HIP graph replay of the 32 calls",
            "dtype": "fp16 inputs, fp32 accumulate (transform on MFMA), codes u8",
            "ms_per_32_layers": round(pass_ms, 4), "ms_per_32_layers_eager": round(pass_ms_eager, 4),
            "value_eager": round(n * wl.n_layers / (pass_ms_eager * 1e-3) / 1e6, 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": pmc_traffic("tq_quantize_kernel:prefill"),
                         "traffic_source": "committed rocprofv3 PMC record of these kernel sources "
                                           "(profiles/pmc_traffic.json); null when the sources changed since",
                         "kernel": "tq_quantize_kernel", "bytes_per_launch": bytes_per_call,
                         "vectors_per_launch": vec_per_call, "avg_launch_us": round(launch_ms * 1e3, 2),
                         "avg_launch_us_events": round(kern_ms * 1e3, 2),
                         "streaming_ceiling_gbs": ceiling,
                         "frac_of_read_ceiling": round(achieved / ceiling["read"], 4)}}


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


# ------------------------------------------------------------------ CPU baseline
#
# The oracle, unchanged, on independent units of the same workloads.  A decode
# unit is one step of one (sequence, KV head): quantize-append of its n_qtok new
# K and V rows (oracle cache_write) and the oracle's attention of its G * n_qtok
# query rows over the whole context (decode_attention).  The context's codes and
# norms are seeded random bytes written before the clock starts (the oracle's
# work does not depend on the code values, and quantizing millions of context
# rows first would only add untimed set-up).  A quantize unit is one (layer, side)
# of the prefill: oracle cache_write of 8192 tokens x 8 KV heads.
# Each unit runs with one BLAS thread.  Single process: units one after another
# for a bounded time.  All cores: one process per usable core (at most 16), the
# units dealt round-robin; the time is the slowest process's own timed total.

def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:
        return None


def _cpu_decode_unit(job):
    """(seconds, algorithmic bytes) of one oracle decode step of one (sequence, KV head)."""
    import oracle as O
    name, b, kv = job
    wl = decode_workload(name)
    length = int(wl.seq_lens[b])
    bs, hb, g, n_qtok = wl.block_size, wl.blocks_per_head, wl.group, wl.n_qtok
    n_pages = -(-length // bs)
    rng = np.random.default_rng([7, b, kv])
    caches = []
    for bits, signs in ((wl.k_bits, wl.signs_k), (wl.v_bits, wl.signs_v)):
        c = O.new_cache(bits, 1, bs, n_pages, signs[kv * hb:(kv + 1) * hb],
                        None if bits == 16 else O.build_codebook(bits), head_dim=wl.head_dim)
        c.codes[...] = rng.integers(0, 256, size=c.codes.shape, dtype=np.uint8)
        if bits == 16:   # float16 rows: finite values
            c.codes.view(np.float16)[...] = rng.standard_normal(c.codes.view(np.float16).shape).astype(np.float16)
        c.norms[...] = rng.uniform(5.0, 15.0, size=c.norms.shape).astype(np.float32)
        caches.append(c)
    new = rng.standard_normal((2, n_qtok, 1, wl.head_dim)).astype(np.float16)
    q = wl.queries()[b:b + 1, :, kv * g:(kv + 1) * g]
    table = np.arange(n_pages, dtype=np.int32)[None, :]
    lens = np.array([length], np.int32)
    new_slots = np.arange(length - n_qtok, length, dtype=np.int64)
    with_limits = _one_thread()
    t0 = time.perf_counter()
    O.cache_write(caches[0], new[0], new_slots)
    O.cache_write(caches[1], new[1], new_slots)
    O.decode_attention(q, caches[0], caches[1], lens, table, n_qtok, 0.0, wl.tau)
    dt = time.perf_counter() - t0
    del with_limits
    per_tok = hb * (cache_bytes_per_token_head(wl.k_bits) + cache_bytes_per_token_head(wl.v_bits))
    nbytes = length * per_tok + n_qtok * (2 * 2 * wl.head_dim + per_tok) + q.size * 6
    return dt, nbytes


def _cpu_quant_unit(job):
    """(seconds, token-layers) of the oracle quantize of one (layer, side) of the prefill."""
    import oracle as O
    _, layer, side = job
    wl = W.prefill()
    x = wl.kv_source(layer)[side]
    bits = wl.k_bits if side == 0 else wl.v_bits
    c = O.new_cache(bits, wl.n_kv_heads, wl.block_size, wl.n_blocks, wl.signs(layer)[side], O.build_codebook(bits))
    slots = np.arange(wl.n_tokens, dtype=np.int64)
    with_limits = _one_thread()
    t0 = time.perf_counter()
    O.cache_write(c, x, slots)
    dt = time.perf_counter() - t0
    del with_limits
    return dt, 0.5 * wl.n_tokens   # a token-layer is K and V of all heads: half of it per side


def _cpu_worker(jobs):
    out = []
    for kind, job in jobs:
        out.append(_cpu_quant_unit(job) if kind == "q" else _cpu_decode_unit(job))
    return out


def cpu_units(name):
    """Every independent unit of a workload, in a seeded order, and a description."""
    if name == "quantize":
        wl = W.prefill()
        units = [("q", ("prefill", layer, side)) for layer in range(wl.n_layers) for side in (0, 1)]
        return units, "prefill: (layer, side) units"
    wl = decode_workload(name)
    units = [("d", (name, b, kv)) for b in range(wl.n_seqs) for kv in range(wl.n_kv_heads)
             if int(wl.seq_lens[b]) > 0]
    order = np.random.default_rng(11).permutation(len(units))
    return [units[i] for i in order], f"{name}: (sequence, KV head) decode steps"


def cpu_baseline(name, budget_s=6.0, max_units=None, procs=None):
    """The oracle on the host: a single process for about budget_s seconds, then one
    process per core over max_units units (all of them by default)."""
    import multiprocessing as mp
    units, what = cpu_units(name)
    info = host_info()
    # single process, bounded (the units in order, cycling for a small workload)
    done, spent, amount = 0, 0.0, 0.0
    while done == 0 or spent < budget_s:
        dt, x = _cpu_worker([units[done % len(units)]])[0]
        spent += dt
        amount += x
        done += 1
        if done >= len(units) and spent >= 0.5 * budget_s:
            break
    single = amount / spent
    # all cores: the sample (repeated when it is too small to keep every process
    # busy for about a second)
    p = procs or min(16, info["usable_cpus"])
    sample = units if max_units is None else units[:max_units]
    rep = max(1, min(64, math.ceil(p * 1.0 / (spent / done * len(sample)))))
    work = sample * rep
    p = min(p, len(work))
    jobs = [work[i::p] for i in range(p)]
    t_wall = time.perf_counter()
    with mp.get_context("spawn").Pool(p) as pool:
        res = pool.map(_cpu_worker, jobs)
    t_wall = time.perf_counter() - t_wall
    makespan = max(sum(dt for dt, _ in r) for r in res)
    total = sum(x for r in res for _, x in r)
    multi = total / makespan
    scale, unit = (1e6, "M token-layers/s") if name == "quantize" else (1e9, "GB/s")
    full = len(sample) == len(units)
    log(f"[bench] cpu oracle {name}: 1 process {done} units in {spent:.1f} s -> {single / scale:.4f} {unit}; "
        f"{p} processes {len(work)} units, slowest {makespan:.1f} s (wall {t_wall:.1f} s) -> "
        f"{multi / scale:.4f} {unit}")
    return {"value": round(multi / scale, 5), "unit": unit, "cores": p, "kind": "oracle",
            "sample": f"{what}: {len(sample)} of {len(units)} units"
                      f"{' (the whole workload)' if full else ' (seeded subset; the rate needs no scaling)'}"
                      f"{f', each run {rep} times' if rep > 1 else ''}, "
                      f"{p} processes x 1 thread, units dealt round-robin, time = the slowest process's timed "
                      f"total {makespan:.1f} s"
                      f"{'' if name == 'quantize' else '; context codes are seeded random bytes (the work does not depend on them)'}",
            "single_process": {"value": round(single / scale, 5), "unit": unit, "cores": 1,
                               "sample": f"{done} units, {spent:.1f} s"},
            "host": info}


# per workload: units of the all-core run (None = all)
CPU_SAMPLE = {"ragged": 64, "longctx": None, "llama8b": None, "tiny": None, "quantize": None}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all", choices=["all"] + DECODE_WORKLOADS,
                    help="all: the ragged headline with the llama8b, longctx, tiny and quantize sub-records")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--separate-append", action="store_true",
                    help="append with tq_quantize_kv and decode with tq_decode_attention (two calls)")
    ap.add_argument("--quantize-reps", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=0,
                    help="tokens per decode pass block (0: the library's choice)")
    ap.add_argument("--no-quantize", action="store_true")
    ap.add_argument("--quantize-only", action="store_true", help="only the prefill quantize measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device copies of 256 MiB (reference for HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("KERNEL:WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="(no GPU) write one kernel's HBM bytes per launch from two rocprofv3 --pmc "
                         "counter_collection.csv files into profiles/pmc_traffic.json")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
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

    head = "ragged" if args.workload == "all" else args.workload
    subs = ["llama8b", "longctx", "tiny"] if args.workload == "all" else []
    wl, rec = run_decode(args, torch, head)
    sub = {}
    for name in subs:
        sub[name] = run_decode(args, torch, name)[1]
    if not args.no_quantize:
        sub["quantize"] = run_quantize(args, torch)
        sub["codebook_fit"] = run_codebook_fit(torch)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(head, max_units=CPU_SAMPLE.get(head, 64))
        for name in subs + ([] if args.no_quantize else ["quantize"]):
            sub[name]["cpu_baseline"] = cpu_baseline(name, max_units=CPU_SAMPLE.get(name))
    else:
        rec["cpu_baseline"] = None
    out = {
        "metric": METRIC, "value": rec["value"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec["dtype"],
        "data": "synthetic",
        "config": {"workload": rec["workload"], "global_batch": wl.n_seqs, "seq_len": int(wl.seq_lens.max()),
                   "replicas": rec["replicas"], "launch": rec["launch"], "ms_per_step_eager": rec["ms_per_step_eager"],
                   "append": rec["append"], "decode_kernel": rec["decode_kernel"], "parallelism": "single GPU"},
        "pct_of_peak": rec["pct_of_peak"], "step_bytes": rec["step_bytes"],
        "query_tokens_per_s": rec["query_tokens_per_s"], "kv_token_heads_per_s": rec["kv_token_heads_per_s"],
        "roofline": rec["roofline"], "cpu_baseline": rec["cpu_baseline"],
    }
    if "sparse_v" in rec:
        out["sparse_v"] = rec["sparse_v"]
    out["sub_records"] = sub
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
