"""Host logic of the measurement script that needs no GPU: the traffic record
written from rocprofv3 counter files (the dominant instantiation, the copy-derived
scales, the source hash that ties the record to the kernel sources)."""

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, [values per XCD])"""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, values in rows:
            for v in values:
                w.writerow([d, d, name, counter, v])


def test_record_traffic_takes_the_dominant_instantiation(tmp_path, monkeypatch):
    score = "void tq::tq_decode_mfma_kernel<3, 2, false, 1, true, 1, false, false>(tq::DecodeArgs)"
    gated = "void tq::tq_decode_mfma_kernel<3, 2, false, 2, true, 1, false, false>(tq::DecodeArgs)"
    other = "tq::tq_merge_kernel<true, false, 8>(tq::DecodeArgs)"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # per dispatch the counters come in several rows (one per XCD) that add up
    _counter_csv(fetch, "FETCH_SIZE", [(1, score, [600.0, 400.0]), (2, gated, [50.0]), (3, other, [5000.0]),
                                       (4, score, [500.0, 500.0]), (5, gated, [70.0])])
    _counter_csv(write, "WRITE_SIZE", [(1, score, [10.0, 10.0]), (2, gated, [1.0]), (4, score, [30.0, 10.0])])
    rec_path = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_RECORD", str(rec_path))
    bench.record_traffic("tq_decode_mfma_kernel:longctx", str(fetch), str(write))
    rec = json.load(open(rec_path))["tq_decode_mfma_kernel:longctx"]
    assert rec["kernel_name"].startswith("void tq::tq_decode_mfma_kernel<3, 2, false, 1,")   # not the gated pass
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_kib_per_dispatch"] == 1000.0 and rec["write_kib_per_dispatch"] == 30.0
    assert rec["fetch_bytes"] == int(bench.FETCH_SCALE * 1000.0 * 1024)
    assert rec["write_bytes"] == int(bench.WRITE_SCALE * 30.0 * 1024)
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["source_hash"] == bench.source_hash("tq_decode_mfma_kernel")
    assert bench.pmc_traffic("tq_decode_mfma_kernel:longctx") == rec["bytes_per_launch"]
    # a record of other sources is not reported
    rec_all = json.load(open(rec_path))
    rec_all["tq_decode_mfma_kernel:longctx"]["source_hash"] = "0" * 16
    json.dump(rec_all, open(rec_path, "w"))
    assert bench.pmc_traffic("tq_decode_mfma_kernel:longctx") is None


def test_committed_traffic_records_match_the_sources():
    """The committed record holds one entry per measured kernel and workload, tied to
    the sources of this tree (so bench reports them)."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "pmc_traffic.json")))
    for key in ("tq_decode_mfma_kernel:ragged", "tq_decode_mfma_kernel:longctx", "tq_decode_mfma_kernel:llama8b",
                "tq_quantize_kernel:prefill"):
        assert key in rec
        assert rec[key]["source_hash"] == bench.source_hash(key.split(":")[0]), key
        assert rec[key]["bytes_per_launch"] == rec[key]["fetch_bytes"] + rec[key]["write_bytes"]
