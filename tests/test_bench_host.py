"""bench.py's host-side arithmetic: the algorithmic bytes and flops of one decode launch, the
choice of the binding roof, and the one-GPU guard.  No GPU is needed."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_algorithmic_counts_records_query_slots_and_output():
    # one row, one head, one valid id: a 656-byte record, 576 bf16 query values, one int32 slot,
    # 512 output values of out_bytes each plus the fp32 LSE; 2 (576 + 512) flops
    b, f = bench.decode_algorithmic(T=1, H=1, K=1, nvalid=1, nunique=1, out_bytes=2)
    assert b == 656 + 1152 + 4 + (1024 + 4)
    assert f == 2 * (576 + 512)
    # -1 entries cost nothing: K grows the slot list only
    b2, f2 = bench.decode_algorithmic(T=1, H=1, K=9, nvalid=1, nunique=1, out_bytes=2)
    assert b2 - b == 8 * 4 and f2 == f
    # a record two rows share is read once but multiplied twice
    b3, f3 = bench.decode_algorithmic(T=2, H=1, K=1, nvalid=2, nunique=1, out_bytes=4, record_bytes=1152)
    assert b3 == 1152 + 2 * (1152 + 4 + 2048 + 4) and f3 == 2 * f
    # the unsharded H = 128, top-k 2048 decode of 256 rows with bf16 output
    b, f = bench.decode_algorithmic(T=256, H=128, K=2048, nvalid=256 * 2048, nunique=256 * 2048, out_bytes=2)
    assert f == 2176 * 128 * 524288
    assert b == 656 * 524288 + 256 * 128 * (1152 + 1028) + 256 * 2048 * 4
    # at H = 128 a record carries 425 flop per byte, above the 312 flop/B bf16 ridge: MFMA-bound
    assert 2176 * 128 / 656 > 2.5e15 / 8e12


def test_unique_records_per_request_and_rank():
    ids = [[0, 1, 2, -1], [2, 3, 1, 5], [0, 4, -1, -1]]
    req = [0, 0, 1]
    # request 0 reads {0, 1, 2, 3, 5}, request 1 reads {0, 4}: the same id in two requests is two
    # records (different sequences)
    assert bench.unique_records(ids, req) == 5 + 2
    # DCP2, rank 0 owns even ids: {0, 2} and {0, 4}; rank 1: {1, 3, 5}
    assert bench.unique_records(ids, req, 2, 0) == 2 + 2
    assert bench.unique_records(ids, req, 2, 1) == 3 + 0


def test_roofline_entry_takes_the_binding_roof():
    e = bench.roofline_entry(8e9, 1e12, 2e-3)  # 1 ms of HBM against 0.4 ms of MFMA
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["peak"] == 8000.0
    assert abs(e["achieved"] - 4000.0) < 1e-6 and e["frac"] == 0.5
    e = bench.roofline_entry(1e9, 5e12, 4e-3)  # 2 ms of MFMA against 0.125 ms of HBM
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s" and e["peak"] == 2500.0
    assert abs(e["achieved"] - 1250.0) < 1e-6 and e["frac"] == 0.5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_shard_split_plan():
    # DCP shard decodes are planned for their ~K / D valid entries: c2's DCP4 shards (T = 36,
    # H = 64, K = 2048) take 2 ranges of >= 256 valid entries instead of 8 ranges of ~64; rows
    # that already cover the CUs, and long lists, follow the library's own rule
    from sparse_mla_decode_topk_amd.pipeline import shard_splits
    assert shard_splits(36, 64, 2048, 4, 256) == 2
    assert shard_splits(32, 64, 2048, 2, 256) == 4
    assert shard_splits(256, 128, 2048, 2, 256) == 1
    assert shard_splits(4224, 128, 2048, 8, 256) == 1
    assert shard_splits(1, 16, 262144, 2, 256) == 64
    assert shard_splits(4, 64, 100, 4, 256) == 1


def test_counter_figures_follow_the_kernel_sources(monkeypatch):
    # the traffic and counter figures belong to the kernel sources they were measured on
    import bench
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: bench.DECODE_COUNTERS["sources_sha256"])
    c = bench.measured_counters()
    assert c is not None and 0.0 < c["mfma_busy"] < 1.0 and 0.0 < c["lds_busy"] < 1.0
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_counters() is None and bench.measured_traffic() is None


def test_parity_tally_reports_the_largest_distances_once_per_row():
    """The bench's oracle comparison: each row counts once, the -inf pattern must match, and the
    largest element distances and the margins to the 2e-2 / 1e-3 bars are what it reports."""
    import numpy as np
    rng = np.random.default_rng(7)
    ref_o = rng.standard_normal((6, 4, 512))
    ref_l = rng.standard_normal((6, 4))
    ref_o[2], ref_l[2] = 0.0, -np.inf  # an empty row
    gpu_o = (ref_o + 1e-3).astype(np.float32)
    gpu_l = ref_l.astype(np.float32)
    gpu_o[4, 1, 7] += 4e-3  # the largest out distance: 5e-3
    gpu_l[5, 3] += 2e-4
    t = bench.ParityTally(gpu_o, gpu_l)
    t.add([0, 1, 2], ref_o[[0, 1, 2]], ref_l[[0, 1, 2]])
    t.add([2, 3, 4, 5], ref_o[[2, 3, 4, 5]], ref_l[[2, 3, 4, 5]])  # row 2 again: counted once
    r = t.result()
    assert r["rows_checked"] == 6
    assert abs(r["max_abs_dout"] - 5e-3) < 1e-6 and abs(r["max_abs_dlse"] - 2e-4) < 1e-6
    assert r["neg_inf_lse_identical"] and r["no_nan"] and r["within_tolerance"]
    assert abs(r["out_margin"] - 4.0) < 0.01
    bad = bench.ParityTally(gpu_o, np.where(np.isinf(gpu_l), np.float32(0.0), gpu_l))
    bad.add([2], ref_o[[2]], ref_l[[2]])  # a finite LSE where the oracle has -inf
    assert not bad.result()["neg_inf_lse_identical"] and not bad.result()["within_tolerance"]
