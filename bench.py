"""Throughput of the sparse-MLA decode step on one MI355X.

Workload: MTP / speculative decode batch, 64 requests x 4 query tokens (T = 256 rows),
H = 128 heads, context 32768 per request, top-k 2048 causal ids per row, fp8_ds_mla cache,
simulated DCP2 (two shard caches on the same GPU).  One step = for each shard, index
conversion + decode (fp32 partial out, LSE in the kernel-native (H, T) layout), then the
LSE merge into bf16 out and (T, H) LSE.

Prints one JSON line on stdout.  `value` is query rows per second of the whole step with
every input resident in HBM, each step replayed as one HIP graph (`ms_per_step_eager` gives
the same steps launched one call at a time).  `roofline` covers the decode kernel:
algorithmic bytes and flops per launch over its mean launch time (HIP events on the launch
stream around a graph of back-to-back launches).
`unsharded_decode` times the same rows against the unsharded cache (the H = 128 / top-k 2048
decode, MFMA-bound) after the step.  `cpu_baseline` times the fp64 oracle on a bounded sample
of the same rows.  `cache_write` times the fp8_ds_mla cache write of one 32768-token chunk
beside the step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode query-rows/s and KV GB/s (H=128, topk=2048) + % roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FLOP_PER_VALID_ID_PER_HEAD = 2 * (576 + 512)  # QK^T over 576 dims + PV over 512 dims


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_algorithmic(T, H, K, nvalid, nunique, out_bytes, record_bytes=656):
    """Bytes and flops one decode launch must move / compute: every distinct record the launch
    reads once (rows of one request that picked the same token share it), q, the slot lists,
    out and LSE; 2176 flops per (valid id, head) of every row."""
    byts = record_bytes * nunique + T * H * 576 * 2 + T * K * 4 + T * H * (512 * out_bytes + 4)
    flops = FLOP_PER_VALID_ID_PER_HEAD * H * nvalid
    return byts, flops


def unique_records(ids, req, dcp_size=1, dcp_rank=0):
    """Distinct valid ids per request that DCP rank `dcp_rank` owns (interleave 1), summed over
    requests: the records one decode launch of that rank must read at least once."""
    import numpy as np
    ids, req = np.asarray(ids), np.asarray(req)
    n = 0
    for b in np.unique(req):
        x = ids[req == b]
        x = x[(x >= 0) & (x % dcp_size == dcp_rank)]
        n += int(np.unique(x).size)
    return n


def roofline_entry(byts, flops, seconds):
    t_hbm = byts / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        achieved = byts / seconds / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}


def time_cache_write(dev, iters=20, n=32768):
    """fp8_ds_mla cache write of one n-token prefill chunk (bf16 latent and rope, no DCP):
    mean launch time over `iters` launches (HIP events on the launch stream) and its rate
    against HBM, counting 1152 B read + 8 B of position and request + 656 B written + 4 B
    of slot mapping per token."""
    import numpy as np
    import torch
    import sparse_mla_decode_topk_amd as smla
    g = torch.Generator(device="cpu").manual_seed(5)
    lat = torch.randn((n, 512), generator=g).to(torch.bfloat16).to(dev)
    rope = torch.randn((n, 64), generator=g).to(torch.bfloat16).to(dev)
    pos = torch.arange(n, dtype=torch.int32, device=dev)
    req = torch.zeros(n, dtype=torch.int32, device=dev)
    bt = torch.randperm(n // 64, generator=g).to(torch.int32).reshape(1, -1).to(dev)
    cache = torch.empty((n, 656), dtype=torch.uint8, device=dev)
    sm = torch.empty((n,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        smla.cache_write(lat, rope, pos, req, bt, cache, 64, slot_mapping=sm)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record(stream)
        smla.cache_write(lat, rope, pos, req, bt, cache, 64, slot_mapping=sm)
        b.record(stream)
    torch.cuda.synchronize()
    s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    byts = n * (1152 + 8 + 656 + 4)
    gbps = byts / s / 1e9
    return {"tokens": n, "dtype": "bf16", "us": round(s * 1e6, 2), "algorithmic_bytes": byts,
            "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4)}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def dense_algorithmic(w):
    """Bytes and flops of one whole-context decode of workload ``w``: every record of every
    request once (the S rows and the head blocks of a request share them), q, out (bf16),
    LSE and the slot lists; 2176 flops per (visible position, head)."""
    import numpy as np
    visible = int(np.maximum(w.row_pos + 1, 0).sum())
    K = int(w.ctx.max())
    byts = 656 * int(w.ctx.sum()) + w.T * w.H * 576 * 2 + w.T * w.H * (512 * 2 + 4) + w.T * K * 4 * 2
    return byts, FLOP_PER_VALID_ID_PER_HEAD * w.H * visible


def main_dense(args):
    """--workload dense: the whole-context decode of 32 requests x 4 MTP tokens (T = 128 rows),
    H = 128, context 4096 per request, one call per step."""
    import numpy as np
    import torch
    import sparse_mla_decode_topk_amd as smla
    from workload import make_dense

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    smla.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    S, n_req, ctx, H = 4, 32, 4096, 128
    log(f"generating dense workload ({n_req} requests x {S} MTP tokens, H={H}, context {ctx}) ...")
    w = make_dense(2000, n_req=n_req, S=S, H=H, ctx=ctx, B=64)
    q = w.q_torch().to(dev)
    caches = [w.cache.to_device(dev) for _ in range(max(1, args.replicas))]
    bt = torch.from_numpy(w.block_table).to(dev)
    seq = torch.from_numpy(w.ctx.astype(np.int32)).to(dev)
    out = torch.empty((w.T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(i):
        smla.dense_decode(q, caches[i % len(caches)], bt, seq, S, w.sm_scale, w.block_size, ctx, out=out, lse=lse)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        run(i)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    byts, flops = dense_algorithmic(w)
    roof = roofline_entry(byts, flops, call_s)
    roof.update({"traffic": None, "kernel": "dense_slots_kernel + decode_row_kernel (one whole-context decode call)",
                 "launch_us": round(call_s * 1e6, 2), "algorithmic_bytes": int(byts), "algorithmic_flops": int(flops)})
    line = {
        "metric": METRIC, "value": round(w.T * args.steps / wall, 1), "unit": "query-rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"dense_mtp: {n_req} req x {S} MTP tokens (T={w.T}), H={H}, whole context {ctx} "
                               f"(causal per MTP token), fp8_ds_mla cache, no DCP", "T": w.T, "H": H, "S": S,
                   "ctx": ctx, "block_size": w.block_size, "cache_replicas": len(caches)},
        "kv_gbps": round(656 * int(np.maximum(w.row_pos + 1, 0).sum()) / call_s / 1e9, 1),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle.smla_oracle as O
        log("timing the CPU oracle on a bounded sample ...")
        tally = ParityTally(*host_result(out, lse))
        rows_done, t0, t_cmp = 0, time.perf_counter(), 0.0
        while time.perf_counter() - t0 - t_cmp < args.cpu_budget:
            t = rows_done % w.T
            sub = w.rows([t])
            sl, _ = O.convert_index(sub.ids, sub.req, sub.block_table, sub.block_size)
            ref = O.attention_rows(sub.q_f32(), sl, sub.cache, sub.cache.num_slots, sub.sm_scale)
            rows_done += 1
            tc = time.perf_counter()
            tally.add([t], *ref)
            t_cmp += time.perf_counter() - tc
        el = time.perf_counter() - t0 - t_cmp
        line["parity"] = tally.result()
        line["cpu_baseline"] = {"value": round(rows_done / el, 3), "unit": "query-rows/s", "cores": blas_threads(),
                                "kind": "oracle",
                                "sample": f"{rows_done} rows of the same workload in order through the fp64 numpy "
                                          f"oracle (each row: its causal position list, block-table conversion, "
                                          f"attention); {el:.1f} s on {blas_threads()} host CPUs"}
    print(json.dumps(line), flush=True)


def main_bf16(args):
    """--workload bf16: the top-k decode of the c3 rows (T = 256, H = 128, top-k 2048, context
    32768) against the unsharded cache in the plain bf16 layout (1152 bytes per token)."""
    import numpy as np
    import torch
    import sparse_mla_decode_topk_amd as smla
    from workload import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    smla.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log("generating workload c3 with bf16 records (T=256, H=128, top-k 2048, ctx 32768) ...")
    w = make_config(3, kv="bf16")
    q = w.q_torch().to(dev)
    caches = [w.cache.to_device(dev) for _ in range(max(1, args.replicas))]
    bt = torch.from_numpy(w.block_table).to(dev)
    slots, _ = smla.convert_index(torch.from_numpy(w.ids).to(dev), torch.from_numpy(w.req).to(dev), bt, w.block_size)
    out = torch.empty((w.T, w.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(i):
        smla.decode(q, caches[i % len(caches)], slots, w.sm_scale, out=out, lse=lse, kv_layout="bf16")

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        run(i)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    nvalid = int((w.ids >= 0).sum())
    byts, flops = decode_algorithmic(w.T, w.H, w.K, nvalid, unique_records(w.ids, w.req), out_bytes=2,
                                     record_bytes=1152)
    roof = roofline_entry(byts, flops, call_s)
    roof.update({"traffic": None, "kernel": "decode_bf16_kernel (one unsharded call)", "launch_us": round(call_s * 1e6, 2),
                 "algorithmic_bytes": int(byts), "algorithmic_flops": int(flops),
                 "mfma_frac": round(flops / call_s / (BF16_PEAK_TFLOPS * 1e12), 4)})
    line = {
        "metric": METRIC, "value": round(w.T * args.steps / wall, 1), "unit": "query-rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "c3_bf16kv: 64 req x 4 MTP tokens (T=256), H=128, top-k 2048 causal, ctx 32768, "
                               "plain bf16 cache (1152 B/token), unsharded", "T": w.T, "H": w.H, "topk": w.K,
                   "ctx": 32768, "block_size": w.block_size, "cache_replicas": len(caches)},
        "kv_gbps": round(1152 * nvalid / call_s / 1e9, 1),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle.smla_oracle as O
        log("timing the CPU oracle on a bounded sample ...")
        tally = ParityTally(*host_result(out, lse))
        rows_done, t0, t_cmp = 0, time.perf_counter(), 0.0
        while time.perf_counter() - t0 - t_cmp < args.cpu_budget:
            t = rows_done % w.T
            sub = w.rows([t])
            sl, _ = O.convert_index(sub.ids, sub.req, sub.block_table, sub.block_size)
            ref = O.attention_rows(sub.q_f32(), sl, sub.cache, sub.cache.num_slots, sub.sm_scale, record_layout="bf16")
            rows_done += 1
            tc = time.perf_counter()
            tally.add([t], *ref)
            t_cmp += time.perf_counter() - tc
        el = time.perf_counter() - t0 - t_cmp
        line["parity"] = tally.result()
        line["cpu_baseline"] = {"value": round(rows_done / el, 3), "unit": "query-rows/s", "cores": blas_threads(),
                                "kind": "oracle",
                                "sample": f"{rows_done} rows of the same workload in order through the fp64 numpy "
                                          f"oracle (conversion and attention over bf16 records); {el:.1f} s on "
                                          f"{blas_threads()} host CPUs"}
    print(json.dumps(line), flush=True)


def host_result(out, lse):
    """The step's final (out, lse) copied to host memory as float32 numpy arrays [T,H,512], [T,H]."""
    return out.float().cpu().numpy(), lse.float().cpu().numpy()


class ParityTally:
    """Distances of GPU results from the oracle's on the rows the oracle computed (each row once)."""

    def __init__(self, gpu_out, gpu_lse):
        self.out, self.lse = gpu_out, gpu_lse
        self.seen = set()
        self.dout = self.dlse = self.max_out = 0.0
        self.inf_ok = True
        self.finite = True

    def add(self, rows, ref_o, ref_l):
        import numpy as np
        keep = [i for i, r in enumerate(rows) if r not in self.seen]
        if not keep:
            return
        rr = [rows[i] for i in keep]
        self.seen.update(rr)
        go, gl = self.out[rr].astype(np.float64), self.lse[rr].astype(np.float64)
        ro, rl = np.asarray(ref_o)[keep], np.asarray(ref_l)[keep]
        self.finite &= bool(np.isfinite(go).all()) and not bool(np.isnan(gl).any())
        self.dout = max(self.dout, float(np.abs(go - ro).max()))
        self.max_out = max(self.max_out, float(np.abs(ro).max()))
        fin = np.isfinite(rl)
        self.inf_ok &= bool(np.array_equal(np.isneginf(gl), np.isneginf(rl)))
        if fin.any():
            self.dlse = max(self.dlse, float(np.abs(gl[fin] - rl[fin]).max()))

    def result(self):
        return {"rows_checked": len(self.seen), "max_abs_dout": self.dout, "max_abs_dlse": self.dlse,
                "max_abs_out": self.max_out, "out_tolerance": 2e-2, "lse_tolerance": 1e-3,
                "out_margin": round(2e-2 / self.dout, 2) if self.dout else None,
                "lse_margin": round(1e-3 / self.dlse, 1) if self.dlse else None,
                "neg_inf_lse_identical": self.inf_ok, "no_nan": self.finite,
                "within_tolerance": bool(self.finite and self.inf_ok and self.dout <= 2e-2 and self.dlse <= 1e-3),
                "against": "the fp64 oracle rows of cpu_baseline, every element of each row"}


def cpu_baseline(w, budget_s, order=None, what=None, gpu=None):
    """fp64 oracle of the same DCP step (converts, shard attention, merge) over the rows in
    `order` (default: in order), wrapping around, until the time budget is spent; rows/s over
    the rows done.  gpu: the step's host (out, lse); the oracle rows are then also compared
    with it (outside the timed part) and the distances come back under "parity"."""
    import numpy as np
    import oracle.smla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    order = list(range(w.T)) if order is None else [int(r) for r in order]
    tally = ParityTally(*gpu) if gpu is not None else None
    rows_done, t0, t_cmp = 0, time.perf_counter(), 0.0
    chunk = 4
    while time.perf_counter() - t0 - t_cmp < budget_s:
        start = rows_done % len(order)
        rows = order[start:start + chunk]
        sub = w.rows(rows)
        q = sub.q_f32()
        outs, lses = [], []
        if sub.dcp_size == 1:  # one cache, no merge
            s, _ = O.convert_index(sub.ids, sub.req, sub.block_table, sub.block_size)
            ref = O.attention_rows(q, s, sub.cache, sub.cache.num_slots, sub.sm_scale)
        else:
            for sh in sub.shards:
                s, _ = O.convert_index(sub.ids, sub.req, sh.block_table, sub.block_size, sub.dcp_size, sh.rank)
                o, l = O.attention_rows(q, s, sh.cache, sh.cache.num_slots, sub.sm_scale)
                outs.append(o)
                lses.append(l)
            ref = O.merge_lse(np.stack(outs), np.stack(lses))
        rows_done += len(rows)
        if tally is not None:
            tc = time.perf_counter()
            tally.add(rows, *ref)
            t_cmp += time.perf_counter() - tc
    dt = time.perf_counter() - t0 - t_cmp
    res = {"value": round(rows_done / dt, 3), "unit": "query-rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows_done} rows ({what or f'the {w.T} rows of the same DCP{w.dcp_size} step in order'}, "
                      f"wrapping) through the fp64 numpy oracle: "
                      + ("convert and attention" if w.dcp_size == 1 else
                         f"{w.dcp_size} shard converts, shard attention, LSE merge")
                      + f"; {dt:.1f} s on {os.cpu_count()} host CPUs"}
    return (res, tally.result()) if tally is not None else res


# HBM bytes per decode launch of this workload, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE, each with --copy-mib 1024) scaled by what the same counters
# read for the plain 1 GiB device copy.  Valid only for the kernel sources they were taken on.
DECODE_TRAFFIC = {"sources_sha256": "14d748d1ae38070c495fe5edfc7a180e8697f0f030d074df6bfd849eee8079b0",
                  "fetch_bytes": 227193197, "write_bytes": 67428577}
# SQ counters of the same shard decode (profiles/decode_row_kernel_c3_dcp2_counters.md): MFMA busy =
# SQ_VALU_MFMA_BUSY_CYCLES per SIMD over busy cycles, LDS busy = SQ_LDS_IDX_ACTIVE per CU over busy cycles
DECODE_COUNTERS = {"sources_sha256": "14d748d1ae38070c495fe5edfc7a180e8697f0f030d074df6bfd849eee8079b0", "mfma_busy": 0.3203, "lds_busy": 0.2265}
KERNEL_SOURCES = ("sparse_mla_decode_topk_amd/csrc/decode_row.hip", "sparse_mla_decode_topk_amd/csrc/decode_common.h",
                  "sparse_mla_decode_topk_amd/csrc/smla_internal.h")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    t = DECODE_TRAFFIC
    if t["sources_sha256"] is None or t["sources_sha256"] != kernel_sources_sha256():
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def measured_counters():
    """MFMA and LDS busy fractions of the shard decode from the committed counter profile, or None
    once the kernel sources differ from the ones profiled."""
    c = DECODE_COUNTERS
    if c["sources_sha256"] != kernel_sources_sha256():
        return None
    return {"mfma_busy": c["mfma_busy"], "lds_busy": c["lds_busy"],
            "source": "profiles/decode_row_kernel_c3_dcp2_counters.md (rocprofv3 SQ counters)"}


def graph_steps(step, q, ids, req, replicas, steps, warmup):
    """Run the step as HIP graph replays: one captured step per cache replica, `warmup` untimed
    replays, then exactly `steps` timed replays (replica i % len(replicas) for step i), bracketed
    by device synchronisation.  Returns the wall time of the timed replays in seconds."""
    import torch
    graphs = [step.capture(q, ids, req, shards) for shards in replicas]
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def decode_launch_ms(step, q, replicas, launches=48, rounds=7):
    """Per-launch decode time: a HIP graph of `launches` back-to-back decode calls (shards and
    cache replicas in rotation, on the slots of the step's last conversion), replayed `rounds`
    times between HIP events on the launch stream; one mean per replay.  Back to back, the
    launches keep the GPU busy, so host-side launch cost stays out of the figure."""
    import torch

    def body():
        for k in range(launches):
            r = k % step.D
            step.decode_shard(q, replicas[(k // step.D) % len(replicas)][r][0], r)

    body()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    stream = torch.cuda.current_stream()
    graph.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(rounds):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / launches)
    return per


def achievable_peaks():
    """What plain loops reach on this device (libsmla_peak.so): streaming HBM read and copy,
    dense bf16 32x32x16 and fp8 32x32x64 MFMA chains at two waves per SIMD."""
    from sparse_mla_decode_topk_amd import peak
    r = peak.run(quick=True)
    return {"hbm_read_gbps": r["read"]["gbps"], "hbm_copy_gbps": r["copy"]["gbps"],
            "bf16_mfma_tflops": r["mfma_bf16_32x32x16_w2"]["tflops"], "fp8_mfma_tflops": r["mfma_fp8_32x32x64_w2"]["tflops"],
            "source": "sparse_mla_decode_topk_amd/peak.py (csrc/peak.hip): streaming read/copy of 1 GiB, "
                      "8 independent MFMA chains per wave, 8 waves per CU"}


def add_achievable(roof, ach):
    """The fraction of the roofline against the achievable peak of the same unit."""
    if ach is None:
        return roof
    key = "hbm_read_gbps" if roof["unit"] == "GB/s" else "bf16_mfma_tflops"
    roof["achievable_peak"] = ach[key]
    roof["frac_of_achievable"] = round(roof["achieved"] / ach[key], 4)
    return roof


def percentiles_us(ms):
    """p10 / median / p90 of launch durations given in milliseconds, in microseconds."""
    import numpy as np
    return [round(float(x) * 1e3, 2) for x in np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])]


def main_small(args, cid):
    """--workload c1 / c2: the small configurations.  c1: 32 single-token decode rows, H = 64,
    context 4096, top-k 2048, one cache (D = 1; the automatic plan splits every row 8 ways).  c2:
    the c1 rows plus 4 rows of 2-token contexts, simulated DCP4.  One c1 cache is 86 MB, so
    `--replicas` (at least 4) copies are rotated between steps to keep the gather in HBM rather
    than the 256 MB MALL."""
    import numpy as np
    import torch
    import sparse_mla_decode_topk_amd as smla
    from sparse_mla_decode_topk_amd.pipeline import DcpDecodeStep, device_shards
    from workload import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    smla.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = make_config(cid)
    reps = max(4, args.replicas)
    log(f"workload {w.name}: T={w.T} H={w.H} top-k {w.K} D={w.dcp_size}; {reps} cache replicas")
    q = w.q_torch().to(dev)
    ids = torch.from_numpy(w.ids).to(dev)
    req = torch.from_numpy(w.req).to(dev)
    replicas = [device_shards(w, dev) for _ in range(reps)]
    torch.cuda.synchronize()
    step = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=w.dcp_size, block_size=w.block_size,
                         softmax_scale=w.sm_scale, out_dtype=torch.float32, partial_dtype=torch.float32, device=dev)
    D = w.dcp_size
    shard_valid = [int(((w.ids >= 0) & (w.ids % D == r)).sum()) for r in range(D)]
    shard_unique = [unique_records(w.ids, w.req, D, r) for r in range(D)]
    log(f"warmup {args.warmup} steps (eager), then {args.steps} eager and {args.steps} graph-replayed steps")
    for i in range(args.warmup):
        step.run(q, ids, req, replicas[i % reps])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step.run(q, ids, req, replicas[i % reps])
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t_start
    wall = graph_steps(step, q, ids, req, replicas, args.steps, args.warmup)
    gpu = None if args.no_cpu_baseline else host_result(step.out, step.lse)  # the last replay's result
    dec_ms = decode_launch_ms(step, q, replicas)
    mean_dec_s = float(np.mean(dec_ms)) / 1e3
    byts, flops = decode_algorithmic(w.T, w.H, w.K, float(np.mean(shard_valid)), float(np.mean(shard_unique)),
                                     out_bytes=4)
    roof = roofline_entry(byts, flops, mean_dec_s)
    roof.update({"traffic": None,
                 "kernel": f"decode_row_kernel (one {'' if D == 1 else f'DCP{D} shard '}call: T={w.T}, H={w.H}, "
                           f"K={w.K}, fp32 {'out' if D == 1 else 'partials'})",
                 "launch_us": round(mean_dec_s * 1e6, 2), "launch_us_p10_p50_p90": percentiles_us(dec_ms),
                 "launch_timing": "mean of back-to-back launches in a HIP graph, events on the launch stream",
                 "algorithmic_bytes": int(byts), "algorithmic_flops": int(flops)})
    desc = {1: "c1_decode: 32 requests x 1 token (T=32), H=64, ctx 4096, top-k 2048, fp8_ds_mla cache, D=1 "
               "(convert + decode, fp32 out)",
            2: "c2_dcp4: the c1 rows + 4 rows of 2-token contexts (T=36), H=64, top-k 2048, fp8_ds_mla cache, "
               "simulated DCP4 (convert+decode per shard, LSE merge)"}[cid]
    line = {
        "metric": METRIC, "value": round(w.T * args.steps / wall, 1), "unit": "query-rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": desc, "T": w.T, "H": w.H, "topk": w.K, "dcp": D, "block_size": w.block_size,
                   "cache_replicas": reps, "launch": "each step replayed as one HIP graph"},
        "ms_per_step_eager": round(eager_wall * 1e3 / args.steps, 4),
        "kv_gbps": round(656 * float(np.mean(shard_valid)) / mean_dec_s / 1e9, 1),
        "roofline": add_achievable(roof, None if args.no_peaks else achievable_peaks()),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"], line["parity"] = cpu_baseline(w, args.cpu_budget, gpu=gpu)
    print(json.dumps(line), flush=True)


def main_c4(args):
    """--workload c4: the long-context mixed batch (128 decode rows with 131072-token contexts
    and 4096 prefill rows of two fresh 2048-token prompts, T = 4224, H = 128, top-k 2048),
    simulated DCP8: per step 8 x (convert + decode into fp32 partials) and one LSE merge."""
    import numpy as np
    import torch
    import sparse_mla_decode_topk_amd as smla
    from sparse_mla_decode_topk_amd.pipeline import DcpDecodeStep, device_shards
    from workload import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    smla.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log("generating workload c4 (T=4224, H=128, top-k 2048, decode ctx 131072, DCP8) ...")
    t0 = time.perf_counter()
    w = make_config(4)
    log(f"  generated in {time.perf_counter() - t0:.1f} s; copying the 8 shard caches to the GPU")
    q = w.q_torch().to(dev)
    ids = torch.from_numpy(w.ids).to(dev)
    req = torch.from_numpy(w.req).to(dev)
    shards = device_shards(w, dev)  # one copy: 8 x 1.4 GB of shard caches, far beyond the 256 MB MALL
    torch.cuda.synchronize()
    step = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=w.dcp_size, block_size=w.block_size,
                         softmax_scale=w.sm_scale, out_dtype=torch.bfloat16, partial_dtype=torch.float32,
                         lse_layout="HT", device=dev)
    shard_valid = [int(((w.ids >= 0) & (w.ids % w.dcp_size == r)).sum()) for r in range(w.dcp_size)]
    shard_unique = [unique_records(w.ids, w.req, w.dcp_size, r) for r in range(w.dcp_size)]
    log(f"warmup {args.warmup} steps (eager), then {args.steps} eager and {args.steps} graph-replayed steps")
    for _ in range(args.warmup):
        step.run(q, ids, req, shards)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step.run(q, ids, req, shards)
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t_start
    wall = graph_steps(step, q, ids, req, [shards], args.steps, args.warmup)
    gpu = None if args.no_cpu_baseline else host_result(step.out, step.lse)  # the last replay's result
    dec_ms = decode_launch_ms(step, q, [shards], launches=16, rounds=3)
    mean_dec_s = float(np.mean(dec_ms)) / 1e3
    byts, flops = decode_algorithmic(w.T, w.H, w.K, float(np.mean(shard_valid)), float(np.mean(shard_unique)),
                                     out_bytes=4)
    roof = roofline_entry(byts, flops, mean_dec_s)
    roof.update({"traffic": None,
                 "kernel": "decode_row_kernel (one DCP8 shard call: T=4224, H=128, K=2048, fp32 partials)",
                 "launch_us": round(mean_dec_s * 1e6, 2), "launch_us_p10_p50_p90": percentiles_us(dec_ms),
                 "launch_timing": "mean of back-to-back launches in a HIP graph, events on the launch stream",
                 "algorithmic_bytes": int(byts), "algorithmic_flops": int(flops),
                 "mfma_frac": round(flops / mean_dec_s / 1e12 / BF16_PEAK_TFLOPS, 4)})
    line = {
        "metric": METRIC, "value": round(w.T * args.steps / wall, 1), "unit": "query-rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "c4_mixed_dcp8: 128 decode rows (ctx 131072) + 4096 prefill rows (2 x 2048), "
                               "H=128, top-k 2048, fp8_ds_mla cache, simulated DCP8 (convert+decode per shard, "
                               "LSE merge)",
                   "T": w.T, "H": w.H, "topk": w.K, "dcp": w.dcp_size, "block_size": w.block_size,
                   "launch": "each step replayed as one HIP graph"},
        "ms_per_step_eager": round(eager_wall * 1e3 / args.steps, 4),
        "kv_gbps": round(656 * float(np.mean(shard_valid)) / mean_dec_s / 1e9, 1),
        "roofline": roof,
    }
    if not args.no_bf16_partials:  # the same step with bf16 shard partials: time and distance
        out32, lse32 = step.out.float().clone(), step.lse.clone()
        del step
        step16 = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=w.dcp_size, block_size=w.block_size,
                               softmax_scale=w.sm_scale, out_dtype=torch.bfloat16, partial_dtype=torch.bfloat16,
                               lse_layout="HT", device=dev)
        wall16 = graph_steps(step16, q, ids, req, [shards], args.steps, args.warmup)
        dec16 = decode_launch_ms(step16, q, [shards], launches=16, rounds=3)
        fin = torch.isfinite(lse32)
        d_out = float((step16.out.float() - out32).abs().max())
        d_lse = float((step16.lse[fin] - lse32[fin]).abs().max()) if bool(fin.any()) else 0.0
        same_inf = bool(torch.equal(torch.isneginf(step16.lse), torch.isneginf(lse32)))
        line["bf16_partials"] = {
            "ms_per_step": round(wall16 * 1e3 / args.steps, 4), "launch_us": round(float(np.mean(dec16)) * 1e3, 2),
            "max_abs_dout_vs_fp32_partials": d_out, "max_abs_dlse_vs_fp32_partials": d_lse,
            "neg_inf_lse_identical": same_inf, "out_tolerance": 2e-2, "out_margin": round(2e-2 / d_out, 1) if d_out else None,
            "note": "the same step with bf16 shard partials (decode writes bf16, the merge reads bf16); distances "
                    "are to the fp32-partial step of this run, every element"}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        order = np.random.Generator(np.random.PCG64(4004)).permutation(w.T)
        line["cpu_baseline"], line["parity"] = cpu_baseline(
            w, args.cpu_budget, order=order, what=f"the {w.T} rows of the DCP8 step in a seeded random order", gpu=gpu)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=2, help="cache copies rotated between steps (beat the 256 MB MALL)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unsharded", action="store_true",
                    help="skip the unsharded decode of the same rows (timed after the step and reported beside it)")
    ap.add_argument("--workload", choices=("c3", "c1", "c2", "dense", "bf16", "c4"), default="c3",
                    help="c3: the DCP2 MTP step (default); c1 / c2: the small single-token decode batch, unsharded / "
                         "under DCP4; dense: the whole-context MTP decode; bf16: the c3 rows unsharded against a plain "
                         "bf16 cache; c4: the long-context mixed batch under DCP8")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak microbenchmarks")
    ap.add_argument("--no-bf16-partials", action="store_true", help="c4: skip the bf16-partial variant of the step")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (got --gpus {args.gpus}); "
              f"the DCP shards are simulated on one device", file=sys.stderr)
        sys.exit(2)
    if args.workload == "dense":
        main_dense(args)
        return
    if args.workload == "bf16":
        main_bf16(args)
        return
    if args.workload == "c4":
        main_c4(args)
        return
    if args.workload in ("c1", "c2"):
        main_small(args, int(args.workload[1]))
        return

    import numpy as np
    import torch

    import sparse_mla_decode_topk_amd as smla
    from sparse_mla_decode_topk_amd.pipeline import DcpDecodeStep, device_shards
    from workload import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    smla.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    log("generating workload c3 (T=256, H=128, top-k 2048, ctx 32768, DCP2) ...")
    t0 = time.perf_counter()
    w = make_config(3)
    log(f"  generated in {time.perf_counter() - t0:.1f} s; copying caches to the GPU ({args.replicas} replicas)")
    q = w.q_torch().to(dev)
    ids = torch.from_numpy(w.ids).to(dev)
    req = torch.from_numpy(w.req).to(dev)
    replicas = [device_shards(w, dev) for _ in range(max(1, args.replicas))]
    if not args.no_unsharded:
        unsharded_cache = w.cache.to_device(dev)
        unsharded_bt = torch.from_numpy(w.block_table).to(dev)
    torch.cuda.synchronize()

    step = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=w.dcp_size, block_size=w.block_size,
                         softmax_scale=w.sm_scale, out_dtype=torch.bfloat16, partial_dtype=torch.float32,
                         lse_layout="HT", device=dev)
    # valid ids per shard (host-side count from the inputs, outside any timed region)
    nvalid = [int((np.asarray(w.ids) >= 0).sum())]
    shard_valid, shard_unique = [], []
    for r in range(w.dcp_size):
        own = (w.ids >= 0) & ((w.ids % w.dcp_size) == r)
        shard_valid.append(int(own.sum()))
        shard_unique.append(unique_records(w.ids, w.req, w.dcp_size, r))

    def run_step(i):
        return step.run(q, ids, req, replicas[i % len(replicas)])

    log(f"warmup {args.warmup} steps (eager), then {args.steps} eager and {args.steps} graph-replayed steps")
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        run_step(i)
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t_start
    wall = graph_steps(step, q, ids, req, replicas, args.steps, args.warmup)
    gpu = None if args.no_cpu_baseline else host_result(step.out, step.lse)  # the last replay's result
    ms_per_step = wall * 1e3 / args.steps
    rows_per_s = w.T * args.steps / wall
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step (graph), {eager_wall * 1e3 / args.steps:.4f} (eager)")

    # decode kernel roofline: mean over back-to-back launches (both shards have ~the same valid count)
    dec_ms = decode_launch_ms(step, q, replicas)
    mean_dec_s = float(np.mean(dec_ms)) / 1e3
    nv_mean = float(np.mean(shard_valid))
    byts, flops = decode_algorithmic(w.T, w.H, w.K, nv_mean, float(np.mean(shard_unique)), out_bytes=4)
    roof = roofline_entry(byts, flops, mean_dec_s)
    roof["traffic"] = measured_traffic()
    roof["counters"] = measured_counters()
    if roof["counters"] is not None:
        roof["mfma_busy"] = roof["counters"]["mfma_busy"]
    roof["kernel"] = "decode_row_kernel (one DCP2 shard call: T=256, H=128, K=2048, ~1024 valid ids/row, fp32 partials)"
    roof["launch_us"] = round(mean_dec_s * 1e6, 2)
    roof["launch_us_p10_p50_p90"] = percentiles_us(dec_ms)
    roof["launch_timing"] = "mean of back-to-back launches in a HIP graph, events on the launch stream"
    roof["algorithmic_bytes"] = int(byts)
    roof["algorithmic_flops"] = int(flops)
    kv_gbps = 656 * float(np.mean(shard_valid)) / mean_dec_s / 1e9

    unsharded = None
    if not args.no_unsharded:  # the unsharded H=128 / top-k 2048 decode of the same rows
        one = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=1, block_size=w.block_size, softmax_scale=w.sm_scale,
                            out_dtype=torch.bfloat16, device=dev)
        one.run(q, ids, req, [(unsharded_cache, unsharded_bt)])
        torch.cuda.synchronize()
        un_ms = decode_launch_ms(one, q, [[(unsharded_cache, unsharded_bt)]], launches=24)
        un_s = float(np.mean(un_ms)) / 1e3
        ub, uf = decode_algorithmic(w.T, w.H, w.K, nvalid[0], unique_records(w.ids, w.req), out_bytes=2)
        unsharded = {"decode_us": round(un_s * 1e6, 2), "decode_us_p10_p50_p90": percentiles_us(un_ms),
                     "tflops": round(uf / un_s / 1e12, 1),
                     "kv_gbps": round(656 * nvalid[0] / un_s / 1e9, 1), "roofline": roofline_entry(ub, uf, un_s)}
    cache_write = time_cache_write(dev)
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    line = {
        "metric": METRIC, "value": round(rows_per_s, 1), "unit": "query-rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "c3_mtp_dcp2: 64 req x 4 MTP tokens (T=256), H=128, top-k 2048 causal, ctx 32768, "
                               "fp8_ds_mla cache, simulated DCP2 (convert+decode per shard, LSE merge)",
                   "T": w.T, "H": w.H, "topk": w.K, "ctx": 32768, "dcp": w.dcp_size, "block_size": w.block_size,
                   "cache_replicas": len(replicas), "launch": "each step replayed as one HIP graph"},
        "ms_per_step_eager": round(eager_wall * 1e3 / args.steps, 4),
        "kv_gbps": round(kv_gbps, 1),
        "roofline": roof,
    }
    ach = None if args.no_peaks else achievable_peaks()
    add_achievable(line["roofline"], ach)
    if unsharded is not None:
        add_achievable(unsharded["roofline"], ach)
        line["unsharded_decode"] = unsharded
    if ach is not None:
        line["achievable_peaks"] = ach
    line["cache_write"] = cache_write
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"], line["parity"] = cpu_baseline(w, args.cpu_budget, gpu=gpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
