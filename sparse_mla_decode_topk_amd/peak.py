"""Achievable-peak microbenchmarks (libsmla_peak.so, built from csrc/peak.hip).

Measures, on the current device, what plain loops reach on the units the decode depends on:
HBM streaming (copy and read), dense MFMA chains (bf16 32x32x16 and 16x16x32, fp8 32x32x64) and
the time per MFMA of 1, 2, 4 or 8 dependent 16x16x32 chains per wave,
the e4m3 -> bf16 widening conversion, and MFMA with independent fp32 FMAs beside it in one
wave.  Each figure is also given as a fraction of MI355X's published peak (HBM 8 TB/s; dense
bf16 2.5 PFLOP/s, fp8 5.0 PFLOP/s) so a kernel's roofline fraction can be read against what
the hardware delivers to a simple loop.  Measurement only: nothing in the decode path uses it.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

PUBLISHED = {"hbm_gbps": 8000.0, "bf16_tflops": 2500.0, "fp8_tflops": 5000.0}
_FLOPS = {0: 32 * 32 * 16 * 2, 1: 16 * 16 * 32 * 2, 2: 32 * 32 * 64 * 2}

_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsmla_peak.so")


def load():
    global _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
            lib = ctypes.CDLL(path)
            lib.smla_peak_copy.argtypes = [_P, _P, _I64, _I32, _P]
            lib.smla_peak_read.argtypes = [_P, _I64, _I32, _P, _P]
            lib.smla_peak_mfma.argtypes = [_I32, _I32, _I32, _I32, _P, _P]
            lib.smla_peak_mix.argtypes = [_I32, _I32, _I32, _I32, _P, _P]
            lib.smla_peak_cvt.argtypes = [_I32, _I32, _I32, _P, _P]
            lib.smla_peak_clock.argtypes = [_I32, _I32, _P, _P]
            lib.smla_peak_mixi.argtypes = [_I32, _I32, _I32, _I32, _P, _P]
            lib.smla_peak_valu.argtypes = [_I32, _I32, _I32, _I32, _P, _P]
            lib.smla_peak_lds.argtypes = [_I32, _I32, _I32, _I32, _P, _P]
            lib.smla_peak_dual.argtypes = [_I32, _I32, _I32, _I32, _P, _P]
            lib.smla_peak_chain.argtypes = [_I32, _I32, _I32, _I32, _P, _P]
            for f in ("smla_peak_copy", "smla_peak_read", "smla_peak_mfma", "smla_peak_mix", "smla_peak_cvt",
                      "smla_peak_clock", "smla_peak_mixi", "smla_peak_valu", "smla_peak_lds", "smla_peak_dual",
                      "smla_peak_chain"):
                getattr(lib, f).restype = ctypes.c_int
            _lib = lib
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _time_ms(launch, reps=5):
    """Mean event time of `reps` launches after one warm-up launch."""
    launch()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        s.record()
        launch()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    return sum(times) / len(times)


def _check(st, what):
    if st != 0:
        raise RuntimeError(f"{what}: status {st}")


def run(mib: int = 1024, iters: int = 4096, cus: int | None = None, quick: bool = False) -> dict:
    """All measurements; returns a JSON-ready dict.  quick: only the streams and the MFMA chains."""
    lib = load()
    dev = torch.device("cuda", torch.cuda.current_device())
    cus = cus or torch.cuda.get_device_properties(dev).multi_processor_count
    res = {"cus": cus}

    n = (mib << 20) // 16
    src = torch.empty(n * 16, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(cus * 8 * 512, dtype=torch.float32, device=dev)
    grid = cus * 8
    ms = _time_ms(lambda: _check(lib.smla_peak_copy(src.data_ptr(), dst.data_ptr(), n, grid, _stream()), "copy"))
    gbps = 32.0 * n / (ms * 1e-3) / 1e9
    res["copy"] = {"bytes": 32 * n, "us": round(ms * 1e3, 1), "gbps": round(gbps, 1),
                   "frac_of_published": round(gbps / PUBLISHED["hbm_gbps"], 3)}
    ms = _time_ms(lambda: _check(lib.smla_peak_read(src.data_ptr(), n, grid, sink.data_ptr(), _stream()), "read"))
    gbps = 16.0 * n / (ms * 1e-3) / 1e9
    res["read"] = {"bytes": 16 * n, "us": round(ms * 1e3, 1), "gbps": round(gbps, 1),
                   "frac_of_published": round(gbps / PUBLISHED["hbm_gbps"], 3)}
    del src, dst

    names = {0: "bf16_32x32x16", 1: "bf16_16x16x32", 2: "fp8_32x32x64"}
    for kind, name in names.items():
        for wps in (1, 2):  # waves per SIMD: 4 or 8 waves per workgroup, one workgroup per CU
            waves = 4 * wps
            ms = _time_ms(lambda: _check(lib.smla_peak_mfma(kind, iters, cus, waves, sink.data_ptr(), _stream()), name))
            flops = _FLOPS[kind] * 8 * iters * waves * cus
            tf = flops / (ms * 1e-3) / 1e12
            peak = PUBLISHED["fp8_tflops" if kind == 2 else "bf16_tflops"]
            res[f"mfma_{name}_w{wps}"] = {"tflops": round(tf, 1), "frac_of_published": round(tf / peak, 3),
                                          "us": round(ms * 1e3, 1)}

    if quick:
        return res

    # MFMA + independent fp32 FMAs in one wave: time per iteration (four 32x32x16 bf16 MFMAs), with
    # the FMAs after the four MFMAs (mix) or spread between them (mixi)
    for fn, key in ((lib.smla_peak_mix, "mix_ns_per_iter"), (lib.smla_peak_mixi, "mix_interleaved_ns_per_iter")):
        mix = {}
        for wps in (1, 2):
            for nv in (0, 16, 32, 64, 128):
                ms = _time_ms(lambda: _check(fn(nv, iters, cus, 4 * wps, sink.data_ptr(), _stream()), key))
                mix[f"w{wps}_nv{nv}"] = round(ms * 1e6 / iters, 2)  # ns per iteration per wave
        res[key] = mix

    # dependent 16x16x32 bf16 MFMA chains: ns per MFMA per SIMD for 1, 2, 4, 8 chains per wave
    chain = {}
    for wps in (1, 2):
        for c in (1, 2, 4, 8):
            ms = _time_ms(lambda: _check(lib.smla_peak_chain(c, iters, cus, 4 * wps, sink.data_ptr(), _stream()), "chain"))
            chain[f"w{wps}_chains{c}"] = round(ms * 1e6 / (iters * c * wps), 3)
    res["mfma16_chain_ns_per_mfma_per_simd"] = chain

    # vector issue: ns per instruction per SIMD for 32 independent instances per iteration
    ops = ("v_fma_f32", "v_cvt_scalef32_pk_bf16_fp8", "v_cvt_pk_f32_fp8", "v_perm_b32", "v_exp_f32",
           "v_cvt_pk_bf16_f32", "v_and_or_b32")
    valu = {}
    for op, name in enumerate(ops):
        for wps in (1, 2):
            ms = _time_ms(lambda: _check(lib.smla_peak_valu(op, iters, cus, 4 * wps, sink.data_ptr(), _stream()), name))
            valu[f"{name}_w{wps}"] = round(ms * 1e6 / (32 * iters * wps), 3)
    res["valu_ns_per_instr_per_simd"] = valu

    # one MFMA wave + one conversion wave per SIMD: us per launch for each side alone and both
    dual = {}
    for name, mf, va in (("mfma_only", 1, 0), ("cvt_only", 0, 1), ("both", 1, 1)):
        ms = _time_ms(lambda: _check(lib.smla_peak_dual(iters, mf, va, cus, sink.data_ptr(), _stream()), "dual"))
        dual[name] = round(ms * 1e3, 1)
    res["dual_wave_us"] = dual

    # LDS: bytes per CU per ns (per shader cycle: divide by the clock in GHz)
    lds = {}
    for op, (name, nbytes) in enumerate((("ds_read_b128", 16), ("ds_read_b64", 8), ("ds_read_b64_tr_b8", 8),
                                         ("ds_write_b128", 16))):
        for waves in (1, 4, 8):
            ms = _time_ms(lambda: _check(lib.smla_peak_lds(op, iters, cus, waves, sink.data_ptr(), _stream()), name))
            lds[f"{name}_waves{waves}"] = round(16 * iters * waves * 64 * nbytes / (ms * 1e6), 1)
    res["lds_bytes_per_ns_per_cu"] = lds

    for wps in (1, 2):
        ms = _time_ms(lambda: _check(lib.smla_peak_cvt(iters, cus, 4 * wps, sink.data_ptr(), _stream()), "cvt"))
        per_simd = 16 * iters * wps  # conversion instructions per SIMD
        res[f"cvt_w{wps}_ns_per_instr_per_simd"] = round(ms * 1e6 / per_simd, 3)

    stamps = torch.zeros(cus * 4, dtype=torch.int64, device=dev)
    _check(lib.smla_peak_clock(iters * 4, cus, stamps.data_ptr(), _stream()), "clock")
    torch.cuda.synchronize()
    st = stamps.view(cus, 4).cpu().double()
    cyc = (st[:, 1] - st[:, 0]).mean().item()
    rt = (st[:, 3] - st[:, 2]).mean().item()  # 100 MHz ticks
    res["clock"] = {"mfma_busy_mhz": round(cyc / (rt / 100.0), 1) if rt > 0 else None,
                    "cycles_per_32x32x16": round(cyc / (iters * 4 * 2), 2)}
    return res


if __name__ == "__main__":
    import json
    import sys

    torch.cuda.set_device(0)
    json.dump(run(), sys.stdout, indent=1)
    print()
