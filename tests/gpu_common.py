"""Shared helpers of the GPU parity tests (inputs to the device, oracle references, checks)."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O

# Bar for floating point results against the fp64 oracle: max |dout| <= 2e-2, max |dlse| <= 1e-3.
OUT_TOL = 2e-2
LSE_TOL = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_decode_topk_amd as smla
    smla.load_library()  # raises when the HIP library is missing: no silent fallback


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def q_dev(w):
    return w.q_torch().cuda()


def oracle_unsharded(w, rows=None):
    """Oracle out/lse of the rows of a workload against its unsharded cache."""
    sub = w if rows is None else w.rows(rows)
    slots, _ = O.convert_index(sub.ids, sub.req, sub.block_table, sub.block_size)
    return O.attention_rows(sub.q_f32(), slots, sub.cache, sub.cache.num_slots, sub.sm_scale)


def check_close(out, lse, ref_out, ref_lse, out_tol=OUT_TOL, lse_tol=LSE_TOL, what=""):
    o = out.float().cpu().numpy() if isinstance(out, torch.Tensor) else np.asarray(out, dtype=np.float64)
    l = lse.float().cpu().numpy() if isinstance(lse, torch.Tensor) else np.asarray(lse, dtype=np.float64)
    assert not np.isnan(o).any(), f"{what}: NaN in out"
    assert not np.isnan(l).any(), f"{what}: NaN in lse"
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref_lse)
    dl = float(np.max(np.abs(l[fin] - ref_lse[fin]), initial=0.0))
    do = float(np.max(np.abs(o - ref_out), initial=0.0))
    assert dl <= lse_tol, f"{what}: max |dlse| = {dl:.3e} > {lse_tol}"
    assert do <= out_tol, f"{what}: max |dout| = {do:.3e} > {out_tol}"
    empty = np.isneginf(ref_lse)
    assert np.all(o[empty] == 0.0), f"{what}: empty rows must be exactly 0"
    return do, dl
