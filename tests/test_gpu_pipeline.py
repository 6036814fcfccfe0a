"""Simulated-DCP pipelines (convert -> decode per shard -> LSE merge) and the merge kernel on
the GPU against the oracle, at the configurations' real sizes."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
import sparse_mla_decode_topk_amd as smla
from sparse_mla_decode_topk_amd.pipeline import DcpDecodeStep, device_shards
from tests.gpu_common import OUT_TOL, check_close, dev, oracle_unsharded, q_dev, require_gpu
from workload import make_config, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def out_dtype_of(w):
    return torch.float32 if w.out_dtype == "fp32" else torch.bfloat16


def run_step(w, shards=None, **kw):
    shards = shards or device_shards(w)
    step = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=w.dcp_size, block_size=w.block_size,
                         softmax_scale=w.sm_scale, out_dtype=out_dtype_of(w), **kw)
    out, lse = step.run(q_dev(w), dev(w.ids), dev(w.req), shards)
    torch.cuda.synchronize()
    return step, out, lse


def unsharded_gpu(w):
    step = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=1, block_size=w.block_size, softmax_scale=w.sm_scale,
                         out_dtype=out_dtype_of(w))
    out, lse = step.run(q_dev(w), dev(w.ids), dev(w.req),
                        [(w.cache.to_device("cuda"), dev(w.block_table))])
    torch.cuda.synchronize()
    return out, lse


def test_dcp4_c2_full():
    w = make_config(2)
    print(f"c2: T={w.T} H={w.H} D={w.dcp_size}", flush=True)
    step, out, lse = run_step(w)
    ref_o, ref_l = oracle_unsharded(w)
    do, dl = check_close(out, lse, ref_o, ref_l, what="c2 merged vs oracle")
    print(f"  merged vs oracle max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)
    # the four context-2 rows: shards 2 and 3 own no candidate and emit (0, -inf)
    lp = step.lse_parts.cpu().numpy()
    pp = step.parts.float().cpu().numpy()
    for r in (2, 3):
        assert np.all(np.isneginf(lp[r, 32:])) and np.all(pp[r, 32:] == 0)
    for r in (0, 1):
        assert np.all(np.isfinite(lp[r, 32:]))
    # merged == unsharded GPU result within the same bar
    uo, ul = unsharded_gpu(w)
    check_close(out, lse, uo.float().cpu().numpy().astype(np.float64), ul.cpu().numpy().astype(np.float64),
                what="c2 merged vs unsharded gpu")


def test_dcp2_c3_full_size_every_row():
    """The timed configuration: MTP rows, H=128, top-k 2048, DCP2, kernel-native (H,T) LSE; every
    row of the merged step and of the unsharded decode against the oracle."""
    w = make_config(3)
    print(f"c3: T={w.T} H={w.H} K={w.K}", flush=True)
    step, out, lse = run_step(w, lse_layout="HT")
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    ref_o, ref_l = oracle_unsharded(w)
    do, dl = check_close(out, lse, ref_o, ref_l, what="c3 merged, every row")
    print(f"  merged max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)
    uo, ul = unsharded_gpu(w)
    do, dl = check_close(uo, ul, ref_o, ref_l, what="c3 unsharded, every row")
    print(f"  unsharded max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)


def test_dcp4_c2_counts_change_nothing():
    """The step passes the conversion's counts to every shard decode; without them the partials are
    bitwise the same (shards 2 and 3 count 0 for the four context-2 rows)."""
    w = make_config(2)
    shards = device_shards(w)
    step, out, lse = run_step(w, shards=shards)
    vc = step.valid.cpu().numpy()
    assert np.all(vc[2:, 32:] == 0) and np.all(vc[:2, 32:] == 1)
    for r, (cache, bt) in enumerate(shards):
        o, l = smla.decode(q_dev(w), cache, step.slots[r], w.sm_scale, out_dtype=torch.float32,
                           num_splits=step.num_splits)
        torch.cuda.synchronize()
        assert torch.equal(o, step.parts[r]) and torch.equal(l, step.lse_parts[r])


@pytest.mark.parametrize("D,I,H,splits", [(2, 2, 128, 0), (2, 3, 64, 3), (4, 2, 64, 0), (4, 3, 128, 2)])
def test_interleaved_dcp_pipeline(D, I, H, splits):
    """DCP with interleave I (page "FlashMLA sparse fp8 path gains DCP and MTP", Implementation
    breakdown step 4): rank r holds the tokens p with (p // I) % D == r; the merged step equals the
    unsharded oracle."""
    w = make_random(500 + 10 * D + I, T=10, H=H, K=320, ctx=1200, B=64, D=D, neg_frac=0.15, n_req=3, interleave=I)
    print(f"D={D} I={I} H={H} splits={splits}", flush=True)
    step, out, lse = run_step(w, interleave=I, num_splits=splits)
    ref_o, ref_l = oracle_unsharded(w)
    do, dl = check_close(out, lse, ref_o, ref_l, what=f"D{D} I{I}")
    print(f"  max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)
    counts = step.valid.cpu().numpy()  # per shard and row: the ids each rank owns
    ids = np.asarray(w.ids)
    for r in range(D):
        own = (ids >= 0) & ((ids // I) % D == r)
        assert np.array_equal(counts[r], own.sum(axis=1))


def test_dcp8_c4_subset_rows_full_caches():
    """Mixed batch at full context (131072-token decode requests, 8 shards) on a row subset."""
    w = make_config(4, scale_rows=48)
    print(f"c4 subset: T={w.T} H={w.H} D={w.dcp_size}", flush=True)
    step, out, lse = run_step(w, lse_layout="HT")
    ref_o, ref_l = oracle_unsharded(w)
    do, dl = check_close(out, lse, ref_o, ref_l, what="c4 subset")
    print(f"  max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)




@pytest.mark.parametrize("partials", [torch.float32, torch.bfloat16])
def test_dcp8_c4_full_size_rows(partials):
    """The mixed batch at its full size (T = 4224, 8 shards), in the launch the c4 bench line times,
    against the oracle on every decode row, every prefill row at positions 0-63 (a row at position p
    has p + 1 candidates, so up to 7 of its 8 shards own none and must drop out of the merge) and a
    sample further along both prompts; with fp32 shard partials (the default) and with bf16 ones
    (one more rounding of every partial row before the merge), both at the 2e-2 / 1e-3 bars."""
    w = make_config(4)
    print(f"c4 full: T={w.T} H={w.H} D={w.dcp_size} partials {partials}", flush=True)
    step, out, lse = run_step(w, lse_layout="HT", partial_dtype=partials)
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    pos = np.asarray(w.row_pos)
    decode_rows = [int(r) for r in np.flatnonzero(pos == pos.max())]
    short = [int(r) for r in np.flatnonzero(pos < 64)]
    assert len(decode_rows) == 128 and len(short) == 128
    rows = sorted(set(decode_rows) | set(short) | set(range(0, w.T, 37)) | {w.T - 1})
    ref_o, ref_l = oracle_unsharded(w, rows)
    do, dl = check_close(out[rows], lse[rows], ref_o, ref_l, out_tol=OUT_TOL, what=f"c4 rows, {partials} partials")
    print(f"  {len(rows)} rows max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)


@pytest.mark.parametrize("S,dtype", [(1, torch.float32), (2, torch.float32), (4, torch.bfloat16), (8, torch.float32)])
def test_merge_against_oracle(S, dtype):
    rng = np.random.default_rng(S)
    T, H = 7, 48
    parts = rng.standard_normal((S, T, H, 512)).astype(np.float32)
    lses = (rng.standard_normal((S, T, H)) * 4).astype(np.float32)
    lses[rng.random((S, T, H)) < 0.3] = -np.inf  # empty partials
    lses[:, 2, :] = -np.inf  # an entry empty everywhere
    parts[np.isneginf(lses)] = 0.0  # an empty partial carries out = 0
    pt = dev(parts).to(dtype)
    ref_o, ref_l = O.merge_lse(pt.float().cpu().numpy().astype(np.float64), lses.astype(np.float64))
    out, lse = smla.merge_lse(pt, dev(lses), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close(out, lse, ref_o, ref_l, out_tol=1e-5, lse_tol=1e-5, what=f"merge S{S}")
    assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_merge_identity_is_exact():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 5, 16, 512)).astype(np.float32)
    l = rng.standard_normal((1, 5, 16)).astype(np.float32)
    parts = np.concatenate([o, np.zeros_like(o)])
    lses = np.concatenate([l, np.full_like(l, -np.inf)])
    out, lse = smla.merge_lse(dev(parts), dev(lses), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.allclose(out.cpu().numpy(), o[0], rtol=0, atol=2e-6)
    assert np.allclose(lse.cpu().numpy(), l[0], rtol=0, atol=2e-6)


def test_graph_capture_replays_match_eager():
    w = make_random(401, T=12, H=128, K=512, ctx=2048, B=64, D=2, neg_frac=0.1, n_req=3)
    shards = device_shards(w)
    q, ids, req = q_dev(w), dev(w.ids), dev(w.req)
    for num_splits in (1, 3):  # 3 exercises the workspace and the split-merge kernel
        step = DcpDecodeStep(T=w.T, H=w.H, K=w.K, dcp_size=2, block_size=w.block_size, softmax_scale=w.sm_scale,
                             num_splits=num_splits)
        out, lse = step.run(q, ids, req, shards)
        torch.cuda.synchronize()
        eager_o, eager_l = out.clone(), lse.clone()
        g = step.capture(q, ids, req, shards)
        for rep in range(3):
            step.out.fill_(123.0)
            step.lse.fill_(-5.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(step.out, eager_o), f"replay {rep} splits {num_splits}: out differs"
            assert torch.equal(step.lse, eager_l), f"replay {rep} splits {num_splits}: lse differs"
        ref_o, ref_l = oracle_unsharded(w)
        check_close(step.out, step.lse, ref_o, ref_l, what=f"graph splits{num_splits}")
        # new contents in the captured storage: the replay reads them, and matches an eager run
        q2 = q.clone()
        q.mul_(-0.5)
        g.replay()
        torch.cuda.synchronize()
        graph_o, graph_l = step.out.clone(), step.lse.clone()
        step.run(q, ids, req, shards)
        torch.cuda.synchronize()
        assert torch.equal(step.out, graph_o) and torch.equal(step.lse, graph_l), f"splits {num_splits}: new q"
        assert not torch.equal(graph_o, eager_o)
        q.copy_(q2)
