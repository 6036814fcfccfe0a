"""Sparse MLA decode over plain bf16 records (576 values, 1152 bytes per token) on the GPU against
the fp64 oracle (max |dout| <= 2e-2, max |dlse| <= 1e-3)."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
import sparse_mla_decode_topk_amd as smla
from tests.gpu_common import check_close, dev, q_dev, require_gpu
from workload import make_config, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(w, cache=None, shard=None, out_dtype=torch.float32, num_splits=0, rows=None):
    sub = w if rows is None else w.rows(rows)
    bt = w.block_table if shard is None else shard.block_table
    c = w.cache if shard is None else shard.cache
    D, r = (1, 0) if shard is None else (w.dcp_size, shard.rank)
    slots, _ = O.convert_index(sub.ids, sub.req, bt, w.block_size, D, r)
    dc = c.to_device("cuda") if cache is None else cache
    out, lse = smla.decode(q_dev(sub), dc, dev(slots), w.sm_scale, out_dtype=out_dtype, num_splits=num_splits,
                           kv_layout="bf16")
    torch.cuda.synchronize()
    ref_o, ref_l = O.attention_rows(sub.q_f32(), slots, c, c.num_slots, w.sm_scale, record_layout="bf16")
    return out, lse, ref_o, ref_l


def test_bf16_c0():
    w = make_config(0, kv="bf16")
    print(f"bf16 c0: T={w.T} H={w.H} K={w.K}", flush=True)
    out, lse, ro, rl = run(w, out_dtype=torch.bfloat16)
    check_close(out, lse, ro, rl, what="bf16 c0")


@pytest.mark.parametrize("H,K,neg", [(16, 48, 0.0), (64, 300, 0.3), (128, 2048, 0.1), (32, 17, 0.0),
                                     (128, 4096, 0.5), (32, 9000, 0.05)])
def test_bf16_random_shapes(H, K, neg):
    w = make_random(500 + H + K, T=9, H=H, K=K, ctx=max(K, 64) + 40, B=16, neg_frac=neg, n_req=3, kv="bf16")
    print(f"bf16 random: T={w.T} H={H} K={K} neg={neg}", flush=True)
    out, lse, ro, rl = run(w)
    check_close(out, lse, ro, rl, what=f"bf16 H{H} K{K}")


@pytest.mark.parametrize("splits", [2, 3, 8])
def test_bf16_forced_splits(splits):
    w = make_random(77, T=6, H=64, K=700, ctx=900, B=32, neg_frac=0.2, n_req=2, kv="bf16")
    out, lse, ro, rl = run(w, num_splits=splits, out_dtype=torch.bfloat16)
    check_close(out, lse, ro, rl, what=f"bf16 splits {splits}")


def test_bf16_empty_rows_and_out_of_range():
    w = make_random(91, T=5, H=32, K=64, ctx=128, B=16, n_req=2, kv="bf16")
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    slots[1] = -1  # a row with no candidate
    slots[3, :10] = w.cache.num_slots + 5  # out of range: skipped like -1
    slots[4, 5] = -7
    cache = w.cache.to_device("cuda")
    out, lse = smla.decode(q_dev(w), cache, dev(slots), w.sm_scale, out_dtype=torch.float32, kv_layout="bf16")
    torch.cuda.synchronize()
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale, record_layout="bf16")
    check_close(out, lse, ro, rl, what="bf16 empty / out of range")
    assert torch.isneginf(lse[1]).all() and (out[1] == 0).all()


def test_bf16_dcp_shards_merge_to_unsharded():
    w = make_random(33, T=8, H=64, K=512, ctx=1500, B=16, D=4, n_req=2, kv="bf16")
    outs, lses = [], []
    for sh in w.shards:
        o, l, ro, rl = run(w, shard=sh)
        check_close(o, l, ro, rl, what=f"bf16 shard {sh.rank}")
        outs.append(o)
        lses.append(l)
    mo, ml = smla.merge_lse(torch.stack(outs), torch.stack(lses), out_dtype=torch.float32)
    torch.cuda.synchronize()
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale, record_layout="bf16")
    check_close(mo, ml, ro, rl, what="bf16 DCP4 merged")


def test_bf16_long_context_h128_sampled():
    """H = 128, top-k 2048 over 32768-token contexts, sampled rows against the oracle."""
    w = make_random(44, T=32, H=128, K=2048, ctx=32768, B=64, n_req=8, all_real=False, kv="bf16")
    cache = w.cache.to_device("cuda")
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    out, lse = smla.decode(q_dev(w), cache, dev(slots), w.sm_scale, out_dtype=torch.bfloat16, kv_layout="bf16")
    torch.cuda.synchronize()
    rows = [0, 7, 19, 31]
    sub = w.rows(rows)
    ro, rl = O.attention_rows(sub.q_f32(), slots[rows], w.cache, w.cache.num_slots, w.sm_scale, record_layout="bf16")
    check_close(out[rows], lse[rows], ro, rl, what="bf16 H128 K2048")
    assert not torch.isnan(out).any() and torch.isfinite(lse).all()


@pytest.mark.parametrize("k", [24, 40])
@pytest.mark.parametrize("splits", [1, 3])
def test_bf16_logits_past_fp32_resolution(k, splits):
    """q multiplied by 2^k (exact in bf16): the scores reach about 2^(k + 4) in log2 units, where a
    fused score * cq - ref exceeds 0 by up to half an ulp of the reference (p = inf once that passes
    2^7).  The first pass sends an overflowed sum to the repeat, which rounds each product before
    subtracting the exact max, so every p <= 1; the weights are then one-hot to fp32 precision and the
    output matches the oracle's to 2e-3 of each row's largest output.  The LSE is held to 1e-6 of
    |lse| (the relative precision of the fp32 scores it comes from)."""
    w = make_random(4100 + k, T=6, H=64, K=500, ctx=900, B=32, neg_frac=0.1, n_req=2, kv="bf16")
    q = w.q_f32() * np.float32(2.0 ** k)
    w.q_bits = torch.from_numpy(np.ascontiguousarray(q)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    out, lse = smla.decode(q_dev(w), w.cache.to_device("cuda"), dev(slots), w.sm_scale, out_dtype=torch.float32,
                           kv_layout="bf16", num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale, record_layout="bf16")
    o, l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin) and np.abs(rl[fin]).max() > 2.0 ** k
    for t in range(w.T):
        big = np.abs(ro[t]).max()
        d = np.abs(o[t] - ro[t]).max()
        print(f"  2^{k} splits {splits} row {t}: max|out| {big:.3e} max|dout|/max|out| {d / big:.2e}", flush=True)
        assert d <= 2e-3 * big
    dl = np.abs(l[fin] - rl[fin])
    print(f"  2^{k}: max|lse| {np.abs(rl[fin]).max():.3e} max|dlse|/|lse| {(dl / np.abs(rl[fin])).max():.2e}", flush=True)
    assert np.all(dl <= 1e-6 * np.abs(rl[fin]) + 1e-3)
