"""Whole-context (dense) decode on the GPU against the oracle, per DCP rank and merged."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
import sparse_mla_decode_topk_amd as smla
from tests.gpu_common import check_close, dev, require_gpu
from workload import make_dense

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_dense(w, S, cache_np, bt, D=1, r=0, out_dtype=torch.float32, max_seq_len=None):
    q = w.q_torch().cuda()
    seq = dev(w.ctx.astype(np.int32))
    mx = int(w.ctx.max()) if max_seq_len is None else max_seq_len
    out, lse = smla.dense_decode(q, dev(cache_np), dev(bt, torch.int32), seq, S, w.sm_scale, w.block_size, mx, D, r,
                                 out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    dict(seed=1, n_req=3, S=2, H=32, ctx=[300, 37, 1], B=16),
    dict(seed=2, n_req=4, S=4, H=128, ctx=[2100, 700, 64, 3], B=64),  # a row list longer than one split
    dict(seed=3, n_req=2, S=1, H=16, ctx=[129, 0], B=32),  # plain decode, and an empty request
    dict(seed=4, n_req=2, S=1, H=16, ctx=[10000, 4097], B=64),  # lists longer than one workgroup compacts
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}S{c['S']}H{c['H']}")
def test_dense_unsharded(case):
    c = dict(case)
    S = c["S"]
    w = make_dense(c.pop("seed"), **c)
    print(f"dense unsharded: T={w.T} H={w.H} S={S} ctx={list(w.ctx)}", flush=True)
    cache = w.cache.dense()
    out, lse = run_dense(w, S, cache, w.block_table)
    ref_o, ref_l = O.dense_decode(w.q_f32(), w.cache, w.cache.num_slots, w.block_table, w.ctx, S, w.block_size,
                                  w.sm_scale)
    check_close(out, lse, ref_o, ref_l, what="dense")


@pytest.mark.parametrize("D", [2, 4])
def test_dense_dcp_shards_and_merge(D):
    S = 2
    w = make_dense(40 + D, n_req=3, S=S, H=64, ctx=[999, 130, 2], B=16, D=D)
    print(f"dense DCP{D}: T={w.T} H={w.H}", flush=True)
    outs, lses = [], []
    for sh in w.shards:
        o, l = run_dense(w, S, sh.cache.dense(), sh.block_table, D, sh.rank)
        ref_o, ref_l = O.dense_decode(w.q_f32(), sh.cache, sh.cache.num_slots, sh.block_table, w.ctx, S, w.block_size,
                                      w.sm_scale, dcp_size=D, dcp_rank=sh.rank)
        check_close(o, l, ref_o, ref_l, what=f"dense shard {sh.rank}")
        outs.append(o)
        lses.append(l)
    mo, ml = smla.merge_lse(torch.stack(outs), torch.stack(lses), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_l = O.dense_decode(w.q_f32(), w.cache, w.cache.num_slots, w.block_table, w.ctx, S, w.block_size,
                                  w.sm_scale)
    check_close(mo, ml, ref_o, ref_l, what=f"dense DCP{D} merged")


def test_dense_matches_topk_path_and_slack():
    """The dense call matches the top-k call fed every causal position (same kernel, lists built
    on the GPU instead of converted), and a max_seq_len well above the longest context (longer
    lists, padded with -1, and another split plan) still gives the oracle's result."""
    S = 4
    w = make_dense(7, n_req=3, S=S, H=64, ctx=[515, 64, 5], B=64)
    cache = w.cache.dense()
    o1, l1 = run_dense(w, S, cache, w.block_table, out_dtype=torch.bfloat16)
    o2, l2 = run_dense(w, S, cache, w.block_table, out_dtype=torch.bfloat16, max_seq_len=4000)
    slots, _ = smla.convert_index(dev(w.ids), dev(w.req), dev(w.block_table), w.block_size)
    o3, l3 = smla.decode(w.q_torch().cuda(), dev(cache), slots, w.sm_scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref_o, ref_l = O.dense_decode(w.q_f32(), w.cache, w.cache.num_slots, w.block_table, w.ctx, S, w.block_size,
                                  w.sm_scale)
    check_close(o1, l1, ref_o, ref_l, what="dense bf16")
    check_close(o2, l2, ref_o, ref_l, what="dense bf16, max_seq_len 4000")
    assert torch.equal(o1, o3) and torch.equal(l1, l3)  # same lists, same plan: same bits
    check_close(o3, l3, ref_o, ref_l, what="top-k with every causal id")


def test_dense_bench_size_sampled():
    """The measured size (32 requests x 4 MTP tokens, H = 128, context 4096): sampled rows
    against the oracle one by one."""
    S = 4
    w = make_dense(11, n_req=32, S=S, H=128, ctx=4096, B=64)
    out, lse = run_dense(w, S, w.cache.dense(), w.block_table, out_dtype=torch.bfloat16)
    rows = [0, 3, 57, 127]
    sub = w.rows(rows)
    slots, _ = O.convert_index(sub.ids, sub.req, sub.block_table, sub.block_size)
    ref_o, ref_l = O.attention_rows(sub.q_f32(), slots, sub.cache, sub.cache.num_slots, sub.sm_scale)
    check_close(out[rows], lse[rows], ref_o, ref_l, what="dense bench size")
    assert not torch.isnan(out).any() and torch.isfinite(lse).all()
