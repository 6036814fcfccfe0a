"""The cache write, the whole-context decode and the bf16-record decode captured in one HIP graph:
every replay equals the eager result (the calls allocate nothing, synchronise nothing and record
kernel nodes only, so the graph can be replayed as is)."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
import sparse_mla_decode_topk_amd as smla
from tests.gpu_common import check_close, dev, q_dev, require_gpu
from workload import make_dense, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_graph_of_cache_write_dense_and_bf16_decode():
    rng = np.random.default_rng(8)
    # cache write inputs
    n, B = 96, 16
    lat = torch.from_numpy(rng.standard_normal((n, 512)).astype(np.float32)).to(torch.bfloat16).cuda()
    rope = torch.from_numpy(rng.standard_normal((n, 64)).astype(np.float32)).to(torch.bfloat16).cuda()
    pos = dev(np.arange(n, dtype=np.int32))
    req = dev(np.zeros(n, dtype=np.int32))
    wbt = dev(rng.permutation(n // B).astype(np.int32)[None])
    wcache = torch.full((n, 656), 0xCD, dtype=torch.uint8, device="cuda")
    smap = torch.empty((n,), dtype=torch.int32, device="cuda")
    # dense decode inputs (a context longer than one split)
    S = 2
    wd = make_dense(3, n_req=2, S=S, H=64, ctx=[4500, 300], B=64)
    dq, dcache = q_dev(wd), wd.cache.to_device("cuda")
    dbt, dseq = dev(wd.block_table), dev(wd.ctx.astype(np.int32))
    dout = torch.empty((wd.T, wd.H, 512), dtype=torch.float32, device="cuda")
    dlse = torch.empty((wd.T, wd.H), dtype=torch.float32, device="cuda")
    # bf16-record decode inputs (three splits per row)
    wb = make_random(12, T=6, H=32, K=600, ctx=800, B=32, neg_frac=0.2, n_req=2, kv="bf16")
    bslots, _ = O.convert_index(wb.ids, wb.req, wb.block_table, wb.block_size)
    bq, bcache, bsl = q_dev(wb), wb.cache.to_device("cuda"), dev(bslots)
    bout = torch.empty((wb.T, wb.H, 512), dtype=torch.bfloat16, device="cuda")
    blse = torch.empty((wb.T, wb.H), dtype=torch.float32, device="cuda")
    bws = torch.empty(smla.decode_workspace_size(wb.T, wb.H, wb.K, 3) + 256, dtype=torch.uint8, device="cuda")

    def work():
        smla.cache_write(lat, rope, pos, req, wbt, wcache, B, slot_mapping=smap)
        smla.dense_decode(dq, dcache, dbt, dseq, S, wd.sm_scale, wd.block_size, int(wd.ctx.max()), out=dout, lse=dlse)
        smla.decode(bq, bcache, bsl, wb.sm_scale, out=bout, lse=blse, num_splits=3, workspace=bws, kv_layout="bf16")

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (wcache, smap, dout, dlse, bout, blse)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        wcache.fill_(0xCD)
        smap.fill_(-7)
        for t in (dout, dlse, bout, blse):
            t.fill_(123.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("cache", "slot map", "dense out", "dense lse", "bf16 out", "bf16 lse"),
                                   (wcache, smap, dout, dlse, bout, blse), eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
    ref_o, ref_l = O.dense_decode(wd.q_f32(), wd.cache, wd.cache.num_slots, wd.block_table, wd.ctx, S, wd.block_size,
                                  wd.sm_scale)
    check_close(dout, dlse, ref_o, ref_l, what="dense in graph")
    ref_o, ref_l = O.attention_rows(wb.q_f32(), bslots, wb.cache, wb.cache.num_slots, wb.sm_scale,
                                    record_layout="bf16")
    check_close(bout, blse, ref_o, ref_l, what="bf16 decode in graph")
