"""Index conversion on the GPU against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
import sparse_mla_decode_topk_amd as smla
from tests.gpu_common import dev, require_gpu
from workload import make_config, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_convert(ids, req, bt, B, D=1, r=0, I=1):
    slots, valid = smla.convert_index(dev(ids, torch.int32), dev(req, torch.int32), dev(bt, torch.int32), B, D, r, I)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), valid.cpu().numpy()


def assert_exact(ids, req, bt, B, D=1, r=0, I=1):
    got_s, got_v = run_convert(ids, req, bt, B, D, r, I)
    ref_s, ref_v = O.convert_index(ids, req, bt, B, D, r, I)
    assert np.array_equal(got_s, ref_s)
    assert np.array_equal(got_v, ref_v)


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_convert_configs(cid):
    w = make_config(cid)
    print(f"convert config {cid}: T={w.T} K={w.K} D={w.dcp_size}", flush=True)
    assert_exact(w.ids, w.req, w.block_table, w.block_size)
    for sh in w.shards:
        assert_exact(w.ids, w.req, sh.block_table, w.block_size, w.dcp_size, sh.rank)


@pytest.mark.parametrize("D,I,B", [(1, 1, 64), (2, 1, 16), (4, 1, 64), (8, 1, 64), (2, 2, 16), (4, 3, 100), (3, 1, 1)])
def test_convert_random(D, I, B):
    rng = np.random.default_rng(100 * D + I)
    T, K, R, W = 37, 300, 5, 20
    ids = rng.integers(-3, W * B * D + 50, size=(T, K)).astype(np.int32)  # negatives and ids past the table
    req = rng.integers(-1, R + 1, size=T).astype(np.int32)  # padded rows and requests past the table
    bt = rng.integers(-1, 1000, size=(R, W)).astype(np.int32)  # holes in the block table
    for r in range(D):
        assert_exact(ids, req, bt, B, D, r, I)


def test_convert_valid_counts_partition_c2():
    w = make_config(2)
    tot = 0
    for sh in w.shards:
        _, v = run_convert(w.ids, w.req, sh.block_table, w.block_size, w.dcp_size, sh.rank)
        tot = tot + v
    assert np.array_equal(tot, (w.ids >= 0).sum(axis=1))
    # the four ctx-2 rows: shards 2 and 3 hold nothing
    for sh in w.shards[2:]:
        _, v = run_convert(w.ids, w.req, sh.block_table, w.block_size, w.dcp_size, sh.rank)
        assert np.all(v[32:] == 0)


def test_convert_misaligned_and_in_place():
    rng = np.random.default_rng(5)
    T, K, B = 9, 33, 16
    ids = rng.integers(-1, 400, size=(T, K)).astype(np.int32)
    req = rng.integers(0, 3, size=T).astype(np.int32)
    bt = rng.permutation(3 * 25).reshape(3, 25).astype(np.int32)
    ref_s, ref_v = O.convert_index(ids, req, bt, B, 2, 1)
    # 4-byte and 12-byte offsets into packed buffers
    big = torch.zeros(T * (K + 1) + 3, dtype=torch.int32, device="cuda")
    ids_v = big[1:1 + T * (K + 1)].view(T, K + 1)[:, :K]
    ids_v.copy_(dev(ids))
    packed = torch.zeros(3 + T, dtype=torch.int32, device="cuda")
    req_v = packed[3:]
    req_v.copy_(dev(req))
    out_big = torch.zeros(T * K + 1, dtype=torch.int32, device="cuda")
    out_v = out_big[1:].view(T, K)
    s, v = smla.convert_index(ids_v, req_v, dev(bt), B, 2, 1, out=out_v)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), ref_s) and np.array_equal(v.cpu().numpy(), ref_v)
    # in place: slots written over the ids
    ids_t = dev(ids)
    s, v = smla.convert_index(ids_t, dev(req), dev(bt), B, 2, 1, out=ids_t)
    torch.cuda.synchronize()
    assert np.array_equal(ids_t.cpu().numpy(), ref_s)


def test_convert_empty_and_degenerate():
    # T = 0 and K = 0 are no-ops; one entry rows
    z = torch.zeros((0, 8), dtype=torch.int32, device="cuda")
    s, _ = smla.convert_index(z, torch.zeros(0, dtype=torch.int32, device="cuda"),
                              torch.zeros((1, 1), dtype=torch.int32, device="cuda"), 64)
    assert s.shape == (0, 8)
    ids = np.zeros((4, 0), dtype=np.int32)
    s, v = run_convert(ids, np.zeros(4, np.int32), np.zeros((1, 1), np.int32), 64)
    assert s.shape == (4, 0) and np.all(v == 0)
    w = make_random(77, T=3, H=16, K=1, ctx=10, B=4)
    assert_exact(w.ids, w.req, w.block_table, 4)
