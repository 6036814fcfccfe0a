"""Cache write and DCP local lengths on the GPU against the oracle: bit-exact bytes and slots."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
import sparse_mla_decode_topk_amd as smla
from tests.gpu_common import check_close, dev, require_gpu

pytestmark = pytest.mark.gpu

POISON = 0xCD


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def as_input(x, dtype):
    """Host fp32 values as the kernel input tensor, and the exact fp32 values it holds."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)
    return t.cuda(), t.float().numpy()


def run_and_check(lat, rope, pos, req, bt, B, num_slots, dtype, D=1, r=0, I=1, what=""):
    print(f"cache write {what}: N={len(pos)} dtype={dtype} D={D} r={r} I={I} B={B}", flush=True)
    lat_d, lat_v = as_input(lat, dtype)
    rope_d, rope_v = as_input(rope, dtype)
    cache = torch.full((num_slots, 656), POISON, dtype=torch.uint8, device="cuda")
    sm = smla.cache_write(lat_d, rope_d, dev(pos, torch.int32), dev(req, torch.int32), dev(bt, torch.int32), cache, B,
                          D, r, I)
    torch.cuda.synchronize()
    rec, ref_sm = O.cache_write(lat_v, rope_v, pos, req, bt, B, num_slots, D, r, I)
    assert np.array_equal(sm.cpu().numpy(), ref_sm), f"{what}: slot mapping differs"
    want = np.full((num_slots, 656), POISON, dtype=np.uint8)
    keep = ref_sm >= 0
    want[ref_sm[keep]] = rec[keep]
    got = cache.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} bytes differ, first at (slot, byte) {tuple(bad[0])}"
    return got, ref_sm


def random_tokens(rng, n, n_req, ctx, B, D, blocks_per_req):
    req = rng.integers(0, n_req, n).astype(np.int32)
    pos = np.empty(n, dtype=np.int32)
    for b in range(n_req):  # distinct positions within a request, so no two tokens share a slot
        idx = np.nonzero(req == b)[0]
        pos[idx] = rng.choice(ctx, size=idx.size, replace=False)
    bt = rng.permutation(n_req * blocks_per_req).reshape(n_req, blocks_per_req).astype(np.int32)
    return pos, req, bt


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D,I", [(1, 1), (2, 1), (4, 1), (4, 2), (3, 5)])
def test_cache_write_random(dtype, D, I):
    rng = np.random.default_rng(10 * D + I)
    n, n_req, ctx, B = 257, 3, 400, 16
    wpr = (ctx // D + I + B - 1) // B + 1  # local blocks per request
    pos, req, bt = random_tokens(rng, n, n_req, ctx, B, D, wpr)
    lat = rng.standard_normal((n, 512)).astype(np.float32) * np.exp2(rng.integers(-8, 8, (n, 1)))
    rope = rng.standard_normal((n, 64)).astype(np.float32)
    owned = 0
    for r in range(D):
        _, sm = run_and_check(lat, rope, pos, req, bt, B, n_req * wpr * B, dtype, D, r, I, what="random")
        owned += int((sm >= 0).sum())
    assert owned == n  # every token lands on exactly one rank


def edge_rows():
    vals = O.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # 126 ties between neighbouring e4m3 values
    rows = np.zeros((4, 512), dtype=np.float64)
    rows[0, 128:256] = -0.0
    rows[0, 256] = 448.0  # scale 1: the tile holds exact ties, which go to the even code
    rows[0, 257:383] = mids
    rows[0, 383] = -mids[40]
    rows[0, 384] = 56.0  # scale 1/8: the same ties, scaled by a power of two
    rows[0, 385:511] = mids / 8
    rows[0, 511] = -mids[3] / 8
    rows[1, 0] = 448.0  # subnormal e4m3 range: multiples of 2^-10, ties between 2^-9 steps
    rows[1, 1:128] = np.arange(1, 128) * 2.0 ** -10 * np.where(np.arange(1, 128) % 3 == 0, -1, 1)
    rows[1, 128:256] = np.linspace(-3, 3, 128)
    rows[1, 256:384] = 1e-3
    rows[1, 384:512] = -7.5
    rows[2] = np.tile([1.0, -1.0, 0.5, 448.0 * 3], 128)  # values above the tile scale's 448 never occur
    rows[3, :128] = 3e-38  # tiny tiles (fp32 keeps them; bf16 rounds them)
    rows[3, 128:256] = np.linspace(-1e30, 1e30, 128)
    rows[3, 256:384] = 1e-40
    rows[3, 384:] = np.geomspace(1e-20, 1e20, 128)
    return rows


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cache_write_edge_tiles(dtype):
    lat = edge_rows().astype(np.float32)
    n = lat.shape[0]
    rope = np.tile(np.array([0.0, -0.0, 1.0 + 2.0 ** -9, 3e-38, -65504.0, 1.00390625, 2.0 ** -133, 1e-3],
                            dtype=np.float32), (n, 8))
    pos = np.arange(n, dtype=np.int32)
    req = np.zeros(n, dtype=np.int32)
    bt = np.array([[1, 0]], dtype=np.int32)
    run_and_check(lat, rope, pos, req, bt, 4, 8, dtype, what="edge tiles")


def near_midpoint_rows():
    """Tiles whose quotients x / scale fall on, or within two fp32 ulps of, every rounding
    midpoint between neighbouring e4m3 values, for several non-power-of-two scales: the
    places where a quotient one ulp off would change the code."""
    vals = O.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    rows = []
    for amax in (313.6, 3.1415927, 1e-3, 1234.5, 0.1, 7.0e-20, 1e-35):  # the last divides directly
        amax = np.float32(amax)
        s = np.float32(np.float64(amax) / 448.0)
        xs = []
        for m in mids:
            c = np.float32(np.float64(m) * np.float64(s))
            for k in range(-2, 3):
                v = c
                for _ in range(abs(k)):
                    v = np.nextafter(v, np.float32(np.inf if k > 0 else -np.inf))
                xs += [v, -v]
        xs = np.array(xs, dtype=np.float32)
        xs = xs[np.abs(xs) <= amax]
        per = 127
        ntiles = (len(xs) + per - 1) // per
        xs = np.concatenate([xs, np.zeros(ntiles * per - len(xs), np.float32)]).reshape(ntiles, per)
        tiles = np.concatenate([np.full((ntiles, 1), amax, np.float32), xs], axis=1)
        pad = (-ntiles) % 4
        tiles = np.concatenate([tiles, np.tile(tiles[:1], (pad, 1))])
        rows.append(tiles.reshape(-1, 512))
    return np.concatenate(rows)


def test_cache_write_near_midpoints():
    lat = near_midpoint_rows()
    n = lat.shape[0]
    rope = np.zeros((n, 64), dtype=np.float32)
    pos = np.arange(n, dtype=np.int32)
    req = np.zeros(n, dtype=np.int32)
    bt = np.arange((n + 3) // 4, dtype=np.int32)[None]  # a one-row table whose row stride numpy sets to 0
    run_and_check(lat, rope, pos, req, bt, 4, 4 * bt.shape[1], torch.float32, what="near midpoints")


def test_cache_write_skips_and_bounds():
    """Negative positions, padded requests, missing blocks and slots past the cache are not written."""
    rng = np.random.default_rng(2)
    lat = rng.standard_normal((10, 512)).astype(np.float32)
    rope = rng.standard_normal((10, 64)).astype(np.float32)
    pos = np.array([-1, 0, 1, 5, 9, 40, 3, 2, 7, 8], dtype=np.int32)
    req = np.array([0, -1, 0, 0, 0, 0, 2, 1, 1, 1], dtype=np.int32)
    bt = np.array([[2, -1, 5], [0, 1, 9]], dtype=np.int32)  # hole, and block 9 lies past num_slots
    _, sm = run_and_check(lat, rope, pos, req, bt, 4, 24, torch.bfloat16, what="skips")
    assert list(sm) == [-1, -1, 9, -1, 21, -1, -1, 2, 7, -1]


def test_cache_write_empty_and_no_mapping():
    cache = torch.full((4, 656), POISON, dtype=torch.uint8, device="cuda")
    e = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    smla.cache_write(e, torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((0,), dtype=torch.int32, device="cuda"),
                     torch.empty((0,), dtype=torch.int32, device="cuda"), dev(np.zeros((1, 1), np.int32)), cache, 4)
    lat = torch.ones((2, 512), dtype=torch.bfloat16, device="cuda")
    rope = torch.ones((2, 64), dtype=torch.bfloat16, device="cuda")
    out = smla.cache_write(lat, rope, dev(np.array([0, 1], np.int32)), dev(np.array([0, 0], np.int32)),
                           dev(np.array([[0]], np.int32)), cache, 4, with_slot_mapping=False)
    torch.cuda.synchronize()
    assert out is None
    c = cache.cpu().numpy()
    assert np.all(c[2:] == POISON) and np.all(c[:2, :512] == 0x7E)  # all-ones tiles: every code is 448


def test_cache_write_then_decode():
    """Tokens written by the kernel, then read back by the decode, against the oracle's attention
    over the oracle-written cache (the two caches are byte-identical)."""
    rng = np.random.default_rng(9)
    n_req, ctx, B, H = 2, 300, 16, 32
    bpr = (ctx + B - 1) // B
    req = np.repeat(np.arange(n_req, dtype=np.int32), ctx)
    pos = np.tile(np.arange(ctx, dtype=np.int32), n_req)
    bt = rng.permutation(n_req * bpr).reshape(n_req, bpr).astype(np.int32)
    lat = rng.standard_normal((n_req * ctx, 512)).astype(np.float32)
    rope = rng.standard_normal((n_req * ctx, 64)).astype(np.float32)
    num_slots = n_req * bpr * B
    cache_np, _ = run_and_check(lat, rope, pos, req, bt, B, num_slots, torch.bfloat16, what="write-then-decode")
    T, K = 6, 128
    ids = np.stack([rng.choice(ctx, K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:, -10:] = -1
    qreq = np.array([0, 1, 0, 1, 1, 0], dtype=np.int32)
    q = torch.randn((T, H, 576), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    slots, _ = smla.convert_index(dev(ids, torch.int32), dev(qreq, torch.int32), dev(bt, torch.int32), B)
    cache = dev(cache_np)
    out, lse = smla.decode(q.cuda(), cache, slots, 192 ** -0.5, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_slots, _ = O.convert_index(ids, qreq, bt, B)
    ref_out, ref_lse = O.attention_rows(q.float().numpy(), ref_slots, cache_np, num_slots, 192 ** -0.5)
    check_close(out, lse, ref_out, ref_lse, what="write-then-decode")


def test_cache_write_prefill_chunk():
    """The measured size: one 32768-token prefill chunk in bf16, every byte checked."""
    rng = np.random.default_rng(4)
    n, B = 32768, 64
    bpr = n // B
    pos = np.arange(n, dtype=np.int32)
    req = np.zeros(n, dtype=np.int32)
    bt = rng.permutation(bpr).reshape(1, bpr).astype(np.int32)
    lat = rng.standard_normal((n, 512)).astype(np.float32)
    rope = rng.standard_normal((n, 64)).astype(np.float32)
    run_and_check(lat, rope, pos, req, bt, B, n, torch.bfloat16, what="prefill chunk")


@pytest.mark.parametrize("D,I", [(1, 1), (2, 1), (4, 1), (8, 1), (4, 2), (3, 7)])
def test_dcp_local_seq_lens(D, I):
    rng = np.random.default_rng(D * 10 + I)
    L = rng.integers(-3, 200000, 1000).astype(np.int32)
    L[:5] = [0, 1, 2, 3, D * I]
    tot = np.zeros(1000, dtype=np.int64)
    for r in range(D):
        got = smla.dcp_local_seq_lens(dev(L), D, r, I)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        assert np.array_equal(got, O.dcp_local_seq_lens(L, D, r, I))
        tot += got
    assert np.array_equal(tot, np.maximum(L, 0))
