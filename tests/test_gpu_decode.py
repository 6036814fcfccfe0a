"""Sparse MLA decode on the GPU against the fp64 oracle (max |dout| <= 2e-2, max |dlse| <= 1e-3)."""
import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
import sparse_mla_decode_topk_amd as smla
from tests.gpu_common import check_close, dev, oracle_unsharded, q_dev, require_gpu
from workload import make_config, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_decode(w, slots_np=None, out_dtype=None, num_splits=0, lse_layout="TH", cache=None):
    if slots_np is None:
        slots_np, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    cache = w.cache.to_device("cuda") if cache is None else cache
    od = out_dtype or (torch.float32 if w.out_dtype == "fp32" else torch.bfloat16)
    out, lse = smla.decode(q_dev(w), cache, dev(slots_np), w.sm_scale, out_dtype=od, num_splits=num_splits,
                           lse_layout=lse_layout)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("cid", [0, 1])
def test_decode_config(cid):
    w = make_config(cid)
    print(f"decode config {cid}: T={w.T} H={w.H} K={w.K}", flush=True)
    out, lse = gpu_decode(w)
    ref_o, ref_l = oracle_unsharded(w)
    do, dl = check_close(out, lse, ref_o, ref_l, what=w.name)
    print(f"  max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)


@pytest.mark.parametrize("H", [16, 32, 48, 64, 96, 128])
@pytest.mark.parametrize("K,neg", [(1, 0.0), (7, 0.0), (64, 0.3), (100, 0.5), (2048, 0.1)])
def test_decode_random_shapes(H, K, neg):
    w = make_random(1000 + H + K, T=5, H=H, K=K, ctx=max(2 * K, 64), B=64, neg_frac=neg, n_req=2)
    print(f"decode random H={H} K={K} neg={neg}", flush=True)
    out, lse = gpu_decode(w, out_dtype=torch.float32)
    ref_o, ref_l = oracle_unsharded(w)
    check_close(out, lse, ref_o, ref_l, what=f"H{H}K{K}")


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_forced_splits(splits, dtype):
    w = make_random(2000 + splits, T=6, H=64, K=700, ctx=1500, B=64, neg_frac=0.2, n_req=3)
    print(f"decode splits={splits} dtype={dtype}", flush=True)
    out, lse = gpu_decode(w, out_dtype=dtype, num_splits=splits)
    ref_o, ref_l = oracle_unsharded(w)
    check_close(out, lse, ref_o, ref_l, what=f"splits{splits}")


def test_decode_split_ranges_with_empty_splits():
    # valid entries only in the first quarter: later splits see nothing and must drop out
    w = make_random(31, T=4, H=128, K=1024, ctx=4096, B=64, n_req=2)
    w.ids[:, 256:] = -1
    out, lse = gpu_decode(w, out_dtype=torch.float32, num_splits=4)
    ref_o, ref_l = oracle_unsharded(w)
    check_close(out, lse, ref_o, ref_l, what="empty splits")


def test_decode_empty_rows_and_out_of_range_slots():
    w = make_random(41, T=6, H=64, K=64, ctx=200, B=16, n_req=2)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    slots[1, :] = -1  # empty row
    slots[2, :] = w.cache.num_slots + 5  # only out-of-range entries: empty too
    slots[3, ::2] = -7  # other negatives
    slots[4, 3] = w.cache.num_slots  # one out-of-range entry among valid ones
    for splits in (1, 3):
        out, lse = gpu_decode(w, slots_np=slots, out_dtype=torch.float32, num_splits=splits)
        ref_o, ref_l = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale)
        check_close(out, lse, ref_o, ref_l, what=f"empty rows s{splits}")
        l = lse.cpu().numpy()
        assert np.all(np.isneginf(l[1])) and np.all(np.isneginf(l[2]))
        assert torch.all(out[1] == 0) and torch.all(out[2] == 0)


def test_decode_k_zero_and_t_zero():
    w = make_random(51, T=3, H=32, K=4, ctx=40, B=16)
    slots = np.zeros((3, 0), dtype=np.int32)
    out, lse = gpu_decode(w, slots_np=slots)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    q = torch.zeros((0, 32, 576), dtype=torch.bfloat16, device="cuda")
    o, l = smla.decode(q, w.cache.to_device("cuda"), torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 0.1)
    assert o.shape == (0, 32, 512)


def test_decode_duplicates_count_twice():
    w = make_random(61, T=3, H=16, K=12, ctx=60, B=16)
    w.ids[0, 1] = w.ids[0, 0]
    w.ids[1, :] = w.ids[1, 0]
    out, lse = gpu_decode(w, out_dtype=torch.float32)
    ref_o, ref_l = oracle_unsharded(w)
    check_close(out, lse, ref_o, ref_l, what="duplicates")


def test_lse_layouts_agree_bitwise():
    w = make_random(71, T=9, H=128, K=256, ctx=1024, B=64, neg_frac=0.2, n_req=3)
    cache = w.cache.to_device("cuda")
    o1, l1 = gpu_decode(w, lse_layout="TH", cache=cache)
    o2, l2 = gpu_decode(w, lse_layout="HT", cache=cache)
    assert l2.stride() == (1, 9)
    assert torch.equal(l1, l2) and torch.equal(o1, o2)
    # the (1, H, T) -> (T, H) transpose of the native layout matches the oracle's reading
    native = l2.t().contiguous().cpu().numpy()[None]
    assert np.array_equal(O.transpose_hT_lse(native), l1.cpu().numpy())


def test_decode_strided_q_and_out():
    w = make_random(81, T=4, H=64, K=128, ctx=512, B=64)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    qbig = torch.zeros((4, 80, 576 + 64), dtype=torch.bfloat16, device="cuda")
    qv = qbig[:, 8:72, :576]
    qv.copy_(q_dev(w))
    obig = torch.full((4, 70, 520), 7.0, dtype=torch.float32, device="cuda")
    ov = obig[:, 3:67, :512]
    out, lse = smla.decode(qv, w.cache.to_device("cuda"), dev(slots), w.sm_scale, out=ov)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_unsharded(w)
    check_close(ov, lse, ref_o, ref_l, what="strided")
    assert torch.all(obig[:, :3] == 7.0) and torch.all(obig[:, :, 512:] == 7.0)


def test_decode_repeat_is_deterministic():
    w = make_random(91, T=8, H=128, K=512, ctx=2048, B=64, n_req=2)
    cache = w.cache.to_device("cuda")
    a = gpu_decode(w, cache=cache, num_splits=4)
    b = gpu_decode(w, cache=cache, num_splits=4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _late_dominant(kv):
    """A row whose head 0 meets, in the 11th 32-entry tile of its list, a record equal to that head's own
    (unscaled) query: its score then exceeds every score of the first tile by ~200 in log2 units, far past the
    kernels' fixed-reference headroom (2^12 for fp8_ds_mla records, 2^64 for bf16 records), so the workgroup
    redoes its range with the exact max."""
    from workload import pack_records, pack_records_bf16
    w = make_random(321, T=3, H=32, K=400, ctx=600, B=16, n_req=1, kv=kv)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    row, e = 1, 330
    slot = int(slots[row, e])
    assert slot >= 0
    q = w.q_f32()
    base = q[row, 0].copy()
    q[row, 0] *= 4.0  # exact in bf16
    w.q_bits = torch.from_numpy(np.ascontiguousarray(q)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pack = pack_records if kv == "fp8_ds_mla" else pack_records_bf16
    i = int(np.searchsorted(w.cache.real_slots, slot))
    assert w.cache.real_slots[i] == slot
    w.cache.records[i] = pack(base[None, :512], base[None, 512:])[0]
    return w, slots


@pytest.mark.parametrize("kv", ["fp8_ds_mla", "bf16"])
@pytest.mark.parametrize("splits", [1, 3])
def test_decode_late_dominant_score_exceeds_headroom(kv, splits):
    w, slots = _late_dominant(kv)
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale, record_layout=kv)
    # the pinned case: head 0 of row 1 is dominated by the planted record (p ~ 1, a log-sum-exp far above
    # the first tile's scores)
    assert rl[1, 0] > 100.0 and np.abs(ro[1, 0]).max() < 8.0
    out, lse = smla.decode(q_dev(w), w.cache.to_device("cuda"), dev(slots), w.sm_scale, out_dtype=torch.float32,
                           num_splits=splits, kv_layout=kv)
    torch.cuda.synchronize()
    check_close(out, lse, ro, rl, what=f"late dominant {kv} splits {splits}")


@pytest.mark.parametrize("splits", [1, 3])
def test_decode_late_record_scale_overflows_fp16(splits):
    """The output MFMAs take p * scale in fp16.  Row 1 (query latent set to zero, so every score is a
    rope product of moderate size) meets, in its 11th tile, a record whose latent values are 2^12 times
    larger than any of the first tile's and whose rope equals head 0's query rope: its p stays inside
    the score headroom, but p * scale overflows fp16, the value waves vote to repeat the range, and the
    repeat scales by the largest record scale of the whole range.  Rows 0 and 2 keep the 2e-2 / 1e-3
    bars; row 1's values reach ~2^14, so its outputs are held to 2e-3 of their largest magnitude."""
    from workload import pack_records
    w = make_random(322, T=3, H=32, K=400, ctx=600, B=16, n_req=1)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    row = 1
    elsewhere = set(slots[0].tolist()) | set(slots[2].tolist())  # the planted record stays out of rows 0, 2
    e = next(j for j in range(300, w.K) if slots[row, j] >= 0 and int(slots[row, j]) not in elsewhere)
    slot = int(slots[row, e])
    assert int((slots[row, :e] >= 0).sum()) >= 64  # at least two tiles before it
    q = w.q_f32()
    q[row, :, :512] = 0.0
    w.q_bits = torch.from_numpy(np.ascontiguousarray(q)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    i = int(np.searchsorted(w.cache.real_slots, slot))
    assert w.cache.real_slots[i] == slot
    lat = np.random.default_rng(5).standard_normal((1, 512)).astype(np.float32) * np.float32(4096.0)
    w.cache.records[i] = pack_records(lat, q[row, 0, 512:][None, :])[0]
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale)
    out, lse = smla.decode(q_dev(w), w.cache.to_device("cuda"), dev(slots), w.sm_scale, out_dtype=torch.float32,
                           num_splits=splits)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    big = np.abs(ro[row]).max()
    assert big > 1000.0  # the planted record carries real weight in row 1
    print(f"  row 1 max|out| {big:.1f} max|dout| {np.abs(o[row] - ro[row]).max():.3e} "
          f"max|dlse| {np.abs(l[row] - rl[row]).max():.3e}", flush=True)
    assert np.abs(o[row] - ro[row]).max() <= 2e-3 * big
    assert np.abs(l[row] - rl[row]).max() <= 1e-3
    others = [0, 2]
    check_close(out[others], lse[others], ro[others], rl[others], what=f"scale overflow rows 0, 2 splits {splits}")


@pytest.mark.parametrize("mode", ["tiny", "huge", "mixed"])
def test_decode_record_scales_far_from_one(mode):
    """The fp16 products p * scale are shifted by the exponent of the first tile's largest record
    scale: record scales multiplied by 2^-60 or 2^60 (every record), or half of the records by 2^30
    and the rest by 2^-30 (a range fp16 cannot hold at once: the small ones underflow), must give
    the oracle's result to fp16 precision relative to the row's largest output.  The query's
    latent part is zero, so the scores (rope only) stay moderate and the LSE keeps the 1e-3 bar."""
    w = make_random(323, T=4, H=32, K=300, ctx=500, B=16, n_req=2)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    q = w.q_f32()
    q[:, :, :512] = 0.0
    w.q_bits = torch.from_numpy(np.ascontiguousarray(q)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rec = w.cache.records
    sc = rec[:, 512:528].copy().view("<f4")  # [n, 4] record scales
    n = rec.shape[0]
    if mode == "tiny":
        f = np.full(n, 2.0 ** -60, np.float32)
    elif mode == "huge":
        f = np.full(n, 2.0 ** 60, np.float32)
    else:
        f = np.where(np.arange(n) % 2 == 0, np.float32(2.0 ** 30), np.float32(2.0 ** -30))
    rec[:, 512:528] = (sc * f[:, None]).astype("<f4").view(np.uint8)  # powers of two: exact
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale)
    out, lse = smla.decode(q_dev(w), w.cache.to_device("cuda"), dev(slots), w.sm_scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    for t in range(w.T):
        big = np.abs(ro[t]).max()
        d = np.abs(o[t] - ro[t]).max()
        print(f"  {mode} row {t}: max|out| {big:.3e} max|dout|/max|out| {d / big:.2e}", flush=True)
        assert d <= 2e-3 * big
    assert np.abs(l - rl).max() <= 1e-3


@pytest.mark.parametrize("seed,T,H,K,ctx,B,n_req,neg,splits,k", [
    (10195, 5, 128, 537, 221, 16, 2, 0.0, 0, 25),
    (10133, 6, 16, 1071, 1564, 64, 3, 0.0, 5, 26),
    (10092, 2, 96, 1826, 2089, 64, 1, 0.5, 3, 29),
])
def test_decode_logits_past_fp32_resolution(seed, T, H, K, ctx, B, n_req, neg, splits, k):
    """Every record scale multiplied by 2^k with the query kept whole: the scores reach 2^28 .. 2^33
    in log2 units, where an fp32 score is a multiple of 16 .. 512 and the weights are close to one-hot.
    A fused score * cq - ref may then exceed 0 by half an ulp of the reference (p up to 2^256); the
    repeated range rounds the product first, so every p <= 1 and the output stays finite and, the
    largest scores being well apart here, matches the oracle to fp16 precision relative to each row's
    largest output.  The LSE is held to the relative precision of the fp32 scores it comes from
    (1e-6 of |lse|, i.e. about 16 units of fp32 rounding)."""
    w = make_random(seed, T=T, H=H, K=K, ctx=ctx, B=B, neg_frac=neg, n_req=n_req)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    rec = w.cache.records
    sc = rec[:, 512:528].copy().view("<f4")
    rec[:, 512:528] = (sc * np.float32(2.0 ** k)).astype("<f4").view(np.uint8)  # a power of two: exact
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale)
    out, lse = smla.decode(q_dev(w), w.cache.to_device("cuda"), dev(slots), w.sm_scale, out_dtype=torch.float32,
                           num_splits=splits)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin) and np.all(o[~fin] == 0.0)
    assert np.abs(rl[fin]).max() > 1e8
    for t in range(w.T):
        if not fin[t].any():
            continue
        big = np.abs(ro[t]).max()
        d = np.abs(o[t] - ro[t]).max()
        print(f"  2^{k} row {t}: max|out| {big:.3e} max|dout|/max|out| {d / big:.2e}", flush=True)
        assert d <= 2e-3 * big
    dl = np.abs(l[fin] - rl[fin])
    print(f"  2^{k}: max|lse| {np.abs(rl[fin]).max():.3e} max|dlse|/|lse| {(dl / np.abs(rl[fin])).max():.2e}", flush=True)
    assert np.all(dl <= 1e-6 * np.abs(rl[fin]) + 1e-3)


@pytest.mark.parametrize("splits", [1, 3])
def test_decode_query_ranges_per_head(splits):
    """Heads of q scaled by powers of two from 2^-110 to 2^3, and one all-zero head: q enters the
    score products as given (bf16), so tiny and zero heads must match as well as the others (their
    scores sit near 0 and their softmax is nearly uniform)."""
    import dataclasses

    w = make_random(91, T=5, H=64, K=300, ctx=700, B=64, neg_frac=0.1, n_req=2)
    q = w.q_f32().copy()
    exps = [-110, -30, -12, -4, 0, 3]
    for h in range(w.H):
        q[:, h, :] *= np.float32(2.0 ** exps[h % len(exps)])
    q[:, 7, :] = 0.0
    bits = q.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "power-of-two scaling keeps the values bf16"
    w = dataclasses.replace(w, q_bits=(bits >> 16).astype(np.uint16))
    print(f"decode query ranges splits={splits}", flush=True)
    out, lse = gpu_decode(w, out_dtype=torch.float32, num_splits=splits)
    ref_o, ref_l = oracle_unsharded(w)
    check_close(out, lse, ref_o, ref_l, what=f"q ranges s{splits}")


@pytest.mark.parametrize("splits", [0, 3, 5])
def test_decode_list_longer_than_one_workgroup(splits):
    """K = 9000 exceeds the 4096 slot entries one workgroup compacts: the call splits the list
    itself (at least three ranges), or takes the forced count when that is enough."""
    w = make_random(97, T=3, H=64, K=9000, ctx=20000, B=64, neg_frac=0.05, n_req=1)
    print(f"decode K=9000 splits={splits}", flush=True)
    out, lse = gpu_decode(w, out_dtype=torch.float32, num_splits=splits)
    ref_o, ref_l = oracle_unsharded(w)
    check_close(out, lse, ref_o, ref_l, what=f"K9000 s{splits}")


def test_decode_longest_list():
    """The longest list a call takes: 64 ranges of 4096 entries (K = 262144), one row, 16 heads."""
    w = make_random(98, T=1, H=16, K=262144, ctx=262244, B=64, neg_frac=0.05, n_req=1)
    print("decode K=262144", flush=True)
    out, lse = gpu_decode(w, out_dtype=torch.float32)
    ref_o, ref_l = oracle_unsharded(w)
    check_close(out, lse, ref_o, ref_l, what="K262144")


def _wide_range_q(w, seed):
    """q whose values inside each head span a wide range: one or two dims per (row, head) at
    +-2^5 .. 2^7 and every other dim +-2^u with u uniform in [-14, -2], all exact in bf16.  Small
    values next to a large one are where any narrower encoding of q (two e4m3 terms under one
    range factor per head, say) stops being exact; the bf16 score products must not care."""
    import dataclasses

    rng = np.random.default_rng(seed)
    T, H = w.T, w.H
    mag = np.exp2(rng.uniform(-14.0, -2.0, size=(T, H, 576)))
    q = (mag * rng.choice([-1.0, 1.0], size=mag.shape)).astype(np.float32)
    for t in range(T):
        for h in range(H):
            for d in rng.choice(576, size=int(rng.integers(1, 3)), replace=False):
                q[t, h, d] = np.float32(rng.choice([-1.0, 1.0]) * np.exp2(rng.uniform(5.0, 7.0)))
    bits = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return dataclasses.replace(w, q_bits=bits)


@pytest.mark.parametrize("kv", ["fp8_ds_mla", "bf16"])
@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("splits", [1, 3])
def test_decode_query_range_within_head(kv, H, splits):
    w = _wide_range_q(make_random(131 + H, T=6, H=H, K=400, ctx=900, B=64, neg_frac=0.1, n_req=2, kv=kv), 7 + H)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    print(f"decode wide-range q kv={kv} H={H} splits={splits}", flush=True)
    out, lse = smla.decode(q_dev(w), w.cache.to_device("cuda"), dev(slots), w.sm_scale, out_dtype=torch.float32,
                           num_splits=splits, kv_layout=kv)
    torch.cuda.synchronize()
    ref_o, ref_l = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale, record_layout=kv)
    do, dl = check_close(out, lse, ref_o, ref_l, what=f"wide-range q {kv} H{H} s{splits}")
    print(f"  max|dout|={do:.2e} max|dlse|={dl:.2e}", flush=True)


@pytest.mark.parametrize("kv", ["fp8_ds_mla", "bf16"])
@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("splits", [1, 3])
def test_decode_valid_count_matches_slots(kv, H, splits):
    """Counts from the conversion change nothing but skip the rows they mark empty: with and without
    them the results are bitwise equal; a row counted 0 is (0, -inf) even if its slots hold entries."""
    w = make_random(141 + H, T=9, H=H, K=300, ctx=700, B=64, neg_frac=0.2, n_req=3, kv=kv)
    w.ids[2, :] = -1
    w.ids[5, :] = -1
    slots, counts = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    cache = w.cache.to_device("cuda")
    ds = dev(slots)
    a = smla.decode(q_dev(w), cache, ds, w.sm_scale, out_dtype=torch.float32, num_splits=splits, kv_layout=kv)
    b = smla.decode(q_dev(w), cache, ds, w.sm_scale, out_dtype=torch.float32, num_splits=splits, kv_layout=kv,
                    valid_count=dev(counts.astype(np.int32)))
    torch.cuda.synchronize()
    assert counts[2] == 0 and counts[5] == 0
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    forced = counts.astype(np.int32).copy()
    forced[7] = 0  # a row the caller marks empty: its slots are not read
    o, l = smla.decode(q_dev(w), cache, ds, w.sm_scale, out_dtype=torch.bfloat16, num_splits=splits, kv_layout=kv,
                       valid_count=dev(forced))
    torch.cuda.synchronize()
    assert torch.all(o[7] == 0) and torch.all(torch.isneginf(l[7]))
    keep = [t for t in range(w.T) if t != 7]
    assert torch.equal(l[keep], a[1][keep])


@pytest.mark.parametrize("case", range(48))
def test_decode_random_sweep(case):
    """Seeded random combinations: T 1-8, H a multiple of 16 up to 128, K 1-3000 over contexts of
    40-3000 tokens, -1 shares 0-0.9, 1-5 forced splits or the automatic plan, block sizes 16/64,
    and one of: plain records, every record scale times its own power of two in [2^-20, 2^20], all
    scales times one power of two in [2^-30, 2^30], 2 % of the records 2^8 larger; a quarter of
    the cases zero the query's latent part.  Bars: the 2e-2 / 1e-3 of the other tests; where the
    scales are rescaled, out within 2e-3 of the largest output when that is larger (fp16 products,
    as in test_decode_record_scales_far_from_one), and the LSE within 1e-6 of its magnitude when
    the rescaled scores pass 1000 (the precision of the fp32 scores it comes from)."""
    rng = np.random.default_rng(7000 + case)
    T = int(rng.integers(1, 9))
    H = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    ctx = int(rng.integers(40, 3001))
    K = int(rng.integers(1, 3001))
    neg = float(rng.choice([0.0, 0.1, 0.5, 0.9]))
    splits = int(rng.choice([0, 1, 2, 3, 5]))
    mode = int(rng.integers(0, 4))
    zero_lat = bool(rng.integers(0, 4) == 0)
    B = int(rng.choice([16, 64]))
    n_req = int(rng.integers(1, T + 1))
    w = make_random(8000 + case, T=T, H=H, K=K, ctx=ctx, B=B, neg_frac=neg, n_req=n_req)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    if mode:
        rec = w.cache.records
        sc = rec[:, 512:528].copy().view("<f4")
        n = rec.shape[0]
        if mode == 1:
            f = np.float32(2.0) ** rng.integers(-20, 21, size=n).astype(np.float32)
        elif mode == 2:
            f = np.full(n, np.float32(2.0) ** int(rng.integers(-30, 31)), np.float32)
        else:
            f = np.where(rng.random(n) < 0.02, np.float32(256.0), np.float32(1.0))
        rec[:, 512:528] = (sc * f[:, None]).astype("<f4").view(np.uint8)  # powers of two: exact
    if zero_lat:
        q = w.q_f32()
        q[:, :, :512] = 0.0
        w.q_bits = torch.from_numpy(np.ascontiguousarray(q)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    print(f"sweep {case}: T={T} H={H} K={K} ctx={ctx} neg={neg} splits={splits} mode={mode} zero_lat={zero_lat}",
          flush=True)
    ro, rl = O.attention_rows(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale)
    out, lse = smla.decode(q_dev(w), w.cache.to_device("cuda"), dev(slots), w.sm_scale, out_dtype=torch.float32,
                           num_splits=splits)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert not np.isnan(o).any() and not np.isnan(l).any()
    assert np.array_equal(np.isneginf(l), np.isneginf(rl)) and np.all(o[np.isneginf(rl)] == 0.0)
    fin = np.isfinite(rl)
    big = float(np.max(np.abs(ro), initial=0.0))
    tol = max(2e-2, 2e-3 * big) if mode else 2e-2
    ltol = 1e-3 * max(1.0, float(np.max(np.abs(rl[fin]), initial=1.0)) / 1000.0) if (mode and not zero_lat) else 1e-3
    do = float(np.max(np.abs(o - ro), initial=0.0))
    dl = float(np.max(np.abs(l[fin] - rl[fin]), initial=0.0))
    print(f"  max|dout| {do:.3e} (bar {tol:.2e})  max|dlse| {dl:.3e} (bar {ltol:.1e})", flush=True)
    assert do <= tol and dl <= ltol
