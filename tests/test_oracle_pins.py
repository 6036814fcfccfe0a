"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check is a function of the oracle's entry points so that the mutation test at
the bottom can re-run it against deliberately broken copies of the oracle and make
sure a plausible mistake (dropped term, wrong index, wrong sign, swapped operand)
fails at least one pin.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle.smla_oracle as O
from workload import make_config, make_random
from workload.gen import _slots_in_order

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ independent decoders (torch)

def torch_decode_records(rec):
    """Library-based record decode: torch float8_e4m3fn / bfloat16 casts, numpy fp32 view."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8).reshape(-1, 656)
    codes = torch.from_numpy(rec[:, :512].copy()).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.from_numpy(rec[:, 512:528].copy().view("<f4").astype(np.float64))
    rope = torch.from_numpy(rec[:, 528:].copy().view(np.int16)).view(torch.bfloat16).to(torch.float64)
    lat = codes * sc.repeat_interleave(128, dim=1)
    return lat.numpy(), rope.numpy()


def brute_force_rows(w, rows):
    """Dense masked softmax over each row's whole context (logical order, placement from the
    generator), -inf outside the row's id list, torch logsumexp/softmax in fp64."""
    q = w.q_f32().astype(np.float64)
    out = np.zeros((len(rows), w.H, 512))
    lse = np.full((len(rows), w.H), -np.inf)
    for i, t in enumerate(rows):
        b = int(w.req[t])
        ctx = int(w.ctx[b])
        slots = _slots_in_order(w.block_table[b], ctx, w.block_size)
        lat, rope = torch_decode_records(w.cache.gather(slots))
        keys = torch.from_numpy(np.concatenate([lat, rope], axis=1))
        ids = w.ids[t]
        ids = ids[(ids >= 0) & (ids < ctx)]
        if ids.size == 0:
            continue
        mult = np.bincount(ids, minlength=ctx).astype(np.float64)  # duplicates count twice
        s = w.sm_scale * (torch.from_numpy(q[t]) @ keys.T)  # [H, ctx]
        with np.errstate(divide="ignore"):
            logm = np.log(mult)
        s = s + torch.from_numpy(logm)[None, :]  # log(0) = -inf masks unselected positions
        l = torch.logsumexp(s, dim=1)
        p = torch.softmax(s, dim=1)
        out[i] = (p @ torch.from_numpy(lat)).numpy()
        lse[i] = l.numpy()
    return out, lse


def oracle_rows(w, rows, convert=None, attention=None):
    convert = convert or O.convert_index
    attention = attention or O.attention_rows
    sub = w.rows(rows)
    slots, _ = convert(sub.ids, sub.req, sub.block_table, sub.block_size)
    return attention(sub.q_f32(), slots, sub.cache, sub.cache.num_slots, sub.sm_scale)


# ------------------------------------------------------------------ checks (parametrised by oracle functions)

def check_e4m3(e4m3=O.e4m3fn_to_f64):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def check_bf16(bf16=O.bf16_to_f64):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = bf16(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def hand_record():
    """A record built by hand; expected values worked out from the OCP E4M3 definition."""
    rec = np.zeros(656, dtype=np.uint8)
    codes = {0: 0x38, 1: 0xB8, 2: 0x01, 3: 0x7E, 127: 0x40, 128: 0x3C, 300: 0x08, 383: 0x57, 511: 0x80}
    for d, c in codes.items():
        rec[d] = c
    rec[512:528] = np.array([0.5, 2.0, 0.25, 3.0], dtype="<f4").view(np.uint8)
    rope_bits = np.zeros(64, dtype="<u2")
    rope_bits[0], rope_bits[1], rope_bits[63] = 0x3F80, 0xC000, 0x4049
    rec[528:] = rope_bits.view(np.uint8)
    lat = np.zeros(512)
    # 0x38 = 0.0111.000 -> 2^(7-7) = 1 ; 0xB8 = -1 ; 0x01 = subnormal 2^-6 * 1/8 = 2^-9 ;
    # 0x7E = 0.1111.110 -> 2^8 * 1.75 = 448 ; 0x40 = 0.1000.000 -> 2 ; 0x3C = 0.0111.100 -> 1.5 ;
    # 0x08 = 0.0001.000 -> 2^-6 ; 0x57 = 0.1010.111 -> 2^3 * 1.875 = 15 ; 0x80 = -0
    lat[0], lat[1], lat[2], lat[3], lat[127] = 0.5, -0.5, 2.0 ** -9 * 0.5, 224.0, 1.0
    lat[128], lat[300], lat[383], lat[511] = 3.0, 2.0 ** -6 * 0.25, 15 * 0.25, -0.0
    rope = np.zeros(64)
    rope[0], rope[1], rope[63] = 1.0, -2.0, 3.140625  # 0x4049 = 0 10000000 1001001 -> 2 * 1.5703125
    return rec, lat, rope


def check_record(decode=O.decode_records):
    rec, lat, rope = hand_record()
    got_lat, got_rope = decode(rec[None])
    assert np.array_equal(got_lat[0], lat)
    assert np.signbit(got_lat[0, 511])
    assert np.array_equal(got_rope[0], rope)


CONVERT_HAND = dict(
    B=4,
    bt=np.array([[2, 0, -1], [1, 3, 4]], dtype=np.int32),
    ids=np.array([[0, 5, 3, -1, 9], [7, 0, 11, 12, -1], [1, 2, 3, 4, 5]], dtype=np.int32),
    req=np.array([0, 1, -1], dtype=np.int32),
    # worked by hand: slot = bt[req][pos // 4] * 4 + pos % 4, -1 where the block is absent
    d1=[[8, 1, 11, -1, -1], [15, 4, 19, -1, -1], [-1] * 5],
    d1_valid=[3, 3, 0],
    # D=2, rank 1, interleave 1: odd ids are owned, local = id // 2, shard table below
    bt_r1=np.array([[1, 0], [2, -1]], dtype=np.int32),
    d2r1=[[-1, 6, 5, -1, 0], [11, -1, -1, -1, -1], [-1] * 5],
    d2r1_valid=[3, 1, 0],
    # D=2, rank 0, interleave 2: owner = (id // 2) % 2, local = (id // 4) * 2 + id % 2
    bt_i2=np.array([[1, 0], [0, 1]], dtype=np.int32),
    d2i2=[[4, 7, -1, -1, 1], [-1, 0, -1, 6, -1], [-1] * 5],
    d2i2_valid=[3, 2, 0],
)


def check_convert_hand(convert=O.convert_index):
    h = CONVERT_HAND
    s, v = convert(h["ids"], h["req"], h["bt"], h["B"])
    assert s.tolist() == h["d1"] and v.tolist() == h["d1_valid"]
    s, v = convert(h["ids"], h["req"], h["bt_r1"], h["B"], dcp_size=2, dcp_rank=1)
    assert s.tolist() == h["d2r1"] and v.tolist() == h["d2r1_valid"]
    s, v = convert(h["ids"], h["req"], h["bt_i2"], h["B"], dcp_size=2, dcp_rank=0, interleave=2)
    assert s.tolist() == h["d2i2"] and v.tolist() == h["d2i2_valid"]


def check_convert_partition(w, convert=O.convert_index):
    """Every valid id lands on exactly one shard; the shard record is the id's record; the
    local position L recovers the id: (L // I) * I * D + rank * I + L % I (L * D + rank at I = 1)."""
    D, I = w.dcp_size, w.interleave
    g_slots, g_valid = convert(w.ids, w.req, w.block_table, w.block_size)
    owners = np.zeros(w.ids.shape, dtype=np.int64)
    total = np.zeros(w.T, dtype=np.int64)
    for sh in w.shards:
        s, v = convert(w.ids, w.req, sh.block_table, w.block_size, dcp_size=D, dcp_rank=sh.rank, interleave=I)
        ok = s >= 0
        owners += ok
        total += v
        assert np.array_equal(v, ok.sum(axis=1))
        # records at the shard slots equal the global records of the same ids
        assert np.array_equal(sh.cache.gather(s[ok]), w.cache.gather(g_slots[ok]))
        # inverse of the shard's block table: local position, times D plus rank, is the id
        rows, cols = np.nonzero(ok)
        slot = s[ok].astype(np.int64)
        blk, off = slot // w.block_size, slot % w.block_size
        for t, j, b_, o_ in zip(rows[:512], cols[:512], blk[:512], off[:512]):
            lb = int(np.nonzero(sh.block_table[w.req[t]] == b_)[0][0])
            L = lb * w.block_size + o_
            assert (L // I) * I * D + sh.rank * I + L % I == w.ids[t, j]
    valid_in = (w.ids >= 0)
    assert np.array_equal(owners, valid_in.astype(np.int64))
    assert np.array_equal(total, g_valid)


def check_brute_force(w, rows, tol=1e-12, **kw):
    o1, l1 = oracle_rows(w, rows, **kw)
    o2, l2 = brute_force_rows(w, rows)
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2))
    fin = np.isfinite(l2)
    assert np.max(np.abs(l1[fin] - l2[fin]), initial=0.0) <= tol
    assert np.max(np.abs(o1 - o2)) <= tol


def check_sdpa(attention=O.attention_rows):
    """top-k = every position, D = 1: torch scaled_dot_product_attention (fp64, one KV head)."""
    w = make_random(7, T=3, H=4, K=40, ctx=40, B=16)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    out, lse = attention(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale)
    for t in range(w.T):
        ctx_slots = _slots_in_order(w.block_table[w.req[t]], 40, 16)
        lat, rope = torch_decode_records(w.cache.gather(ctx_slots))
        k = torch.from_numpy(np.concatenate([lat, rope], 1))[None, None].expand(1, w.H, 40, 576)
        v = torch.from_numpy(lat)[None, None].expand(1, w.H, 40, 512)
        q = torch.from_numpy(w.q_f32()[t].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=w.sm_scale)[0, :, 0]
        ref_lse = torch.logsumexp(w.sm_scale * (q[0, :, 0] @ k[0, 0].T), dim=1)
        assert np.max(np.abs(out[t] - ref.numpy())) <= 1e-12
        assert np.max(np.abs(lse[t] - ref_lse.numpy())) <= 1e-12


def check_closed_forms(attention=O.attention_rows):
    w = make_random(11, T=2, H=3, K=8, ctx=64, B=16)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    q = w.q_f32().astype(np.float64)
    # one valid id: out = v, lse = s
    one = np.full_like(slots, -1)
    one[:, 3] = slots[:, 0]
    out, lse = attention(q, one, w.cache, w.cache.num_slots, w.sm_scale)
    for t in range(w.T):
        lat, rope = torch_decode_records(w.cache.gather([slots[t, 0]]))
        k = np.concatenate([lat[0], rope[0]])
        assert np.allclose(out[t], lat[0][None, :], rtol=0, atol=1e-13)
        assert np.allclose(lse[t], w.sm_scale * (q[t] @ k), rtol=0, atol=1e-12)
    # q = 0: out = mean of the valid values, lse = log(n)
    out, lse = attention(np.zeros_like(q), slots, w.cache, w.cache.num_slots, w.sm_scale)
    for t in range(w.T):
        J = slots[t][slots[t] >= 0]
        lat, _ = torch_decode_records(w.cache.gather(J))
        assert np.allclose(out[t], lat.mean(axis=0)[None, :], rtol=0, atol=1e-12)
        assert np.allclose(lse[t], np.log(J.size), rtol=0, atol=1e-13)
    # all -1: (0, -inf)
    out, lse = attention(q, np.full_like(slots, -1), w.cache, w.cache.num_slots, w.sm_scale)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def check_merge_shards(w, rows, merge=O.merge_lse, convert=O.convert_index, attention=O.attention_rows, tol=1e-12):
    sub = w.rows(rows)
    q = sub.q_f32()
    parts_o, parts_l = [], []
    for sh in sub.shards:
        s, _ = convert(sub.ids, sub.req, sh.block_table, sub.block_size, dcp_size=sub.dcp_size, dcp_rank=sh.rank,
                       interleave=sub.interleave)
        o, l = attention(q, s, sh.cache, sh.cache.num_slots, sub.sm_scale)
        parts_o.append(o)
        parts_l.append(l)
    mo, ml = merge(np.stack(parts_o), np.stack(parts_l))
    g, _ = convert(sub.ids, sub.req, sub.block_table, sub.block_size)
    uo, ul = attention(q, g, sub.cache, sub.cache.num_slots, sub.sm_scale)
    assert not np.isnan(mo).any() and not np.isnan(ml).any()
    assert np.array_equal(np.isneginf(ml), np.isneginf(ul))
    fin = np.isfinite(ul)
    assert np.max(np.abs(ml[fin] - ul[fin]), initial=0.0) <= tol
    assert np.max(np.abs(mo - uo)) <= tol


def check_merge_identities(merge=O.merge_lse):
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 4, 8))
    l = rng.standard_normal((3, 4)) * 3
    # (0, -inf) is the identity, bitwise
    mo, ml = merge(np.stack([o, np.zeros_like(o)]), np.stack([l, np.full_like(l, -np.inf)]))
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = merge(np.stack([np.zeros_like(o), o]), np.stack([np.full_like(l, -np.inf), l]))
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    # all empty -> (0, -inf), no NaN
    mo, ml = merge(np.zeros((4, 3, 4, 8)), np.full((4, 3, 4), -np.inf))
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # closed form for two parts: weights are sigmoid(l1 - l2)
    o2 = rng.standard_normal((3, 4, 8))
    l2 = rng.standard_normal((3, 4))
    mo, ml = merge(np.stack([o, o2]), np.stack([l, l2]))
    w1 = 1.0 / (1.0 + np.exp(l2 - l))
    assert np.allclose(ml, np.logaddexp(l, l2), atol=1e-14, rtol=0)
    assert np.allclose(mo, w1[..., None] * o + (1 - w1)[..., None] * o2, atol=1e-14, rtol=0)
    # associativity: merge(a, b, c) == merge(merge(a, b), c)
    o3 = rng.standard_normal((3, 4, 8))
    l3 = rng.standard_normal((3, 4))
    a_o, a_l = merge(np.stack([o, o2, o3]), np.stack([l, l2, l3]))
    ab_o, ab_l = merge(np.stack([o, o2]), np.stack([l, l2]))
    b_o, b_l = merge(np.stack([ab_o, o3]), np.stack([ab_l, l3]))
    assert np.allclose(a_o, b_o, atol=1e-14, rtol=0) and np.allclose(a_l, b_l, atol=1e-14, rtol=0)


def check_page_example(attention=O.attention_rows, merge=O.merge_lse):
    """The localised index pattern of the page's empty-row test, run against a real tiny cache
    whose slots 0..3 are real and every other slot is NaN poison."""
    with open(os.path.join(GOLDEN, "page_empty_row_example.json")) as f:
        ex = json.load(f)
    w = make_random(3, T=1, H=ex["num_heads"], K=4, ctx=4, B=4, spare_blocks=3)
    idx = np.array(ex["local_indices"], dtype=np.int32)
    phys = _slots_in_order(w.block_table[0], 4, 4)  # the 4 real slots
    slots = np.where(idx >= 0, phys[np.maximum(idx, 0)], -1).astype(np.int32)
    q = np.random.default_rng(0).standard_normal((ex["num_tokens"], ex["num_heads"], 576))
    out, lse = attention(q, slots, w.cache, w.cache.num_slots, w.sm_scale)
    for t in ex["empty_rows"]:
        assert np.all(out[t] == 0) and np.all(np.isneginf(lse[t]))
    for t in ex["nonempty_rows"]:
        assert np.all(np.isfinite(out[t])) and np.all(np.isfinite(lse[t]))
    assert out.flags.c_contiguous
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    # the row that is empty on this rank merges with another rank's partial unchanged
    other_o = np.random.default_rng(1).standard_normal(out.shape)
    other_l = np.random.default_rng(2).standard_normal(lse.shape)
    mo, ml = merge(np.stack([out, other_o]), np.stack([lse, other_l]))
    for t in ex["empty_rows"]:
        assert np.array_equal(mo[t], other_o[t]) and np.array_equal(ml[t], other_l[t])


def check_layouts(transpose=O.transpose_hT_lse, flatten=O.flatten_bhs_lse):
    lse_th = np.arange(12.0).reshape(4, 3)  # T=4, H=3
    native = np.ascontiguousarray(lse_th.T)[None]  # (1, H, T)
    assert np.array_equal(transpose(native), lse_th)
    # [B=2, H=3, S=2] -> [B*S, H]: row b*S + s holds lse[b, :, s]
    bhs = np.array([[[0, 1], [10, 11], [20, 21]], [[100, 101], [110, 111], [120, 121]]], dtype=np.float64)
    want = np.array([[0, 10, 20], [1, 11, 21], [100, 110, 120], [101, 111, 121]], dtype=np.float64)
    assert np.array_equal(flatten(bhs), want)


# ------------------------------------------------------------------ tests

def test_e4m3_all_codes():
    check_e4m3()


def test_bf16_all_patterns():
    check_bf16()


def test_record_hand_values():
    check_record()


def test_convert_hand_examples():
    check_convert_hand()


@pytest.mark.parametrize("D", [2, 4, 8])
def test_convert_dcp_partition(D):
    w = make_random(100 + D, T=6, H=16, K=96, ctx=300, B=16, D=D, neg_frac=0.1, n_req=3)
    check_convert_partition(w)


def test_convert_dcp_partition_c2():
    check_convert_partition(make_config(2))


def test_brute_force_c0():
    w = make_config(0)
    check_brute_force(w, list(range(w.T)))


@pytest.mark.parametrize("seed,T,H,K,ctx,B,neg", [(21, 4, 8, 40, 200, 16, 0.2), (22, 8, 16, 17, 512, 64, 0.5),
                                                   (23, 2, 2, 1, 33, 8, 0.0), (24, 5, 4, 64, 64, 32, 0.9)])
def test_brute_force_random(seed, T, H, K, ctx, B, neg):
    w = make_random(seed, T=T, H=H, K=K, ctx=ctx, B=B, neg_frac=neg)
    check_brute_force(w, list(range(T)))


def test_brute_force_duplicates_and_padding():
    w = make_random(31, T=3, H=4, K=10, ctx=50, B=16)
    w.ids[0, 5] = w.ids[0, 2]  # duplicate id: two terms
    w.ids[1, :] = -1  # empty row
    w.req = w.req.copy()
    check_brute_force(w, [0, 1, 2])


def test_sdpa_all_positions():
    check_sdpa()


def test_closed_forms():
    check_closed_forms()


@pytest.mark.parametrize("D", [2, 4, 8])
def test_merge_of_shards_equals_unsharded(D):
    w = make_random(200 + D, T=5, H=8, K=64, ctx=160, B=16, D=D, neg_frac=0.3, n_req=2)
    check_merge_shards(w, list(range(w.T)))


@pytest.mark.parametrize("D,I", [(2, 2), (2, 3), (4, 2), (4, 3)])
def test_convert_dcp_partition_interleaved(D, I):
    """Page "FlashMLA sparse fp8 path gains DCP and MTP", Implementation breakdown step 4: the
    interleave argument groups I consecutive tokens per rank."""
    w = make_random(110 + 10 * D + I, T=6, H=16, K=96, ctx=300, B=16, D=D, neg_frac=0.1, n_req=3, interleave=I)
    check_convert_partition(w)


@pytest.mark.parametrize("D,I", [(2, 2), (2, 3), (4, 2), (4, 3)])
def test_merge_of_interleaved_shards_equals_unsharded(D, I):
    w = make_random(210 + 10 * D + I, T=5, H=8, K=64, ctx=161, B=16, D=D, neg_frac=0.3, n_req=2, interleave=I)
    check_merge_shards(w, list(range(w.T)))


def test_merge_of_shards_c2_short_rows():
    w = make_config(2)
    check_merge_shards(w, [0, 1, 32, 33, 34, 35])


def test_merge_identities():
    check_merge_identities()


def test_page_empty_row_example():
    check_page_example()


def test_layouts():
    check_layouts()


def test_lse_allgather_counts():
    with open(os.path.join(GOLDEN, "lse_allgather_counts.json")) as f:
        ex = json.load(f)
    for rows, numel in ex["cases"]:
        lse = np.zeros((rows, ex["heads"]))
        assert O.transpose_hT_lse(np.ascontiguousarray(lse.T)[None]).size == numel


def test_generator_determinism():
    a, b = make_config(0), make_config(0)
    assert np.array_equal(a.q_bits, b.q_bits) and np.array_equal(a.ids, b.ids)
    assert np.array_equal(a.cache.records, b.cache.records)
    # c2's first 32 rows are c1's rows (same draws)
    c1, c2 = make_config(1), make_config(2)
    assert np.array_equal(c2.q_bits[:32], c1.q_bits) and np.array_equal(c2.ids[:32], c1.ids)


# ------------------------------------------------------------------ cache write (quantiser, placement)

def check_e4m3_encode(enc):
    """The encoder against the decoder's table, the midpoints, saturation and torch's cast."""
    vals = O.e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(enc(vals[finite]), finite.astype(np.uint8))  # every value is its own code
    pos = vals[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0  # exact in fp32: one more mantissa bit
    got = enc(mids).astype(np.int64)
    assert np.all(got % 2 == 0) and np.all((got == np.arange(126)) | (got == np.arange(1, 127)))
    up = np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    assert np.array_equal(enc(up), np.arange(1, 127, dtype=np.uint8))  # just above a midpoint: upper
    assert np.array_equal(enc(-up), (np.arange(1, 127) | 0x80).astype(np.uint8))
    assert list(enc(np.array([449.0, 1e30, -500.0, -0.0, 0.0, -1e-30]))) == [0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80]
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-12, 9, 200000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc(x.astype(np.float64)), ref)


def check_quantize(quant):
    """Quantised records against the error bound, the tile maximum, zero tiles, torch's bf16
    cast and the workload generator's own (torch-cast based) packer."""
    from workload.gen import pack_records
    rng = np.random.default_rng(11)
    lat = rng.standard_normal((64, 512)).astype(np.float32)
    lat[3, :128] = 0.0
    lat[4, 128:256] = -0.0
    lat[5, 256:384] *= np.float32(1e-30)
    lat[6] *= np.float32(1e4)
    rope = rng.standard_normal((64, 64)).astype(np.float32)
    rec = quant(lat.astype(np.float64), rope.astype(np.float64))
    assert rec.shape == (64, 656) and rec.dtype == np.uint8
    assert np.array_equal(rec, pack_records(lat, rope))
    sc = rec[:, 512:528].copy().view("<f4")
    assert sc[3, 0] == 1.0 and not rec[3, :128].any()
    assert sc[4, 1] == 1.0 and np.all(rec[4, 128:256] == 0x80)
    codes = rec[:, :512].reshape(64, 4, 128)
    tiles = lat.reshape(64, 4, 128)
    nz = np.abs(tiles).max(axis=2) > 0
    at_max = np.take_along_axis(codes, np.abs(tiles).argmax(axis=2)[..., None], axis=2)[..., 0] & 0x7F
    assert np.all(at_max[nz] == 0x7E)  # the tile maximum encodes as +-448
    dq = O.e4m3fn_to_f64(codes) * sc[:, :, None]
    y = np.abs(tiles / sc[:, :, None]).astype(np.float64)
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    half_ulp = np.exp2(e - 4)  # half of 2^(e-3); subnormals share the 2^-9 step
    assert np.all(np.abs(dq - tiles) <= half_ulp * sc[:, :, None] * (1 + 2.0 ** -20) + 1e-45)
    rope_ref = torch.from_numpy(rope).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rec[:, 528:].copy().view("<u2"), rope_ref)


def check_cache_write_hand(cw):
    """Worked by hand from the ownership rule: D = 2, block size 4, shard table of rank 1."""
    lat = np.zeros((6, 512))
    rope = np.zeros((6, 64))
    pos = np.array([0, 1, 2, 3, 5, 7])
    req = np.array([0, 0, 0, 1, 1, 1])
    bt = np.array([[3, 0], [1, 2]])
    # rank 1, I = 1: owns odd positions at local p // 2 -> (req 0, pos 1): bt[0][0]*4 + 0 = 12,
    # (req 1, pos 3): local 1 -> 1*4 + 1 = 5, pos 5 -> local 2 -> 6, pos 7 -> local 3 -> 7
    _, sm = cw(lat, rope, pos, req, bt, 4, 16, dcp_size=2, dcp_rank=1, interleave=1)
    assert list(sm) == [-1, 12, -1, 5, 6, 7]
    # rank 0, I = 2: owns positions 0,1 (and 4,5, 8,9, ...), local (p // 4) * 2 + p % 2
    _, sm = cw(lat, rope, pos, req, bt, 4, 16, dcp_size=2, dcp_rank=0, interleave=2)
    assert list(sm) == [12, 13, -1, -1, 7, -1]  # pos 5 of req 1: local 3 -> bt[1][0]*4 + 3
    # no DCP: position p -> bt[req][p // 4] * 4 + p % 4; slot 9 and beyond are cut by num_slots
    _, sm = cw(lat, rope, pos, req, bt, 4, 9, dcp_size=1, dcp_rank=0, interleave=1)
    assert list(sm) == [-1, -1, -1, 7, -1, -1]  # 12, 13, 14 >= 9; pos 5, 7 of req 1 -> 9, 11 >= 9


def check_cache_write_partition(cw):
    """Every token is written by exactly one rank, at a slot that the id conversion of the
    same position also yields (two oracle functions, one rule), with the same record bytes."""
    rng = np.random.default_rng(5)
    n, B = 40, 8
    lat = rng.standard_normal((n, 512))
    rope = rng.standard_normal((n, 64))
    req = rng.integers(0, 3, n)
    pos = rng.integers(0, 60, n)
    for D, I in ((2, 1), (4, 1), (4, 2), (3, 3)):
        owners = np.zeros(n, dtype=np.int64)
        for r in range(D):
            bt = rng.permutation(3 * 8).reshape(3, 8)
            rec, sm = cw(lat, rope, pos, req, bt, B, 24 * B, dcp_size=D, dcp_rank=r, interleave=I)
            owners += sm >= 0
            assert np.array_equal(rec, O.quantize_records(lat, rope))
            assert np.all(((pos // I) % D == r) == (sm >= 0))
    assert np.all(owners == 1)


def check_local_seq_lens(f):
    """Hand examples, the closed form and the partition of every length over the ranks."""
    assert list(f([10], 4, 0, 1)) + list(f([10], 4, 3, 1)) == [3, 2]
    assert [int(f([10], 4, r, 2)[0]) for r in range(4)] == [4, 2, 2, 2]
    assert list(f([0, 1, 2], 2, 1, 1)) == [0, 0, 1]
    rng = np.random.default_rng(3)
    L = rng.integers(0, 5000, 50)
    for D, I in ((2, 1), (4, 1), (8, 1), (4, 3)):
        tot = np.zeros(50, dtype=np.int64)
        for r in range(D):
            got = f(L, D, r, I).astype(np.int64)
            closed = (L // (I * D)) * I + np.clip(L % (I * D) - r * I, 0, I)
            assert np.array_equal(got, closed)
            tot += got
        assert np.array_equal(tot, L)


def test_e4m3_encode():
    check_e4m3_encode(O.e4m3fn_encode)


def test_quantize_records():
    check_quantize(O.quantize_records)


def test_cache_write_hand():
    check_cache_write_hand(O.cache_write)


def test_cache_write_partition():
    check_cache_write_partition(O.cache_write)


def test_dcp_local_seq_lens():
    check_local_seq_lens(O.dcp_local_seq_lens)


# ------------------------------------------------------------------ dense decode (whole context, MTP rows)

def check_dense_sdpa(dense):
    """Dense decode against torch's scaled_dot_product_attention over each request's logical
    context (records decoded by torch casts), a causal mask per query position, fp64; the LSE
    comes out in the pages' native [batch, heads, seq_len] layout and is flattened with the
    oracle's own (pinned) flatten to the [batch * seq_len, heads] rows."""
    from workload import make_dense
    S = 3
    w = make_dense(21, n_req=3, S=S, H=8, ctx=[70, 9, 2], B=16)
    out, lse = dense(w.q_f32(), w.cache, w.cache.num_slots, w.block_table, w.ctx, S, w.block_size, w.sm_scale)
    q = torch.from_numpy(w.q_f32().astype(np.float64))
    nb = len(w.ctx)
    native_lse = np.full((nb, w.H, S), -np.inf)
    native_out = np.zeros((nb, S, w.H, 512))
    for b in range(nb):
        L = int(w.ctx[b])
        lat, rope = torch_decode_records(w.cache.gather(_slots_in_order(w.block_table[b], L, w.block_size)))
        k = torch.from_numpy(np.concatenate([lat, rope], axis=1))[None, None]  # [1,1,L,576]
        v = torch.from_numpy(lat)[None, None]
        qb = q[b * S:(b + 1) * S].permute(1, 0, 2)[None]  # [1,H,S,576]
        pos = L - S + np.arange(S)
        visible = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])  # [S, L]
        if not visible.any():
            continue
        o = torch.nn.functional.scaled_dot_product_attention(qb, k.expand(1, w.H, L, 576), v.expand(1, w.H, L, 512),
                                                             attn_mask=visible, scale=w.sm_scale)
        sc = (qb @ k.transpose(-1, -2))[0] * w.sm_scale  # [H,S,L]
        l = torch.logsumexp(sc.masked_fill(~visible[None], -np.inf), dim=-1)  # [H,S]
        for s in range(S):
            if visible[s].any():
                native_out[b, s] = o[0, :, s].numpy()
                native_lse[b, :, s] = l[:, s].numpy()
    ref_lse = O.flatten_bhs_lse(native_lse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0) < 1e-10
    assert np.max(np.abs(out - native_out.reshape(nb * S, w.H, 512)), initial=0) < 1e-10
    assert np.all(out[~fin] == 0)


def check_dense_dcp_merge(dense, merge):
    """The merge of the D shards' dense partials equals the unsharded dense decode."""
    from workload import make_dense
    for D in (2, 4):
        w = make_dense(30 + D, n_req=2, S=2, H=4, ctx=[45, 3], B=8, D=D)
        args = (w.ctx, 2, w.block_size, w.sm_scale)
        ref_o, ref_l = dense(w.q_f32(), w.cache, w.cache.num_slots, w.block_table, *args)
        parts = [dense(w.q_f32(), sh.cache, sh.cache.num_slots, sh.block_table, *args, dcp_size=D, dcp_rank=sh.rank)
                 for sh in w.shards]
        o, l = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.max(np.abs(o - ref_o)) < 1e-12 and np.array_equal(np.isneginf(l), np.isneginf(ref_l))
        fin = np.isfinite(ref_l)
        assert np.max(np.abs(l[fin] - ref_l[fin]), initial=0) < 1e-12


def test_dense_sdpa():
    check_dense_sdpa(O.dense_decode)


def test_dense_dcp_merge():
    check_dense_dcp_merge(O.dense_decode, O.merge_lse)


# ------------------------------------------------------------------ plain bf16 records

def torch_decode_records_bf16(rec):
    """Library-based decode of plain bf16 records: torch's bfloat16 view widened to fp64."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8).reshape(-1, 1152)
    v = torch.from_numpy(rec.copy().view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return v[:, :512], v[:, 512:]


def check_bf16_records_sdpa(decode_bf16, attention):
    """bf16 records: the decoder against torch's bf16 view, and top-k = every position against
    scaled_dot_product_attention over the torch-decoded context (fp64, one KV head)."""
    w = make_random(17, T=3, H=4, K=48, ctx=48, B=16, kv="bf16")
    assert w.cache.record_bytes == 1152
    lat, rope = decode_bf16(w.cache.records)
    tl, tr = torch_decode_records_bf16(w.cache.records)
    assert np.array_equal(lat, tl) and np.array_equal(rope, tr)
    slots, _ = O.convert_index(w.ids, w.req, w.block_table, w.block_size)
    out, lse = attention(w.q_f32(), slots, w.cache, w.cache.num_slots, w.sm_scale, record_layout="bf16")
    for t in range(w.T):
        lat, rope = torch_decode_records_bf16(w.cache.gather(_slots_in_order(w.block_table[w.req[t]], 48, 16)))
        k = torch.from_numpy(np.concatenate([lat, rope], 1))[None, None].expand(1, w.H, 48, 576)
        v = torch.from_numpy(lat)[None, None].expand(1, w.H, 48, 512)
        q = torch.from_numpy(w.q_f32()[t].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=w.sm_scale)[0, :, 0]
        ref_lse = torch.logsumexp(w.sm_scale * (q[0, :, 0] @ k[0, 0].T), dim=1)
        assert np.max(np.abs(out[t] - ref.numpy())) <= 1e-12
        assert np.max(np.abs(lse[t] - ref_lse.numpy())) <= 1e-12


def test_bf16_records_sdpa():
    check_bf16_records_sdpa(O.decode_records_bf16, O.attention_rows)


# ------------------------------------------------------------------ planted mistakes

ORIG = {name: getattr(O, name) for name in
        ("decode_records", "e4m3fn_to_f64", "attention_rows", "convert_index", "merge_lse", "e4m3fn_encode",
         "quantize_records", "cache_write", "dcp_local_seq_lens", "dense_decode", "decode_records_bf16")}


def _mutants():
    def drop_rope(rec):
        lat, rope = ORIG["decode_records"](rec)
        return lat, np.zeros_like(rope)

    def wrong_scale_index(rec):
        rec = np.ascontiguousarray(np.asarray(rec, dtype=np.uint8).reshape(-1, 656))
        lat, rope = ORIG["decode_records"](rec)
        sc = rec[:, 512:528].copy().view("<f4").astype(np.float64)
        codes = O._E4M3_TABLE[rec[:, :512]]
        return codes * np.tile(sc, 128), rope  # scale index d % 4 instead of d // 128

    def sign_flip_e4m3(codes):
        return -ORIG["e4m3fn_to_f64"](codes)

    def lse_without_max(q, slots, cache, n, sc, **kw):
        out, lse = ORIG["attention_rows"](q, slots, cache, n, sc, **kw)
        return out, lse - 0.5

    def convert_swapped_owner(ids, req, bt, B, dcp_size=1, dcp_rank=0, interleave=1):
        if dcp_size > 1:
            ids = np.where(np.asarray(ids) >= 0, np.asarray(ids) + 1, ids)  # off-by-one ownership
        return ORIG["convert_index"](ids, req, bt, B, dcp_size, dcp_rank, interleave)

    def convert_offset_swap(ids, req, bt, B, dcp_size=1, dcp_rank=0, interleave=1):
        s, v = ORIG["convert_index"](ids, req, bt, B, dcp_size, dcp_rank, interleave)
        return np.where(s >= 0, (s // B) * B + (B - 1 - s % B), s).astype(np.int32), v

    def merge_unnormalised(outs, lses):
        o, l = ORIG["merge_lse"](outs, lses)
        return np.asarray(outs).sum(axis=0), l

    def qk_transposed_value(q, slots, cache, n, sc, **kw):
        out, lse = ORIG["attention_rows"](q, slots, cache, n, sc, **kw)
        return out[..., ::-1].copy(), lse

    def encode_ties_away(x):
        x = np.asarray(x, dtype=np.float64)
        return ORIG["e4m3fn_encode"](x * (1 + 2.0 ** -30))  # midpoints go up, not to even

    def quantize_wrong_max(lat, rope):
        return ORIG["quantize_records"](np.asarray(lat) * (447.0 / 448.0), rope)

    def quantize_rope_truncated(lat, rope):
        rec = ORIG["quantize_records"](lat, rope).copy()
        r32 = np.asarray(rope, dtype=np.float32).reshape(rec.shape[0], 64)
        rec[:, 528:] = (r32.view(np.uint32) >> 16).astype("<u2").view(np.uint8).reshape(rec.shape[0], 128)
        return rec

    def cache_write_dcp_blind(lat, rope, pos, req, bt, B, n, dcp_size=1, dcp_rank=0, interleave=1):
        rec, sm = ORIG["cache_write"](lat, rope, pos, req, bt, B, n)
        own = (np.asarray(pos) // interleave) % dcp_size == dcp_rank
        return rec, np.where(own, sm, -1).astype(np.int32)

    def local_lens_ceil(L, D, r, I=1):
        return ORIG["dcp_local_seq_lens"](np.asarray(L) + 1, D, r, I)

    def dense_causal_short(q, cache, n, bt, L, S, B, sc, dcp_size=1, dcp_rank=0, interleave=1):
        return ORIG["dense_decode"](q, cache, n, bt, np.asarray(L) - 1, S, B, sc, dcp_size, dcp_rank, interleave)

    def dense_rows_s_major(q, cache, n, bt, L, S, B, sc, dcp_size=1, dcp_rank=0, interleave=1):
        o, l = ORIG["dense_decode"](q, cache, n, bt, L, S, B, sc, dcp_size, dcp_rank, interleave)
        nb = len(np.asarray(L))
        perm = np.arange(nb * S).reshape(nb, S).T.reshape(-1)
        return o[perm], l[perm]

    def bf16_rope_first(rec):
        rec = np.ascontiguousarray(np.asarray(rec, dtype=np.uint8).reshape(-1, 1152))
        v = O.bf16_to_f64(rec.copy().view("<u2"))
        return v[:, 64:], v[:, :64]

    return {
        "decode_records_bf16": [bf16_rope_first],
        "dense_decode": [dense_causal_short, dense_rows_s_major],
        "e4m3fn_encode": [encode_ties_away],
        "quantize_records": [quantize_wrong_max, quantize_rope_truncated],
        "cache_write": [cache_write_dcp_blind],
        "dcp_local_seq_lens": [local_lens_ceil],
        "decode_records": [drop_rope, wrong_scale_index],
        "e4m3fn_to_f64": [sign_flip_e4m3],
        "attention_rows": [lse_without_max, qk_transposed_value],
        "convert_index": [convert_swapped_owner, convert_offset_swap],
        "merge_lse": [merge_unnormalised],
    }


def _all_pins():
    w0 = make_config(0)
    wd = make_random(300, T=4, H=8, K=48, ctx=120, B=16, D=4, neg_frac=0.2, n_req=2)
    return [
        lambda: check_e4m3(O.e4m3fn_to_f64),
        lambda: check_record(O.decode_records),
        lambda: check_convert_hand(O.convert_index),
        lambda: check_convert_partition(wd, O.convert_index),
        lambda: check_brute_force(w0, list(range(w0.T)), convert=O.convert_index, attention=O.attention_rows),
        lambda: check_sdpa(O.attention_rows),
        lambda: check_closed_forms(O.attention_rows),
        lambda: check_merge_shards(wd, list(range(wd.T)), merge=O.merge_lse, convert=O.convert_index,
                                   attention=O.attention_rows),
        lambda: check_merge_identities(O.merge_lse),
        lambda: check_page_example(O.attention_rows, O.merge_lse),
        lambda: check_e4m3_encode(O.e4m3fn_encode),
        lambda: check_quantize(O.quantize_records),
        lambda: check_cache_write_hand(O.cache_write),
        lambda: check_cache_write_partition(O.cache_write),
        lambda: check_local_seq_lens(O.dcp_local_seq_lens),
        lambda: check_dense_sdpa(O.dense_decode),
        lambda: check_bf16_records_sdpa(O.decode_records_bf16, O.attention_rows),
        lambda: check_dense_dcp_merge(O.dense_decode, O.merge_lse),
    ]


@pytest.mark.parametrize("target,idx", [(k, i) for k, v in _mutants().items() for i in range(len(v))])
def test_planted_mistake_is_caught(monkeypatch, target, idx):
    mutant = _mutants()[target][idx]
    monkeypatch.setattr(O, target, mutant)
    caught = 0
    for pin in _all_pins():
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches the planted mistake {mutant.__name__} in {target}"
