"""Seeded synthetic workloads for sparse MLA decode over top-k ids.

Shapes and value distributions follow the five benchmark configurations of the
sparse-MLA decode path (tiny check case, plain decode batch, simulated DCP4,
MTP with DCP2, long-context mixed batch with DCP8).  Every array is drawn from
``numpy.random.Generator(PCG64(seed))`` in a fixed order:

    global block tables -> shard block tables -> top-k ids -> q -> KV records

fp8_ds_mla record (656 bytes per token; the pages give only the size, 656 vs
576, so the byte order is this project's own choice; ``kv="bf16"`` draws the same
values into the plain 576-value bf16 layout, 1152 bytes per token, instead):

    [0, 512)    512 latent values, OCP e4m3fn codes
    [512, 528)  4 little-endian fp32 scales, scale i covers latent dims 128i..128i+127
    [528, 656)  64 rope values, little-endian bf16

Quantisation of a record (generator only; the method reads stored bytes):
scale = fp32(amax / 448) per 128-value tile (1.0 if amax is 0), code =
e4m3fn(round-to-nearest-even(clamp(x / scale, -448, 448))).

Slots that no valid id may reference carry 0xFF bytes: NaN codes, NaN scales
and NaN rope, so a read of a wrong slot shows up as NaN.

Placement is constructive: request b's physical slots, in logical order, are the
concatenated slot ranges of its block-table row.  A DCP shard r with interleave I
holds the positions p of request b whose owner (p // I) % D is r, in increasing
order (local index (p // (I D)) I + p % I), placed through the shard's own block
table; with I = 1 these are r, r + D, r + 2D, ...
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

LATENT_DIM = 512
ROPE_DIM = 64
HEAD_DIM = LATENT_DIM + ROPE_DIM  # 576
SCALE_TILE = 128
RECORD_BYTES = LATENT_DIM + 4 * 4 + ROPE_DIM * 2  # 656
BF16_RECORD_BYTES = 2 * (LATENT_DIM + ROPE_DIM)  # 1152: the plain bf16 layout [latent 512 | rope 64]
KV_KINDS = {"fp8_ds_mla": RECORD_BYTES, "bf16": BF16_RECORD_BYTES}
E4M3_MAX = 448.0
POISON = 0xFF


# --------------------------------------------------------------------------- packing

def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pack_records(latent: np.ndarray, rope: np.ndarray) -> np.ndarray:
    """Quantise ``latent`` [n,512] fp32 and ``rope`` [n,64] fp32 into [n,656] uint8 records."""
    latent = np.ascontiguousarray(latent, dtype=np.float32)
    n = latent.shape[0]
    tiles = latent.reshape(n, LATENT_DIM // SCALE_TILE, SCALE_TILE)
    amax = np.abs(tiles).max(axis=2)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    y = np.clip(tiles / scale[:, :, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y.reshape(n, LATENT_DIM)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    rec = np.empty((n, RECORD_BYTES), dtype=np.uint8)
    rec[:, :LATENT_DIM] = codes
    rec[:, LATENT_DIM:LATENT_DIM + 16] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    rec[:, LATENT_DIM + 16:] = _to_bf16_bits(rope).astype("<u2").view(np.uint8).reshape(n, ROPE_DIM * 2)
    return rec


def pack_records_bf16(latent: np.ndarray, rope: np.ndarray) -> np.ndarray:
    """``latent`` [n,512] and ``rope`` [n,64] fp32 -> [n,1152] uint8 records of 576 little-endian bf16
    (nearest, ties to even): the latent values, then the rope values."""
    n = np.asarray(latent).shape[0]
    rec = np.empty((n, BF16_RECORD_BYTES), dtype=np.uint8)
    rec[:, :2 * LATENT_DIM] = _to_bf16_bits(latent).astype("<u2").view(np.uint8).reshape(n, 2 * LATENT_DIM)
    rec[:, 2 * LATENT_DIM:] = _to_bf16_bits(rope).astype("<u2").view(np.uint8).reshape(n, 2 * ROPE_DIM)
    return rec


# --------------------------------------------------------------------------- caches

class SparseCache:
    """A paged fp8_ds_mla cache of ``num_slots`` records of which only some are real.

    Every slot outside ``real_slots`` holds poison (0xFF bytes).  ``gather`` returns
    raw record bytes; nothing here interprets them.
    """

    def __init__(self, num_slots: int, real_slots: np.ndarray, records: np.ndarray):
        self.record_bytes = int(records.shape[1])
        order = np.argsort(real_slots, kind="stable")
        self.num_slots = int(num_slots)
        self.real_slots = np.asarray(real_slots, dtype=np.int64)[order]
        self.records = np.ascontiguousarray(records[order])
        if len(self.real_slots) and (self.real_slots[0] < 0 or self.real_slots[-1] >= num_slots):
            raise ValueError("real slot out of range")
        if len(np.unique(self.real_slots)) != len(self.real_slots):
            raise ValueError("duplicate real slot")

    @property
    def nbytes(self) -> int:
        return self.num_slots * self.record_bytes

    def gather(self, slots: np.ndarray) -> np.ndarray:
        slots = np.asarray(slots, dtype=np.int64).reshape(-1)
        out = np.full((slots.size, self.record_bytes), POISON, dtype=np.uint8)
        if self.real_slots.size == 0 or slots.size == 0:
            return out
        pos = np.searchsorted(self.real_slots, slots)
        pos_c = np.minimum(pos, self.real_slots.size - 1)
        hit = (pos < self.real_slots.size) & (self.real_slots[pos_c] == slots)
        out[hit] = self.records[pos_c[hit]]
        return out

    def dense(self) -> np.ndarray:
        out = np.full((self.num_slots, self.record_bytes), POISON, dtype=np.uint8)
        out[self.real_slots] = self.records
        return out

    def to_device(self, device) -> torch.Tensor:
        """Materialise the cache as a [num_slots, record_bytes] uint8 tensor on ``device``."""
        t = torch.full((self.num_slots, self.record_bytes), POISON, dtype=torch.uint8, device=device)
        if self.real_slots.size:
            idx = torch.from_numpy(self.real_slots).to(device)
            chunk = 1 << 18
            for s in range(0, idx.numel(), chunk):
                t.index_copy_(0, idx[s:s + chunk], torch.from_numpy(self.records[s:s + chunk]).to(device))
        return t


@dataclasses.dataclass
class ShardCache:
    """One simulated DCP shard: its own block table and its own paged cache."""

    rank: int
    block_table: np.ndarray  # [R, W_r] int32, -1 padded
    cache: SparseCache


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    K: int
    block_size: int
    dcp_size: int
    sm_scale: float
    out_dtype: str  # "bf16" or "fp32"
    q_bits: np.ndarray  # [T,H,576] uint16 (bf16 bit patterns)
    ids: np.ndarray  # [T,K] int32 global token ids, -1 = none
    req: np.ndarray  # [T] int32 request of each row
    row_pos: np.ndarray  # [T] int64 query position of each row (documentation / causal checks)
    ctx: np.ndarray  # [R] int64 context length of each request
    block_table: np.ndarray  # [R,W] int32, -1 padded
    cache: SparseCache
    shards: List[ShardCache]
    note: str = ""
    interleave: int = 1  # DCP interleave of the shard caches

    @property
    def R(self) -> int:
        return int(self.ctx.shape[0])

    def q_f32(self) -> np.ndarray:
        return (self.q_bits.astype(np.uint32) << 16).view(np.float32)

    def q_torch(self) -> torch.Tensor:
        return torch.from_numpy(self.q_bits.view(np.int16)).view(torch.bfloat16)

    def rows(self, idx) -> "Workload":
        """Sub-workload restricted to a subset of query rows (same caches)."""
        idx = np.asarray(idx)
        return dataclasses.replace(self, T=int(idx.size), q_bits=self.q_bits[idx], ids=self.ids[idx],
                                   req=self.req[idx], row_pos=self.row_pos[idx])


# --------------------------------------------------------------------------- helpers

def _block_table(rng: np.random.Generator, nblocks: np.ndarray, spare: int = 0):
    """Random permutation of all physical blocks, handed out to requests in order."""
    total = int(nblocks.sum()) + spare
    perm = rng.permutation(total).astype(np.int32)
    width = max(1, int(nblocks.max()) if nblocks.size else 1)
    bt = np.full((nblocks.size, width), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblocks):
        bt[b, :n] = perm[off:off + n]
        off += int(n)
    return bt, total


def _slots_in_order(bt_row: np.ndarray, n_tokens: int, block_size: int) -> np.ndarray:
    """Physical slots of logical positions 0..n_tokens-1: the block ranges laid end to end."""
    nb = -(-n_tokens // block_size)
    starts = bt_row[:nb].astype(np.int64) * block_size
    return (starts[:, None] + np.arange(block_size, dtype=np.int64)[None, :]).reshape(-1)[:n_tokens]


def _draw_records(rng: np.random.Generator, n: int, kv: str = "fp8_ds_mla") -> np.ndarray:
    pack = pack_records if kv == "fp8_ds_mla" else pack_records_bf16
    out = np.empty((n, KV_KINDS[kv]), dtype=np.uint8)
    step = 1 << 16
    for s in range(0, n, step):
        m = min(step, n - s)
        lat = rng.standard_normal((m, LATENT_DIM), dtype=np.float32)
        rope = rng.standard_normal((m, ROPE_DIM), dtype=np.float32)
        out[s:s + m] = pack(lat, rope)
    return out


class _Builder:
    """Accumulates requests, real positions and records, then places them in caches."""

    def __init__(self, block_size: int, dcp_size: int, record_bytes: int = RECORD_BYTES, interleave: int = 1):
        self.B = block_size
        self.D = dcp_size
        self.I = interleave
        self.rb = record_bytes

    def place(self, ctx, real_pos, records_by_req, bt, nphys, shard_bts):
        """Place records (one per real position, per request) in the global and shard caches."""
        B, D = self.B, self.D
        g_slots, g_recs = [], []
        s_slots = [[] for _ in range(D)] if D > 1 else []
        s_recs = [[] for _ in range(D)] if D > 1 else []
        for b, (pos, recs) in enumerate(zip(real_pos, records_by_req)):
            if pos.size == 0:
                continue
            order = _slots_in_order(bt[b], int(ctx[b]), B)
            g_slots.append(order[pos])
            g_recs.append(recs)
            if D > 1:
                for r in range(D):
                    owned = _owned_positions(int(ctx[b]), D, self.I, r)  # held by shard r, local order
                    if owned.size == 0:
                        continue
                    local_slots = _slots_in_order(shard_bts[r][0][b], owned.size, B)
                    # positions of this request that are real and owned by r, with their local index
                    sel = np.searchsorted(owned, pos)
                    ok = (sel < owned.size) & (owned[np.minimum(sel, owned.size - 1)] == pos)
                    s_slots[r].append(local_slots[sel[ok]])
                    s_recs[r].append(recs[ok])
        cat = lambda xs, shape: np.concatenate(xs) if xs else np.zeros(shape, dtype=np.int64)
        gcache = SparseCache(nphys * B, cat(g_slots, (0,)),
                             np.concatenate(g_recs) if g_recs else np.zeros((0, self.rb), np.uint8))
        shards = []
        if D > 1:
            for r in range(D):
                bt_r, nphys_r = shard_bts[r]
                recs = np.concatenate(s_recs[r]) if s_recs[r] else np.zeros((0, self.rb), np.uint8)
                shards.append(ShardCache(r, bt_r, SparseCache(max(nphys_r, 1) * B, cat(s_slots[r], (0,)), recs)))
        return gcache, shards


def _distinct(rng, hi: int, k: int) -> np.ndarray:
    """k distinct ids drawn uniformly from [0, hi), in random order."""
    if k > hi:
        raise ValueError("not enough positions")
    return rng.choice(hi, size=k, replace=False).astype(np.int32)


def _records_for(rng, real_pos: List[np.ndarray], kv: str = "fp8_ds_mla") -> List[np.ndarray]:
    n = sum(int(p.size) for p in real_pos)
    allrec = _draw_records(rng, n, kv)
    out, off = [], 0
    for p in real_pos:
        out.append(allrec[off:off + p.size])
        off += p.size
    return out


# --------------------------------------------------------------------------- configs

SM_SCALE = 192.0 ** -0.5

CONFIGS: Dict[int, dict] = {
    0: dict(name="c0_tiny", desc="T=4 (2 req x 2 tok), H=16, ctx 256, block 64, top-k 64 (56 ids + 8 x -1), D=1, out bf16"),
    1: dict(name="c1_decode", desc="T=32 (32 req x 1 tok), H=64, ctx 4096, top-k 2048, D=1, out fp32"),
    2: dict(name="c2_dcp4", desc="c1 rows + 4 req with ctx 2 (T=36), H=64, simulated DCP4, partials fp32"),
    3: dict(name="c3_mtp_dcp2", desc="T=256 (64 req x 4 MTP tok), H=128, ctx 32768, causal top-k 2048, simulated DCP2, out bf16"),
    4: dict(name="c4_mixed_dcp8", desc="128 decode rows (ctx 131072) + 4096 prefill rows (2 x 2048), H=128, top-k 2048, simulated DCP8, out bf16"),
}


def _finish(name, rng, *, H, K, B, D, out_dtype, ids, req, row_pos, ctx, real_pos, bt_pack, shard_bts, note="",
            kv="fp8_ds_mla", interleave=1):
    T = ids.shape[0]
    q = rng.standard_normal((T, H, HEAD_DIM), dtype=np.float32)
    q_bits = _to_bf16_bits(q)
    recs = _records_for(rng, real_pos, kv)
    bt, nphys = bt_pack
    cache, shards = _Builder(B, D, KV_KINDS[kv], interleave).place(ctx, real_pos, recs, bt, nphys, shard_bts)
    return Workload(name=name, T=T, H=H, K=K, block_size=B, dcp_size=D, sm_scale=SM_SCALE, out_dtype=out_dtype,
                    q_bits=q_bits, ids=ids.astype(np.int32), req=req.astype(np.int32), row_pos=row_pos.astype(np.int64),
                    ctx=ctx.astype(np.int64), block_table=bt, cache=cache, shards=shards, note=note,
                    interleave=interleave)


def _owned_positions(n: int, D: int, I: int, r: int) -> np.ndarray:
    """Positions p < n that DCP rank r of D holds with interleave I ((p // I) % D == r), in
    increasing order, which is their local order."""
    p = np.arange(n)
    return p[(p // I) % D == r]


def _shard_tables(rng, ctx, B, D, I: int = 1):
    out = []
    if D > 1:
        for r in range(D):
            local_ctx = np.array([_owned_positions(int(c), D, I, r).size for c in ctx], dtype=np.int64)
            out.append(_block_table(rng, -(-local_ctx // B)))
    return out


def make_config(cid: int, *, scale_rows: Optional[int] = None, kv: str = "fp8_ds_mla") -> Workload:
    """Build benchmark configuration ``cid`` (0..4) with seed 1000 + cid.

    ``scale_rows`` (c4 only) keeps the first n decode rows and every k-th prefill row so the
    mixed batch fits a CPU test; the full configuration is used when it is None.
    """
    B = 64
    if cid == 0:
        rng = np.random.Generator(np.random.PCG64(1000))
        ctx = np.array([256, 256], dtype=np.int64)
        bt_pack = _block_table(rng, -(-ctx // B))
        ids = np.full((4, 64), -1, dtype=np.int32)
        for t in range(4):
            ids[t, :56] = _distinct(rng, 256, 56)
        req = np.array([0, 0, 1, 1])
        row_pos = np.array([254, 255, 254, 255])
        real = [np.arange(c) for c in ctx]
        return _finish("c0_tiny", rng, H=16, K=64, B=B, D=1, out_dtype="bf16", ids=ids, req=req, row_pos=row_pos,
                       ctx=ctx, real_pos=real, bt_pack=bt_pack, shard_bts=[], kv=kv)
    if cid == 1:
        return _make_c1(np.random.Generator(np.random.PCG64(1001)), kv)
    if cid == 2:
        return _make_c2(kv)
    if cid == 3:
        rng = np.random.Generator(np.random.PCG64(1003))
        nreq, ntok, ctxlen, K, D = 64, 4, 32768, 2048, 2
        ctx = np.full(nreq, ctxlen, dtype=np.int64)
        bt_pack = _block_table(rng, -(-ctx // B))
        shard_bts = _shard_tables(rng, ctx, B, D)
        T = nreq * ntok
        ids = np.empty((T, K), dtype=np.int32)
        req = np.repeat(np.arange(nreq), ntok)
        row_pos = np.tile(ctxlen - ntok + np.arange(ntok), nreq)
        for t in range(T):
            ids[t] = _distinct(rng, int(row_pos[t]) + 1, K)  # causal: ids within [0, pos]
        real = [np.unique(ids[req == b]) for b in range(nreq)]
        return _finish("c3_mtp_dcp2", rng, H=128, K=K, B=B, D=D, out_dtype="bf16", ids=ids, req=req,
                       row_pos=row_pos, ctx=ctx, real_pos=real, bt_pack=bt_pack, shard_bts=shard_bts, kv=kv)
    if cid == 4:
        rng = np.random.Generator(np.random.PCG64(1004))
        n_dec, dec_ctx, n_pre, pre_len, K, D = 128, 131072, 2, 2048, 2048, 8
        ctx = np.concatenate([np.full(n_dec, dec_ctx), np.full(n_pre, pre_len)]).astype(np.int64)
        bt_pack = _block_table(rng, -(-ctx // B))
        shard_bts = _shard_tables(rng, ctx, B, D)
        dec_rows = list(range(n_dec))
        pre_rows = [(n_dec + p, pos) for p in range(n_pre) for pos in range(pre_len)]
        if scale_rows is not None:
            dec_rows = dec_rows[:scale_rows]
            step = max(1, len(pre_rows) // scale_rows)
            pre_rows = pre_rows[::step][:scale_rows]
        T = len(dec_rows) + len(pre_rows)
        ids = np.full((T, K), -1, dtype=np.int32)
        req = np.empty(T, dtype=np.int64)
        row_pos = np.empty(T, dtype=np.int64)
        for t, b in enumerate(dec_rows):
            ids[t] = _distinct(rng, dec_ctx, K)
            req[t], row_pos[t] = b, dec_ctx - 1
        for j, (b, pos) in enumerate(pre_rows):
            t = len(dec_rows) + j
            ids[t, :pos + 1] = rng.permutation(pos + 1).astype(np.int32)  # a fresh prompt: every earlier position
            req[t], row_pos[t] = b, pos
        real = []
        for b in range(ctx.size):
            sel = ids[req == b]
            real.append(np.unique(sel[sel >= 0]))
        name = "c4_mixed_dcp8" if scale_rows is None else f"c4_mixed_dcp8_sub{scale_rows}"
        return _finish(name, rng, H=128, K=K, B=B, D=D, out_dtype="bf16", ids=ids, req=req, row_pos=row_pos,
                       ctx=ctx, real_pos=real, bt_pack=bt_pack, shard_bts=shard_bts, kv=kv)
    raise ValueError(f"unknown config {cid}")


def _make_c1(rng, kv: str = "fp8_ds_mla") -> Workload:
    B = 64
    nreq, ctxlen, K = 32, 4096, 2048
    ctx = np.full(nreq, ctxlen, dtype=np.int64)
    bt_pack = _block_table(rng, -(-ctx // B))
    ids = np.stack([_distinct(rng, ctxlen, K) for _ in range(nreq)])
    req = np.arange(nreq)
    row_pos = np.full(nreq, ctxlen - 1)
    real = [np.arange(c) for c in ctx]
    return _finish("c1_decode", rng, H=64, K=K, B=B, D=1, out_dtype="fp32", ids=ids, req=req, row_pos=row_pos,
                   ctx=ctx, real_pos=real, bt_pack=bt_pack, shard_bts=[], kv=kv)


def _make_c2(kv: str = "fp8_ds_mla") -> Workload:
    """c1's 32 rows (identical draws, seed 1001) plus 4 requests of context 2 (seed 1002), DCP4."""
    B, D, K, H = 64, 4, 2048, 64
    base = _make_c1(np.random.Generator(np.random.PCG64(1001)), kv)
    rng = np.random.Generator(np.random.PCG64(1002))
    n_short = 4
    ctx = np.concatenate([base.ctx, np.full(n_short, 2)]).astype(np.int64)
    nb_base = int(base.cache.num_slots // B)
    bt = np.full((ctx.size, base.block_table.shape[1]), -1, dtype=np.int32)
    bt[:base.R] = base.block_table
    extra = rng.permutation(n_short).astype(np.int32) + nb_base
    bt[base.R:, 0] = extra
    nphys = nb_base + n_short
    shard_bts = _shard_tables(rng, ctx, B, D)
    ids = np.full((base.T + n_short, K), -1, dtype=np.int32)
    ids[:base.T] = base.ids
    for j in range(n_short):
        ids[base.T + j, :2] = rng.permutation(2).astype(np.int32)
    req = np.concatenate([base.req, base.R + np.arange(n_short)])
    row_pos = np.concatenate([base.row_pos, np.full(n_short, 1)])
    q_short = _to_bf16_bits(rng.standard_normal((n_short, H, HEAD_DIM), dtype=np.float32))
    q_bits = np.concatenate([base.q_bits, q_short])
    # records: c1's real records for its requests, fresh records for the short requests
    short_pos = [np.arange(2) for _ in range(n_short)]
    short_recs = _records_for(rng, short_pos, kv)
    base_real = [np.arange(c) for c in base.ctx]
    order_slots = [_slots_in_order(base.block_table[b], int(base.ctx[b]), B) for b in range(base.R)]
    base_recs = [base.cache.gather(s) for s in order_slots]
    cache, shards = _Builder(B, D, KV_KINDS[kv]).place(ctx, base_real + short_pos, base_recs + short_recs, bt, nphys,
                                                       shard_bts)
    return Workload(name="c2_dcp4", T=ids.shape[0], H=H, K=K, block_size=B, dcp_size=D, sm_scale=SM_SCALE,
                    out_dtype="fp32", q_bits=q_bits, ids=ids, req=req.astype(np.int32),
                    row_pos=row_pos.astype(np.int64), ctx=ctx, block_table=bt, cache=cache, shards=shards)


def make_random(seed: int, *, T: int, H: int, K: int, ctx: int, B: int = 64, D: int = 1, n_req: Optional[int] = None,
                neg_frac: float = 0.0, valid_max: Optional[int] = None, out_dtype: str = "bf16",
                all_real: bool = True, spare_blocks: int = 0, kv: str = "fp8_ds_mla", interleave: int = 1) -> Workload:
    """Small random workload for parity sweeps: ragged -1 patterns, any H/K/D and DCP interleave.

    Each row draws ``min(K, ctx)`` distinct ids (or ``valid_max``), scatters them over the K
    entries and sets a ``neg_frac`` share of the entries to -1.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n_req = n_req or T
    ctxs = np.full(n_req, ctx, dtype=np.int64)
    bt_pack = _block_table(rng, -(-ctxs // B), spare_blocks)
    shard_bts = _shard_tables(rng, ctxs, B, D, interleave)
    req = np.arange(T) % n_req
    ids = np.full((T, K), -1, dtype=np.int32)
    for t in range(T):
        nv = min(K, ctx) if valid_max is None else min(valid_max, K, ctx)
        nv = int(round(nv * (1.0 - neg_frac)))
        cols = rng.choice(K, size=nv, replace=False)
        ids[t, cols] = _distinct(rng, ctx, nv)
    row_pos = np.full(T, ctx - 1)
    if all_real:
        real = [np.arange(c) for c in ctxs]
    else:
        real = []
        for b in range(n_req):
            sel = ids[req == b]
            real.append(np.unique(sel[sel >= 0]))
    return _finish(f"rand{seed}", rng, H=H, K=K, B=B, D=D, out_dtype=out_dtype, ids=ids, req=req,
                   row_pos=row_pos, ctx=ctxs, real_pos=real, bt_pack=bt_pack, shard_bts=shard_bts, kv=kv,
                   interleave=interleave)


def make_dense(seed: int, *, n_req: int, S: int, H: int, ctx, B: int = 64, D: int = 1,
               out_dtype: str = "bf16", kv: str = "fp8_ds_mla") -> Workload:
    """Whole-context (dense) decode workload with S query tokens per request (MTP shape).

    Request b has context length ctx[b] (an int applies to all); its S query tokens are its
    last S positions, row b*S + s at position ctx[b] - S + s.  ``ids`` lists, per row, every
    position up to and including the row's own (causal), padded with -1 to K = max ctx, so the
    same workload also feeds the top-k path.  Every in-context position holds a real record.
    Draw order: block tables, shard tables, q, records.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ctxs = np.broadcast_to(np.asarray(ctx, dtype=np.int64), (n_req,)).copy()
    bt_pack = _block_table(rng, -(-ctxs // B))
    shard_bts = _shard_tables(rng, ctxs, B, D)
    T = n_req * S
    K = max(1, int(ctxs.max()) if n_req else 1)
    req = np.repeat(np.arange(n_req), S)
    row_pos = np.array([int(ctxs[b]) - S + s for b in range(n_req) for s in range(S)], dtype=np.int64)
    ids = np.full((T, K), -1, dtype=np.int32)
    for t in range(T):
        n = max(0, int(row_pos[t]) + 1)
        ids[t, :n] = np.arange(n, dtype=np.int32)
    real = [np.arange(c) for c in ctxs]
    return _finish(f"dense{seed}", rng, H=H, K=K, B=B, D=D, out_dtype=out_dtype, ids=ids, req=req,
                   row_pos=row_pos, ctx=ctxs, real_pos=real, bt_pack=bt_pack, shard_bts=shard_bts,
                   note=f"dense, S={S}", kv=kv)
