"""fp64 CPU oracle: sparse MLA decode over indexer top-k ids, fp8_ds_mla cache.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP path.

What it follows (the three pages this project is built from):

* Page "FlashMLA sparse fp8 path gains DCP and MTP" (prhub.com.cn summary of
  vLLM pull request 46514), sections "Implementation breakdown" (steps 1-3 and 5)
  and "Key source snippets" (flashmla_sparse.py ``_forward_fp8_kv_mixed_batch``,
  flashmla.py ``forward_mqa`` LSE flatten, and the test that neutralises empty
  rows).
* Page "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA"
  (local-inference-lab/vllm pull request 60), sections "Summary", "Why" and
  "Scope / Limitations" (global -> local DCP slot conversion, LSE returned for the
  DCP merge, packed fp8_ds_mla cache).
* Page "[Bugfix][Attention] Stabilize sparse-MLA DCP for GLM PCP evals"
  (vllm-project/vllm pull request 55879), "Root causes and fixes", subsection
  "Zero-local-sequence DCP warmup rank" (a shard with no local rows emits -inf LSE).

Readings where the pages are silent (R8-R12, on layouts, causality and tolerances,
need no code of their own here):

* R1 record layout: 656 bytes = 512 e4m3fn codes, 4 fp32 LE scales (scale i for
  latent dims 128i..128i+127), 64 bf16 LE rope values.  The pages give only the
  size (656 against 576 for the plain layout), so this order is a choice, and
  agreement with any real-world fp8_ds_mla byte order is parity unpinned.
* R2 fp8 flavour: OCP E4M3FN (bias 7, max 448, S.1111.111 is NaN, no infinities).
* R3 q = [latent 512 | rope 64]; key = [dequantised latent | rope]; value = the
  dequantised latent only (the output is 512 wide).
* R4 LSE is the natural log-sum-exp of the scaled logits sm_scale * <q, k>.
* R5 any negative id is "no candidate"; every remaining list entry is its own term
  (duplicates count twice); a slot outside [0, num_slots) is skipped like -1.
* R6 DCP ownership with interleave I: owner = (id // I) % D, local position =
  (id // (I * D)) * I + id % I; with I = 1 token t lives on shard t % D at t // D.
* R7 a row with no candidate (all -1, padded row, empty shard) is (out = 0,
  lse = -inf), the identity of the LSE merge; a merge whose inputs are all -inf
  is (0, -inf) too, never NaN.
* R15 plain bf16 record (the layout the pages contrast with fp8_ds_mla: 576
  values, 1152 bytes per token): 512 latent then 64 rope values, little-endian
  bf16; key = all 576, value = the 512 latent values.
* R13 quantiser of a record (only the cache write uses it; the decode reads stored
  bytes): per 128-value tile scale = fp32(amax / 448), or 1.0 when that is not
  positive (amax = 0, or an underflowing quotient); each latent value becomes
  fp32(x / scale) rounded to the nearest E4M3FN value, ties to the even code,
  magnitudes beyond 448 saturating to 448, the sign bit kept (so -0.0 and small
  negatives give 0x80); rope values are rounded to bf16 (nearest, ties to even).
  The pages name the packed cache but not its quantiser; the amax / 448 tile
  scale is the recipe of the tiny check configuration of the benchmark set.
* R14 cache placement under DCP: a new token at request position p is written
  only by the rank that owns p (R6) at its local position, through that rank's
  block table; with DCP off the position goes through the request's table as is.
  Page "FlashMLA sparse fp8 path gains DCP and MTP", "Review highlights", item 2:
  a draft model that maps ctx_pos // block_size without DCP disagrees with the
  target model's DCP-aware mapping.  A rank's local sequence length counts the
  positions below the request's length that it owns (page "[Bugfix][Attention]
  Stabilize sparse-MLA DCP for GLM PCP evals", "Root causes and fixes",
  subsection "DCP decode rank scalar", names the helper get_dcp_local_seq_lens).
"""
from __future__ import annotations

import numpy as np

LATENT = 512
ROPE = 64
TILE = 128
RECORD = 656


# ----------------------------------------------------------------- element decoders

def e4m3fn_to_f64(codes) -> np.ndarray:
    """Value of OCP E4M3FN codes (reading R2): sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & (c & 0x7 == 0x7), np.nan, v)


def bf16_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns: the upper half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


_E4M3_TABLE = e4m3fn_to_f64(np.arange(256, dtype=np.uint8))


def decode_records(rec) -> tuple:
    """Dequantise fp8_ds_mla records [n, 656] -> (latent [n,512], rope [n,64]) in fp64.

    latent[d] = e4m3(code[d]) * scale[d // 128] (reading R1); rope is bf16 as stored.
    Page "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA",
    "Scope / Limitations" names the packed fp8_ds_mla layout; the 656-byte size is
    stated on page "FlashMLA sparse fp8 path gains DCP and MTP", "Related".
    """
    rec = np.ascontiguousarray(np.asarray(rec, dtype=np.uint8).reshape(-1, RECORD))
    n = rec.shape[0]
    codes = rec[:, :LATENT]
    scales = rec[:, LATENT:LATENT + 16].copy().view("<f4").astype(np.float64)  # [n,4]
    rope_bits = rec[:, LATENT + 16:].copy().view("<u2")  # [n,64]
    latent = _E4M3_TABLE[codes] * np.repeat(scales, TILE, axis=1)
    return latent.reshape(n, LATENT), bf16_to_f64(rope_bits).reshape(n, ROPE)


BF16_RECORD = 2 * (LATENT + ROPE)  # 1152


def decode_records_bf16(rec) -> tuple:
    """Plain bf16 records [n, 1152] -> (latent [n,512], rope [n,64]) in fp64 (reading R15).
    Page "FlashMLA sparse fp8 path gains DCP and MTP", "Related" contrasts the 576-value
    layout with the packed 656-byte one; "Risks and impact" names the bf16 sparse path."""
    rec = np.ascontiguousarray(np.asarray(rec, dtype=np.uint8).reshape(-1, BF16_RECORD))
    v = bf16_to_f64(rec.copy().view("<u2"))
    return v[:, :LATENT], v[:, LATENT:]


RECORD_LAYOUTS = {"fp8_ds_mla": (RECORD, decode_records), "bf16": (BF16_RECORD, decode_records_bf16)}


# ----------------------------------------------------------------- index conversion

def convert_index(ids, req, block_table, block_size, dcp_size=1, dcp_rank=0, interleave=1):
    """Global top-k token ids -> physical cache slots, -1 where there is no candidate.

    Page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown"
    step 2 and "Key source snippets" (``_forward_fp8_kv_mixed_batch``): without DCP
    each request-relative id goes through the request's block table; under DCP the
    ids this rank does not own are set to -1 in place (no front compaction) and the
    rest become local slots of the rank's shard (reading R6).  ``req`` is the row's
    request (rows beyond the top-k rows are not used).  Returns (slots [T,K] int32,
    valid [T] int32 = number of entries that are not -1).
    """
    ids = np.asarray(ids, dtype=np.int64)
    req = np.asarray(req, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    T, K = ids.shape
    R, W = bt.shape
    B, D, r, I = int(block_size), int(dcp_size), int(dcp_rank), int(interleave)

    keep = ids >= 0
    if D > 1:
        owner = (ids // I) % D
        keep &= owner == r
        pos = (ids // (I * D)) * I + ids % I
    else:
        pos = ids.copy()
    pos = np.where(keep, pos, 0)
    blk = pos // B
    rq = np.broadcast_to(req[:, None], (T, K))
    keep &= (rq >= 0) & (rq < R) & (blk < W)
    phys = np.full((T, K), -1, dtype=np.int64)
    phys[keep] = bt[rq[keep], blk[keep]]
    keep &= phys >= 0
    slots = np.where(keep, phys * B + pos % B, -1)
    return slots.astype(np.int32), keep.sum(axis=1).astype(np.int32)


# ----------------------------------------------------------------- attention

def _gather(cache, slots):
    if hasattr(cache, "gather"):
        return cache.gather(slots)
    return np.asarray(cache)[np.asarray(slots, dtype=np.int64)]


def attention_rows(q, slots, cache, num_slots, sm_scale, record_layout="fp8_ds_mla"):
    """Softmax attention of each (row, head) over the row's own candidate records.

    Page "FlashMLA sparse fp8 path gains DCP and MTP", "Key source snippets": the
    fp8 kernel is called per query row with that row's top-k slot list and returns
    the output and the LSE; -1 entries are masked natively.  For a row with slot
    multiset J (reading R5):  s_j = sm_scale * <q, k_j>,  lse = log sum_j exp(s_j),
    out = sum_j exp(s_j - lse) * v_j.  A row with no candidate is (0, -inf)
    (reading R7, same page, "Implementation breakdown" step 3).

    q [T,H,576] float (fp64 arithmetic); slots [T,K]; cache: [num_slots, record] uint8
    array or an object with ``gather(slots) -> [n, record] bytes``; ``record_layout``
    "fp8_ds_mla" (656-byte records) or "bf16" (1152-byte records, reading R15).
    Returns out [T,H,512] fp64, lse [T,H] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    slots = np.asarray(slots, dtype=np.int64)
    T, H, _ = q.shape
    out = np.zeros((T, H, LATENT), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    for t in range(T):
        row = slots[t]
        J = row[(row >= 0) & (row < num_slots)]
        if J.size == 0:
            continue
        latent, rope = RECORD_LAYOUTS[record_layout][1](_gather(cache, J))
        keys = np.concatenate([latent, rope], axis=1)  # [n,576]
        s = sm_scale * (q[t] @ keys.T)  # [H,n]
        m = s.max(axis=1, keepdims=True)
        l = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        p = np.exp(s - l[:, None])
        out[t] = p @ latent
        lse[t] = l
    return out, lse


def sparse_mla_decode(q, slots, cache, num_slots, sm_scale):
    """Same as :func:`attention_rows`; named after the library call it checks."""
    return attention_rows(q, slots, cache, num_slots, sm_scale)


def sparse_mla_decode_bf16(q, slots, cache, num_slots, sm_scale):
    """:func:`attention_rows` over plain bf16 records (reading R15)."""
    return attention_rows(q, slots, cache, num_slots, sm_scale, record_layout="bf16")


# ----------------------------------------------------------------- DCP merge and layouts

def merge_lse(outs, lses):
    """Combine S shard partials (out_s [S,T,H,Dv], lse_s [S,T,H]) into (out, lse).

    lse = log sum_s exp(lse_s), out = sum_s exp(lse_s - lse) * out_s.  An all -inf
    entry is (0, -inf): (0, -inf) is the merge identity, so an empty shard changes
    nothing and never brings in NaN (page "FlashMLA sparse fp8 path gains DCP and
    MTP", "Implementation breakdown" step 3; page "[eldritch] attention: support DCP
    in SM120 FlashInfer sparse MLA", "Why": the common MLA layer merges the ranks'
    partial results with the returned LSE).
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)  # [T,H]
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(lses - m_safe[None])  # exp(-inf) = 0
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = w / np.where(finite, tot, 1.0)[None]
    out = (wn[..., None] * outs).sum(axis=0)
    out[~finite] = 0.0
    return out, lse


def transpose_hT_lse(lse_1ht):
    """Kernel-native LSE layout (1, H, T) -> (T, H) for the cross-rank merge
    (page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown"
    step 1 and the flashmla_sparse.py snippet: squeeze the batch axis, transpose)."""
    a = np.asarray(lse_1ht)
    return a.reshape(a.shape[-2], a.shape[-1]).T.copy()


def flatten_bhs_lse(lse_bhs):
    """Dense-decode LSE [batch, heads, seq_len] -> [batch * seq_len, heads], row b*S + s
    (page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown"
    step 5 and the flashmla.py snippet: permute(0, 2, 1) then reshape)."""
    a = np.asarray(lse_bhs)
    Bn, H, S = a.shape
    return np.transpose(a, (0, 2, 1)).reshape(Bn * S, H).copy()


# ----------------------------------------------------------------- cache write (DCP-aware)

_E4M3_POS = _E4M3_TABLE[:0x7F]  # values of codes 0x00 .. 0x7E, ascending; 0x7E = 448


def e4m3fn_encode(x) -> np.ndarray:
    """Nearest E4M3FN code of each value (reading R13): the nearest of the 127
    non-negative finite values to |x| (|x| clamped to 448), the even code on a tie,
    plus the sign bit of x.  Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _to_f32(x) -> np.ndarray:
    """Round fp64 values to the nearest fp32 (numpy's cast rounds to nearest, ties even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_encode(x) -> np.ndarray:
    """bf16 bit patterns of values already in fp32: nearest bf16, ties to even, as the
    upper 16 bits of the fp32 pattern after adding 0x7FFF plus the lowest kept bit."""
    b = np.ascontiguousarray(_to_f32(x)).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def quantize_records(latent, rope) -> np.ndarray:
    """Pack tokens into fp8_ds_mla records [n, 656] (readings R1 and R13).

    ``latent`` [n, 512] and ``rope`` [n, 64] hold fp32-representable values (bf16 or
    fp32 inputs).  Per 128-value tile: scale = fp32(amax / 448) (1.0 if that is not
    positive), code = E4M3FN-nearest of fp32(x / scale); rope is stored as bf16.
    The fp64 quotients rounded once to fp32 equal the correctly rounded fp32 divisions.
    """
    lat = np.asarray(latent, dtype=np.float64).reshape(-1, LATENT)
    n = lat.shape[0]
    tiles = lat.reshape(n, LATENT // TILE, TILE)
    amax = np.abs(tiles).max(axis=2)  # [n, 4]
    scale = _to_f32(amax / 448.0).astype(np.float64)
    scale = np.where(scale > 0.0, scale, 1.0)
    y = _to_f32(tiles / scale[:, :, None]).astype(np.float64)
    rec = np.zeros((n, RECORD), dtype=np.uint8)
    rec[:, :LATENT] = e4m3fn_encode(y).reshape(n, LATENT)
    rec[:, LATENT:LATENT + 16] = _to_f32(scale).astype("<f4").view(np.uint8).reshape(n, 16)
    rec[:, LATENT + 16:] = bf16_encode(np.asarray(rope, dtype=np.float64).reshape(n, ROPE)).astype("<u2").view(
        np.uint8).reshape(n, 2 * ROPE)
    return rec


def cache_write(latent, rope, positions, req, block_table, block_size, num_slots, dcp_size=1, dcp_rank=0,
                interleave=1):
    """Records of new tokens and the slots this rank writes them to (readings R13, R14).

    Token i sits at request position ``positions[i]`` of request ``req[i]``; the rank
    writes it iff it owns that position, at the slot the id-to-slot conversion gives
    for the same position (page "FlashMLA sparse fp8 path gains DCP and MTP",
    "Implementation breakdown" step 2 describes that conversion for reads).  A negative
    position, a missing block or a slot outside [0, num_slots) is not written.
    Returns (records [n, 656] uint8, slot_mapping [n] int32 with -1 = not written).
    """
    pos = np.asarray(positions, dtype=np.int64).reshape(-1, 1)
    slots, _ = convert_index(pos, req, block_table, block_size, dcp_size, dcp_rank, interleave)
    slots = slots[:, 0].astype(np.int64)
    slots = np.where((slots >= 0) & (slots < int(num_slots)), slots, -1)
    return quantize_records(latent, rope), slots.astype(np.int32)


def dcp_local_seq_lens(seq_lens, dcp_size, dcp_rank, interleave=1) -> np.ndarray:
    """Number of positions below each request's length that rank ``dcp_rank`` owns
    (reading R14 with the ownership of R6), counted position by position."""
    D, r, I = int(dcp_size), int(dcp_rank), int(interleave)
    out = []
    for L in np.asarray(seq_lens, dtype=np.int64).reshape(-1):
        p = np.arange(max(int(L), 0), dtype=np.int64)
        out.append(int(((p // I) % D == r).sum()))
    return np.asarray(out, dtype=np.int32)


# ----------------------------------------------------------------- dense decode (whole context)

def dense_decode(q, cache, num_slots, block_table, seq_lens, S, block_size, sm_scale, dcp_size=1, dcp_rank=0,
                 interleave=1):
    """Whole-context MLA decode with S query tokens per request, on one DCP rank.

    Page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown" step 5
    and the flashmla.py ``forward_mqa`` snippet: the dense path attends over the request's
    whole paged context and returns an LSE of layout [batch, heads, seq_len] that the DCP
    merge consumes flattened to [batch * seq_len, heads] (row b*S + s).  Query token s of
    request b sits at position seq_lens[b] - S + s and sees every position up to its own
    (reading R9, the same causality as the top-k rows); under DCP a rank sees the positions
    it owns (R6).  Written as the top-k attention with the list of all those positions.
    q [B*S, H, 576]; returns out [B*S, H, 512], lse [B*S, H] in fp64.
    """
    L = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    nb = L.shape[0]
    K = max(1, int(L.max()) if nb else 1)
    ids = np.full((nb * S, K), -1, dtype=np.int64)
    for b in range(nb):
        for s in range(S):
            n = max(0, int(L[b]) - S + s + 1)
            ids[b * S + s, :n] = np.arange(n)
    req = np.repeat(np.arange(nb), S)
    slots, _ = convert_index(ids, req, block_table, block_size, dcp_size, dcp_rank, interleave)
    return attention_rows(q, slots, cache, num_slots, sm_scale)
