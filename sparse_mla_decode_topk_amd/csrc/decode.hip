// Sparse MLA decode over per-row top-k slot lists against a packed fp8_ds_mla cache.
//
// Computes, per query row t and head h, softmax attention over the row's own candidate
// records and returns out[t,h,0:512] and lse[t,h] (page "FlashMLA sparse fp8 path gains
// DCP and MTP", "Key source snippets" and "Implementation breakdown" steps 1-3; page
// "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA", "Why").
//
// gfx950 design
//  * A workgroup owns one row, up to 64 heads of it and one range of the row's top-k list.
//    It runs 8 waves, two per SIMD, in two roles that overlap on every SIMD: four score
//    waves (16 heads each) run QK^T on fp8 MFMA plus the softmax on the VALU for tile n,
//    while four value waves (one 128-dim scale tile of the output each) run PV on bf16
//    MFMA for tile n-1.  One SIMD thus interleaves one wave's vector work with the other's
//    matrix work.  The query lives in the score waves' registers, the output accumulators
//    in the value waves'; the roles branch apart at the top so neither holds the other's.
//  * Gather: the row's slot range is compacted in LDS (-1 and out-of-range entries are
//    skipped; no front-pack on the host), then tiles of 32 records are copied HBM -> LDS
//    with global_load_lds_dwordx4 by the value waves, kAhead tiles ahead.  One load moves
//    two 16-byte chunks of all 32 records, so a tile sits chunk-major in LDS
//    ([41 chunks][32 records][16 B]) and every MFMA operand read is contiguous.
//  * QK^T latent part on v_mfma_scale_f32_16x16x128_f8f6f4: the raw e4m3 codes are the
//    record operand as stored; q is split exactly into two e4m3 terms, q * 2^e_h = hi + lo
//    (hi = rne(q * 2^e_h), lo = rne(q * 2^e_h - hi), e_h a per-head power of two that puts
//    max|q| just under 448; exact wherever |q * 2^e_h| >= 2^-2), so two fp8 MFMAs give the
//    bf16-exact product at the cost of one bf16 MFMA and no widening; the MFMA's E8M0 scale
//    of each q row takes 2^-e_h back out.  One MFMA k-step spans exactly one 128-dim scale
//    tile, whose fp32 record scale then multiplies that tile's partial dot product.  Rope
//    dims (bf16) run on v_mfma_f32_16x16x32_bf16.  Scores come out as heads x tokens: a lane
//    holds one token of each 16-token half and four heads, so it needs the record scales of
//    two tokens only, and keeps a running max per head without cross-lane work per tile.
//  * Softmax in base 2 against a per-head reference max fixed at the first tile: later
//    probabilities are 2^(s - ref) and may exceed 1, which fp32 accumulators and bf16
//    probabilities hold without loss.  Should a score ever exceed the reference by more
//    than 2^64 the workgroup recomputes the range once with the exact max as reference, so
//    the output accumulators are never rescaled inside the loop and the value waves never
//    wait on a max.
//  * PV: O^T[dim, head] += V^T[dim, token] . P'^T[token, head] on bf16 MFMA, with
//    P' = p * scale(token, tile) rounded once to bf16 and handed over in LDS per scale tile
//    as [token][head] rows (double-buffered), read back transposed by ds_read_b64_tr_b16;
//    V^T fragments come straight from the staged tile through ds_read_b64_tr_b8 and are
//    widened exactly.
//  * One workgroup barrier per tile orders it all: tile n staged, P'(n-1) written, and
//    tile n-2 plus P'(n-2) consumed, so its buffers may be refilled.
//  * Split-K over the top-k list with an in-kernel combine: every split writes its
//    unnormalised partial (O, max, sum) to the workspace; the last split to arrive (device
//    scope counter, zeroed by a small kernel before the decode kernel) merges them.
//  * The output leaves through LDS: after the loop the value waves write O as [head][dim]
//    rows into the freed tile, probability and slot-list buffers, and all eight waves store
//    whole rows.
//  * A row with no valid entry yields out = 0, lse = -inf.

#include "decode_common.h"

namespace smla {
namespace {

using namespace dec;

constexpr int kUnitScale = 127;       // E8M0 encoding of 2^0 for the scaled fp8 MFMA

constexpr int kTT = 32;                         // records per tile
constexpr int kChunks = kRecordBytes / 16;      // 41 chunks of 16 bytes per record
constexpr int kCS = 16 * kTT;                   // bytes per chunk row of a tile
constexpr int kTileBytes = kChunks * kCS;       // 20992
constexpr int kStages = 4;                      // tile buffers: scores on n, values on n-1,
constexpr int kAhead = kStages - 2;             //   loads in flight for n+1 .. n+kAhead
constexpr int kLoads = (kChunks + 1) / 2;       // 21 global_load_lds per tile, two chunks each
constexpr int kPRow = 2 * kHB;                  // bytes per token row of a probability tile
constexpr int kPTile = kTT * kPRow;             // one scale tile of probabilities (4 KB)
constexpr int kPBuf = 4 * kPTile;               // all four scale tiles (16 KB)
constexpr int kScaleChunk = kScaleOffset / 16;  // 32
constexpr int kRopeChunk = kRopeOffset / 16;    // 33

static_assert(kRecordBytes % 16 == 0, "records are whole 16-byte chunks");
static_assert(kAhead >= 1 && kAhead <= 3, "load waits below cover up to 3 tiles ahead");
static_assert(kHB * kMaxSplits * 4 <= kStages * kTileBytes, "split weights fit in the tile buffers");
static_assert(kHB * (kLatent / 4) % kThreads == 0 && kThreads % (kLatent / 4) == 0, "combine item split");

struct Shared {
  uint8_t stage[kStages * kTileBytes];  // followed directly by pbuf and clist: the output staging
  uint8_t pbuf[2 * kPBuf];              // rows span all three once the tile loop is done
  int32_t clist[kMaxEntriesPerSplit];
  float ml[2 * kHB];  // per head of the block: (reference max, sum)
  int32_t wave_cnt[kThreads / 64];
  int32_t last_flag;
};
static_assert(offsetof(Shared, pbuf) == offsetof(Shared, stage) + sizeof(Shared::stage) &&
                  offsetof(Shared, clist) == offsetof(Shared, pbuf) + sizeof(Shared::pbuf),
              "tile, probability and slot-list buffers are contiguous");
static_assert(kStages * kTileBytes + 2 * kPBuf + 4 * kMaxEntriesPerSplit >= kOutStageBytes,
              "output staging rows fit in the tile, probability and slot-list buffers");
static_assert(kHB * (4 * kLatent / 16) % kThreads == 0 && kHB * (2 * kLatent / 16) % kThreads == 0, "row store split");

// Start of the output staging rows (the tile, probability and slot-list buffers as one span).
__device__ __forceinline__ uint8_t* staging(Shared& sh) { return reinterpret_cast<uint8_t*>(&sh) + offsetof(Shared, stage); }
__device__ __forceinline__ const uint8_t* staging(const Shared& sh) {
  return reinterpret_cast<const uint8_t*>(&sh) + offsetof(Shared, stage);
}

__device__ __forceinline__ bf16x8 widen_fp8x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A x B on fp8 with the A rows scaled by 2^(sa - 127) (E8M0 sa, this lane's row) and unit B scales.
__device__ __forceinline__ f32x4 mfma16_fp8(const i32x8& a, const i32x8& b, const f32x4& c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, kUnitScale);
}

// Four fp32 values -> packed e4m3 hi terms and the exact residual lo terms.
__device__ __forceinline__ void split_e4m3(float x0, float x1, float x2, float x3, int& hi, int& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - b01[0], x1 - b01[1], 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - b23[0], x3 - b23[1], l, true);
  hi = h;
  lo = l;
}

// Global->LDS loads one value wave issues per tile: load j of a tile belongs to wave j % 4.
__device__ __forceinline__ int loads_of_wave(int b) { return b < kLoads % 4 ? kLoads / 4 + 1 : kLoads / 4; }

// Wait until this wave's loads of tile n have landed, given `tiles_newer` later tiles of
// this wave still in flight (wave-uniform).
__device__ __forceinline__ void wait_tile(int tiles_newer, int b) {
  const int newer = tiles_newer * loads_of_wave(b);
  switch (newer) {
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 12: wait_vmcnt<12>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// HBM -> LDS copy of one tile by value wave b (0..3): load j moves chunks 2j and 2j+1 of all
// 32 records (lane r < 32: chunk 2j of record r, lane 32 + r: chunk 2j + 1 of record r), so
// its LDS destination is the contiguous kilobyte j of the tile.  `rec` is this lane's record
// (plus 16 bytes in the upper half-wave).
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* rec, int b, int lane) {
#pragma unroll
  for (int k = 0; k < (kLoads + 3) / 4; ++k) {
    const int j = b + 4 * k;
    if (j < kLoads - 1 || (j == kLoads - 1 && lane < 32)) lds_dma16(rec + 32 * j, stage + 1024 * j);
  }
}

// Slot of tile entry (lane & 31); entries past the end of the list repeat the last one.
__device__ __forceinline__ int lane_slot(const Shared& sh, int n, int total, int lane) {
  return sh.clist[min(n * kTT + (lane & 31), total - 1)];
}
// This lane's 16-byte column of that slot's record.
__device__ __forceinline__ const uint8_t* lane_record(const DecodeParams& p, int slot, int lane) {
  return p.kv + (int64_t)slot * kRecordBytes + 16 * (lane >> 5);
}

// A score wave lane's query values as loaded: latent dims 128t + 32g + 8c .. +7 in lat[4t + c]
// and rope dims 32kk + 8g .. +7 in rope[kk] (g = lane >> 4), bf16 bits.
struct QRaw {
  i32x4 lat[16];
  i32x4 rope[2];
};

// Issued before the slot compaction, so the query and slot-list loads share one memory round
// trip.
__device__ __forceinline__ void load_q(const DecodeParams& p, const Block& bk, int sw, int lane, QRaw& qv) {
  const int g = lane >> 4;
  const uint16_t* qp = p.q + (int64_t)bk.row * p.q_st + (int64_t)(bk.h_lo + 16 * sw + (lane & 15)) * p.q_sh;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c) qv.lat[4 * t + c] = *reinterpret_cast<const i32x4*>(qp + 128 * t + 32 * g + 8 * c);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) qv.rope[kk] = *reinterpret_cast<const i32x4*>(qp + kLatent + 32 * kk + 8 * g);
}

// ---------------------------------------------------------------------------------------
// Score wave `sw` (0..3): heads h_lo + 16sw + (lane & 15); lane group g = lane >> 4 holds
// the query dims 128t + 32g .. +31 of every scale tile t and rope dims 32kk + 8g .. +7.
__device__ __forceinline__ void score_role(const DecodeParams& p, Shared& sh, const Block& bk, const QRaw& qv,
                                           int sw, int lane) {
  const int g = lane >> 4;
  const int hl = 16 * sw + (lane & 15);  // head within the block
  const bool active = 16 * sw < bk.nh;
  i32x8 qh[4], ql[4];  // q * 2^e as e4m3 hi / lo: byte i of tile t <-> dim 128t + 32g + i
  bf16x8 qr[2];        // rope q (bf16 as given): element i of kk <-> rope dim 32kk + 8g + i
  int qsa = kUnitScale;  // E8M0 of 2^-e: the latent MFMAs scale q's rows back by it
  if (active) {
    // pass 1: per-head max |q| over the latent dims (the rope dims are used as given), as an
    // integer max of the bf16 magnitude bits, two values per instruction (lanes l, l^16, l^32,
    // l^48 hold one head)
    typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
    u16x2 mbits = {0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x4 v = qv.lat[4 * t + c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mbits = __builtin_elementwise_max(mbits, __builtin_bit_cast(u16x2, (uint32_t)v[i] & 0x7FFF7FFFu));
      }
    float amax = __uint_as_float((uint32_t)max(mbits[0], mbits[1]) << 16);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int e = 0;
    if (amax > 0.0f) {
      e = (int)floorf(__log2f(448.0f / amax));
      if (ldexpf(amax, e) > 448.0f) --e;
      e = max(-100, min(100, e));
    }
    qsa = kUnitScale - e;
    // pass 2: q * 2^e = hi + lo, both e4m3
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, qv.lat[4 * t + c]);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          int hi, lo;
          split_e4m3(ldexpf((float)v[4 * hf], e), ldexpf((float)v[4 * hf + 1], e), ldexpf((float)v[4 * hf + 2], e),
                     ldexpf((float)v[4 * hf + 3], e), hi, lo);
          qh[t][2 * c + hf] = hi;
          ql[t][2 * c + hf] = lo;
        }
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      qr[kk] = __builtin_bit_cast(bf16x8, qv.rope[kk]);
    }
  } else {
    // an idle score wave (fewer than 64 heads) keeps its heads' probability segments at zero
    for (int i = lane; i < 2 * 4 * kTT * 4; i += 64) {
      const int s = 4 * sw + (i & 3), j = (i >> 2) % kTT, tb = i / (4 * kTT);
      *reinterpret_cast<i32x2*>(sh.pbuf + tb * kPTile + j * kPRow + 8 * (s ^ pswz(j))) = i32x2{0, 0};
    }
  }

  // S = q K^T per 16-token half hf: lane holds token 16hf + tok and heads 16sw + 4g + r (r < 4),
  // so each lane needs the record scales of only its two tokens.
  const int tok = lane & 15;
  const float cq = p.scale_log2;  // scores come out in true units: softmax_scale * log2(e)
  const int pseg = (4 * sw + g) ^ pswz(tok);  // P' segment of this lane's four heads in token row tok

  float m_ref[4], m_raw[4], l_run[4];  // per output head: reference, running raw max, running sum
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_ref[r] = -INFINITY;
    m_raw[r] = -INFINITY;
    l_run[r] = 0.0f;
  }
  for (int pass = 0; pass < 2; ++pass) {
    for (int n = 0; n <= bk.ntiles; ++n) {
      lds_barrier();  // tile n staged; P'(n-2) consumed by the value waves
      if (!active || n >= bk.ntiles) continue;
      const uint8_t* tile = sh.stage + (n % kStages) * kTileBytes;
      const int nin = min(kTT, bk.total - n * kTT);
      f32x4 s[2];
      // every operand of the tile is read from LDS first, in the order the MFMAs use them
      bf16x8 rb[2][2];
      i32x4 kb[4][2][2];
      f32x4 sc[2];  // [hf]: the four tile scales of token 16hf + tok
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint8_t* kr = tile + 16 * (16 * hf + tok);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          rb[hf][kk] = *reinterpret_cast<const bf16x8*>(kr + (kRopeChunk + 4 * kk + g) * kCS);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        sc[hf] = *reinterpret_cast<const f32x4*>(tile + kScaleChunk * kCS + 16 * (16 * hf + tok));
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint8_t* kr = tile + 16 * (16 * hf + tok) + (8 * t + 2 * g) * kCS;
          kb[t][hf][0] = *reinterpret_cast<const i32x4*>(kr);
          kb[t][hf][1] = *reinterpret_cast<const i32x4*>(kr + kCS);
        }
      // keep all the reads ahead of the MFMAs: the scheduler would otherwise reuse a few operand
      // registers and wait out one LDS round trip per scale tile
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 acc = {};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) acc = mfma16_bf16(qr[kk], rb[hf][kk], acc);
        s[hf] = acc;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const i32x4 a0 = kb[t][hf][0], a1 = kb[t][hf][1];
          const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          f32x4 acc = mfma16_fp8(qh[t], a, f32x4{}, qsa);
          acc = mfma16_fp8(ql[t], a, acc, qsa);
#pragma unroll
          for (int r = 0; r < 4; ++r) s[hf][r] += sc[hf][t] * acc[r];
        }
      if (nin < kTT) {  // tail tile: entries past the end of the list get p = 0
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          if (16 * hf + tok >= nin) s[hf] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        m_raw[r] = __builtin_elementwise_maximum(m_raw[r], __builtin_elementwise_maximum(s[0][r], s[1][r]));
      if (pass == 0 && n == 0) {
        // the reference of the first pass: each head's max over the first tile (scaling by
        // cq > 0 commutes with the max)
#pragma unroll
        for (int r = 0; r < 4; ++r) m_ref[r] = max16(m_raw[r]) * cq;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[0][r] = fast_exp2(fmaf(s[0][r], cq, -m_ref[r]));
        s[1][r] = fast_exp2(fmaf(s[1][r], cq, -m_ref[r]));
        l_run[r] += s[0][r] + s[1][r];
      }
      // P'_t = bf16(p * scale(token, t)) as [t][token][head]
      uint8_t* pw = sh.pbuf + (n & 1) * kPBuf + tok * kPRow + 8 * pseg;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float f = sc[hf][t];
          const bf16x4 v = {(__bf16)(s[hf][0] * f), (__bf16)(s[hf][1] * f), (__bf16)(s[hf][2] * f),
                            (__bf16)(s[hf][3] * f)};
          *reinterpret_cast<bf16x4*>(pw + t * kPTile + 16 * hf * kPRow) = v;
        }
    }
    // a second pass, with the exact max as reference, only if some score outgrew the headroom
    bool over = false;
    float m_max[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_max[r] = active ? max16(m_raw[r]) * cq : -INFINITY;
      over |= m_max[r] > m_ref[r] + kRefHeadroom;
    }
    if (!__syncthreads_or(over)) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_ref[r] = m_max[r];
      m_raw[r] = -INFINITY;
      l_run[r] = 0.0f;
    }
  }

  // ---- per-head (max, sum) for the value waves; lse or the split partial
  if (active) {
    float l_tot[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) l_tot[r] = sum16(l_run[r]);
    if (tok == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * sw + 4 * g + r;
        const float mo = l_tot[r] > 0.0f ? m_ref[r] : -INFINITY;
        sh.ml[2 * h] = mo;
        sh.ml[2 * h + 1] = l_tot[r];
        const int head = bk.h_lo + h;
        if (p.splits == 1) {
          p.lse[(int64_t)bk.row * p.l_st + (int64_t)head * p.l_sh] =
              l_tot[r] > 0.0f ? (m_ref[r] + __log2f(l_tot[r])) * kLn2 : -INFINITY;
        } else {
          const int64_t pidx = ((int64_t)bk.row * p.splits + bk.split) * p.H + head;
          p.ws_ml[pidx * 2 + 0] = mo;
          p.ws_ml[pidx * 2 + 1] = l_tot[r];
        }
      }
    }
  }
  __syncthreads();  // sums visible to the value waves
}

// ---------------------------------------------------------------------------------------
// Value wave `vw` (0..3): output dims 128vw .. +127 (scale tile vw) of every head of the
// block; also the loader of the tiles.
__device__ __forceinline__ void value_role(const DecodeParams& p, Shared& sh, const Block& bk, int vw, int lane) {
  // O^T blocks o[db][hg]: dims 128vw + 32db + 8(r/4) + 4(lane/32) + r%4, head 32hg + lane%32
  f32x16 o[4][2];
  // P'^T operand of head block hg (heads 32hg + lane%32, tokens 16ks + 8(lane/32) .. +7) as two
  // transposed reads: in its 16-lane group G the lane a addresses token T0 + a/4 (T0 = 16ks +
  // 8(G/2), then + 4) and heads H0 + 4(a%4) .. +3 (H0 = 32hg + 16(G%2)), and receives head H0 + a
  // of the four tokens.  Offsets within a probability tile, less the 16ks token rows.
  int poff[2][2];
  {
    const int G = lane >> 4, a = lane & 15;
#pragma unroll
    for (int hg = 0; hg < 2; ++hg)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tk = 8 * (G >> 1) + (a >> 2) + 4 * half;
        const int seg = 8 * hg + 4 * (G & 1) + (a & 3);
        poff[hg][half] = tk * kPRow + 8 * (seg ^ pswz(tk));
      }
  }
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) o[db][hg] = f32x16{};
    for (int n = 0; n < kAhead && n < bk.ntiles; ++n)
      issue_tile(sh.stage + n * kTileBytes, lane_record(p, lane_slot(sh, n, bk.total, lane), lane), vw, lane);
    // the slot of the next tile to copy is read one step early, so its LDS round trip is
    // hidden behind the PV work instead of sitting between the barrier and the copy
    int next_slot = kAhead < bk.ntiles ? lane_slot(sh, kAhead, bk.total, lane) : 0;
    for (int n = 0; n <= bk.ntiles; ++n) {
      wait_tile(min(kAhead - 1, max(bk.ntiles - 1 - n, 0)), vw);  // tile n is in
      lds_barrier();  // tile n staged; P'(n-1) written; tile n-2 and P'(n-2) consumed
      if (n + kAhead < bk.ntiles) {
        issue_tile(sh.stage + ((n + kAhead) % kStages) * kTileBytes, lane_record(p, next_slot, lane), vw, lane);
        if (n + kAhead + 1 < bk.ntiles) next_slot = lane_slot(sh, n + kAhead + 1, bk.total, lane);
      }
      if (n == 0) continue;
      // ---- O^T += V^T P'^T for tile n-1
      const int m = n - 1;
      const uint8_t* tile = sh.stage + (m % kStages) * kTileBytes;
      const uint8_t* pb = sh.pbuf + (m & 1) * kPBuf + vw * kPTile;
      const int lh = lane >> 5;
      // tr8 row of this lane: record 8(lane/32) + (lane%16)/2, 8-byte half lane&1, chunk (lane/16)&1
      const int vrow = 16 * (8 * lh + ((lane & 15) >> 1)) + 8 * (lane & 1) + ((lane >> 4) & 1) * kCS;
      // all operands of the tile first (tokens past the end carry P' = 0 against real records)
      bf16x8 pf[2][2], va[2][4];
#pragma unroll
      for (int ks = 0; ks < kTT / 16; ++ks) {
#pragma unroll
        for (int hg = 0; hg < 2; ++hg) {
          const uint8_t* src = pb + ks * 16 * kPRow;
          const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS i16x4*)(src + poff[hg][0]));
          const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS i16x4*)(src + poff[hg][1]));
          pf[ks][hg] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int cb = 4 * vw + db;  // global 32-dim block: chunks 2cb, 2cb + 1
          const i32x2 raw =
              __builtin_amdgcn_ds_read_tr8_b64_v2i32((SMLA_LDS i32x2*)(tile + 2 * cb * kCS + 256 * ks + vrow));
          va[ks][db] = widen_fp8x8((uint32_t)raw[0], (uint32_t)raw[1]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < kTT / 16; ++ks)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int hg = 0; hg < 2; ++hg) o[db][hg] = mfma32_bf16(va[ks][db], pf[ks][hg], o[db][hg]);
    }
    if (!__syncthreads_or(false)) break;
  }
  __syncthreads();  // the score waves' (max, sum) are in LDS
  stage_output(p, sh.ml, staging(sh), o, vw, lane);
}

__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) Shared sh;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;

  Block bk;
  if (!block_of(p, bk)) return;
  QRaw qv;
  if (wave < 4 && 16 * wave < bk.nh) load_q(p, bk, wave, lane, qv);
  bk.total = compact_slots(p, bk, sh, tid, wave, lane);
  bk.ntiles = (bk.total + kTT - 1) / kTT;

  // The two roles run the same number of workgroup barriers, one per loop step.
  if (wave < 4)
    score_role(p, sh, bk, qv, wave, lane);
  else
    value_role(p, sh, bk, wave - 4, lane);
  __syncthreads();  // output rows staged
  store_rows(p, bk, staging(sh), tid);
  if (p.splits == 1) return;

  if (arrive_last(p, bk, sh, tid)) combine_splits(p, bk, sh, tid);

}

__global__ void zero_counters(int32_t* cnt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) cnt[i] = 0;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream) {
  const int64_t items = (int64_t)p.T * plan.head_blocks * plan.splits;
  const unsigned grid = (unsigned)((items + 7) / 8 * 8);
  if (plan.splits > 1) {
    // arrival counters start at zero on every call (a kernel, not a memset node, so the
    // call stays safe to capture in a graph)
    const int64_t n = (int64_t)p.T * plan.head_blocks;
    hipLaunchKernelGGL(zero_counters, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p.ws_cnt, n);
  }
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
