// Sparse MLA decode over per-row top-k slot lists against the packed fp8_ds_mla cache.
//
// Computes, per query row t and head h, softmax attention over the row's own candidate
// records and returns out[t,h,0:512] and lse[t,h] (page "FlashMLA sparse fp8 path gains
// DCP and MTP", "Key source snippets" and "Implementation breakdown" steps 1-3; page
// "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA", "Why").
//
// gfx950 design
//  * A workgroup owns one row, a block of up to 64 of its heads and one range of its top-k
//    list.  The two head blocks of an H = 128 row are consecutive work items that run side by
//    side on one XCD, so the second copy of each record comes from that XCD's L2.
//  * Eight waves, two per SIMD: four score waves and four value waves.  A wave alone on a SIMD
//    issues its vector instructions slowly and leaves every LDS and MFMA latency exposed; with
//    a score wave and a value wave on each SIMD, one runs while the other waits, and their
//    MFMA and vector streams overlap.  Each role runs its own loop, so the score waves' q and
//    the value waves' output accumulators share the same registers (256 per wave).
//  * Score wave s scores tokens 16(s & 1) .. + 15 of each 32-record tile for heads
//    32(s >> 1) .. + 31 of the block (q: 144 VGPRs), on v_mfma_f32_16x16x32_bf16 as
//    S^T = K . q^T.  The record codes are widened exactly from e4m3 to bf16 for the A operand,
//    one widened operand feeding the MFMAs of both 16-head blocks; q is the B operand as given.
//    (The scaled fp8 MFMA sums its products with about 12 bits of precision relative to the
//    largest product, so splitting q into fp8 terms is not exact; the bf16 MFMA accumulates in
//    fp32.)  Each 128-dim scale tile is four k-steps; its fp32 record scale then multiplies the
//    tile's partial scores.  The score wave then runs the softmax of its scores: base 2, against
//    a per-head reference max fixed at the first tile (the two waves that share a head exchange
//    their halves of that max through LDS once, and the reference also carries 2^e, e the
//    exponent of the first tile's largest record scale); later probabilities are 2^(s - ref) and
//    may exceed 2^-e; should a score exceed the reference by more than 2^12, or a product
//    p * scale overflow fp16 below, the workgroup recomputes the range once with the exact max
//    and the exponent of the range's largest scale, so the output accumulators are never
//    rescaled inside the loop.
//  * Value wave v copies a quarter of every tile HBM -> LDS and produces the output of every
//    head of the block over the latent dims 128v .. 128v + 127, i.e. over record scale tile v
//    (128 dims x 64 heads of fp32 accumulators), as O^T = V^T . P'^T on
//    v_mfma_f32_32x32x16_f16: V^T fragments come from the staged tile through
//    ds_read_b64_tr_b8 and are widened exactly to fp16; P' = p * scale(token, v) is rounded once
//    to fp16 (11 significant bits, four times finer than bf16) from the fp32 probabilities,
//    which cross from the score waves through LDS, double-buffered.  Step n scores tile n and outputs tile n - 1; one workgroup barrier per
//    step orders that hand-over and the tile ring.
//  * Gather: the row's slot range is compacted in LDS (-1 and out-of-range entries dropped),
//    then tiles of 32 records are copied with global_load_lds, two tiles ahead.  A tile sits
//    chunk-major in LDS: [40 chunk rows][32 records][16 B] for the 512 codes and 64 rope
//    values, then the record scales as [4 tiles][32 tokens] fp32.  Odd chunk rows hold record r
//    at position r ^ 8 and odd scale rows token r at r ^ 8, so the transposed value reads of two
//    lane groups fall in different banks.
//  * Output rows are staged through LDS and written as whole rows.  Split-K over the top-k list
//    leaves fp32 partials and (max, sum) pairs that a second kernel merges (split_combine.hip);
//    a row with no valid entry yields out = 0, lse = -inf.

#include "decode_common.h"

namespace smla {
namespace {

using namespace dec;

constexpr int kRT = 512;                              // four score waves + four value waves
constexpr int kRH = kRowHeads;                        // heads one workgroup covers
constexpr int kTT = 32;                               // records per tile
constexpr int kChunkRows = 40;                        // 32 code + 8 rope chunks of 16 bytes per record
constexpr int kCS = 16 * kTT;                         // bytes per chunk row (512)
constexpr int kScaleBase = kChunkRows * kCS;          // record scales [4][32] fp32 after the chunk rows
constexpr int kTileBytes = kScaleBase + 4 * kTT * 4;  // 20992
constexpr int kStages = 4;                            // tile ring: scores on n, values on n-1,
constexpr int kAhead = 2;                             //   copies in flight for n+1, n+2
constexpr int kPRow = 4 * kTT + 16;                   // fp32 probabilities of one head for one tile, padded
constexpr int kPBuf = kRH * kPRow;                    // 9 KB: the probabilities of one tile
constexpr int kStg32 = 4 * kLatent + 16;              // staged output rows: fp32 and bf16 pitches
constexpr int kStg16 = 2 * kLatent + 16;              //   (16 bytes of padding: rows 4 banks apart)

// First-pass headroom (log2 units): probabilities stay below 2^12 times the power of two that
// scales them (see score_role), so p * scale fits fp16 unless a later record's scale is far
// larger than the first tile's; such a product overflows, the value waves see a non-finite
// accumulator and the range is repeated with exact references.
constexpr float kPHeadroom = 12.0f;

static_assert(kRH == 64, "score waves: 2 token halves x 2 head halves of 32; output blocks of 32 heads");
static_assert(kStages == kAhead + 2, "ring: the tile being scored, the one being valued, the copies");
static_assert(32 * kStg32 <= kStages * kTileBytes && 64 * kStg16 <= kStages * kTileBytes, "output staging fits");

struct RowShared {
  uint8_t stage[kStages * kTileBytes];
  uint8_t pbuf[2 * kPBuf];  // [buffer][head][token] fp32, head rows 144 bytes apart
  int32_t clist[kMaxEntriesPerSplit];
  float xch[2][kRH];  // per token half: the block's per-head maxima or sums, exchanged between halves
  float smax[kRT / 64];  // largest record scales: tile 0's in [0] (first pass), per wave when a range is repeated
  int32_t wave_cnt[kRT / 64];
};

// Position of record r in chunk row c of a tile, and of token r in scale row t.
__device__ __forceinline__ int rpos(int c, int r) { return r ^ ((c & 1) << 3); }

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// Eight e4m3 codes -> eight fp16 values, exactly (4 exponent and 3 mantissa bits fit fp16's 5 and
// 10, subnormal codes included).
__device__ __forceinline__ f16x8 widen8h(uint32_t lo, uint32_t hi) {
  const f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
  const f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
  const f16x2 c = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
  const f16x2 d = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3), cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x16 mfma32_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Largest value over all 64 lanes.
__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, m));
  return x;
}

// floor(log2(x)) of a positive record scale as a float (0 for 0; the exponent field of x, so
// 2^-e scales exactly), at least -100: probabilities carry 2^-e, and with e down to -100 they and
// their sums stay inside fp32 (scales below 2^-100 only make their products underflow fp16,
// which at such magnitudes costs nothing measurable).
__device__ __forceinline__ float scale_exponent(float x) {
  const int e = (int)((__float_as_uint(x) >> 23) & 0xffu) - 127;
  return x > 0.0f ? (float)max(e, -100) : 0.0f;
}

// The largest record scale of the workgroup's compacted entries, read from the records (all
// eight waves; only when a range is repeated): this wave's part goes to sh.smax.
template <typename Shared>
__device__ __forceinline__ void scan_scales(const DecodeParams& p, const Block& bk, Shared& sh, int w, int tid) {
  float m = 0.0f;
  for (int i = tid; i < bk.total; i += kRT) {
    const f32x4 sc = *reinterpret_cast<const f32x4*>(p.kv + (int64_t)sh.clist[i] * kRecordBytes + kScaleOffset);
    m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[0], sc[1]),
                                                                       __builtin_elementwise_maximum(sc[2], sc[3])));
  }
  m = wave_max64(m);
  if ((tid & 63) == 0) sh.smax[w] = m;
}

// e of a repeated range: the exponent of the largest record scale that scan_scales found (at
// most 126, so that 2^-e and 2^e are normal floats).
template <typename Shared>
__device__ __forceinline__ int repeat_exponent(const Shared& sh) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kRT / 64; ++k) m = __builtin_elementwise_maximum(m, sh.smax[k]);
  return min((int)scale_exponent(m), 126);
}

// Four e4m3 codes -> four bf16 values, exactly.
__device__ __forceinline__ bf16x4 widen4(uint32_t x) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  return bf16x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ bf16x8 join8(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) { return join8(widen4(lo), widen4(hi)); }

// One global_load_lds_dwordx4: lane i's 16 bytes from src land at LDS lds + 16 i.  (No immediate
// offset: on this path it would move the LDS destination as well as the source.)
__device__ __forceinline__ void dma16(const uint8_t* src, const uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(SMLA_LDS void*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
}
// One global_load_lds_dword: lane i's 4 bytes land at LDS lds + 4 i.
__device__ __forceinline__ void dma4(const uint8_t* src, const uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(SMLA_LDS void*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory");
}

// Copies per tile and value wave: five chunk-row pairs, and one scale row pair for waves 0, 1.
__device__ __forceinline__ void wait_row_tile(bool newer_in_flight, int v) {
  if (!newer_in_flight) wait_vmcnt<0>();
  else if (v < 2) wait_vmcnt<6>();
  else wait_vmcnt<5>();
}

// HBM -> LDS copy of one tile by value wave v.  Load j (0..19) fills chunk rows 2j (lanes 0-31)
// and 2j + 1 (lanes 32-63); wave v issues j = v, v + 4, .., v + 16.  Lane i writes position i & 31
// of its row, i.e. record (i & 31) ^ 8 (i >> 5), whose bytes start at `rec`.  Chunk c of a record
// starts at byte 16c (codes) or 16c + 16 (rope, after the 16 scale bytes).  Waves 0 and 1 also
// copy scale tiles 2v and 2v + 1 of the same records into the scale rows.
__device__ __forceinline__ void issue_row_tile(uint8_t* tile, const uint8_t* rec, int v, int lane) {
  const uint8_t* src = rec + 16 * (lane >> 5) + 32 * v;
  uint8_t* dst = tile + 1024 * v;
  dma16(src, dst);
  dma16(src + 128, dst + 4096);
  dma16(src + 256, dst + 8192);
  dma16(src + 384, dst + 12288);
  dma16(src + 528, dst + 16384);
  if (v < 2) dma4(rec + kScaleOffset + 8 * v + 4 * (lane >> 5), tile + kScaleBase + 256 * v);
}

// Slot of this lane's copy record in tile n; entries past the end repeat the last one.
__device__ __forceinline__ int copy_slot(const RowShared& sh, int n, int total, int lane) {
  return sh.clist[min(n * kTT + ((lane & 31) ^ ((lane >> 5) << 3)), total - 1)];
}

// ---------------------------------------------------------------------------------------------
// Score side

// q of a score lane as B operands of the score MFMAs: head block hb (heads 32hh + 16hb + r of the
// block), lane group G = lane >> 4.  Latent k-steps 2p and 2p + 1 together take dims 64p .. 64p + 63:
// lat[hb][2p + h] = dims 64p + 16G + 8h + 0..7; rope k-step u: rope[hb][u] = rope dims 32u + 8G +
// 0..7.  The record operand puts the same dims in the same k-slots.
struct QOps {
  bf16x8 lat[2][16];
  bf16x8 rope[2][2];
};

template <bool kFull>
__device__ __forceinline__ void load_q_row(const DecodeParams& p, int row, int h_first, int G, QOps& q) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int h = h_first + 16 * hb;
    if (!kFull && h >= p.H) {
#pragma unroll
      for (int j = 0; j < 16; ++j) q.lat[hb][j] = bf16x8{};
      q.rope[hb][0] = q.rope[hb][1] = bf16x8{};
      continue;
    }
    const uint16_t* qp = p.q + (int64_t)row * p.q_st + (int64_t)h * p.q_sh;
#pragma unroll
    for (int j = 0; j < 16; ++j) q.lat[hb][j] = *reinterpret_cast<const bf16x8*>(qp + 64 * (j >> 1) + 16 * G + 8 * (j & 1));
    q.rope[hb][0] = *reinterpret_cast<const bf16x8*>(qp + kLatent + 8 * G);
    q.rope[hb][1] = *reinterpret_cast<const bf16x8*>(qp + kLatent + 32 + 8 * G);
  }
}

// Raw scores (before the softmax scale) of this wave's tile quarter: s[hb][i] <-> head
// 32hh + 16hb + r, token 16tb + 4G + i.
struct Scores {
  f32x4 s[2];
};

// The record operands of latent k-steps 2p and 2p + 1 for token tok = 16tb + r are the two halves
// of chunk 4p + G (dims 64p + 16G .. + 15), one ds_read_b128 at kb + 4p kCS, so that a quarter-wave
// reads 16 whole chunks of one chunk row; each pair is read three pairs ahead and each half widened
// in the k-step before its MFMAs.  Rope k-step u reads rope chunk 4u + G (chunk row 32 + 4u + G).
// Tile t's partial scores (k-steps 4t .. 4t + 3) are scaled and added during k-steps 4t + 5 ..
// 4t + 7, and after the loop for the last tile.
__device__ __forceinline__ Scores score_tile(const uint8_t* tile, const QOps& q, int tb, int G, int r) {
  const int tok = 16 * tb + r;
  const uint8_t* kb = tile + G * kCS + 16 * (tok ^ (8 * (G & 1)));
  const uint8_t* rb = tile + (32 + G) * kCS + 16 * (tok ^ (8 * (G & 1)));
  const float* srow = reinterpret_cast<const float*>(tile + kScaleBase);
  const int sx = 16 * tb + 4 * G;  // first of this lane's four score tokens
  Scores S;
  i32x4 kr[8];
  const bf16x8 ra0 = *reinterpret_cast<const bf16x8*>(rb);
  const bf16x8 ra1 = *reinterpret_cast<const bf16x8*>(rb + 4 * kCS);
#pragma unroll
  for (int p = 0; p < 3; ++p) kr[p] = *reinterpret_cast<const i32x4*>(kb + 4 * p * kCS);
  S.s[0] = mfma16_bf16(ra0, q.rope[0][0], f32x4{});
  S.s[1] = mfma16_bf16(ra0, q.rope[1][0], f32x4{});
  S.s[0] = mfma16_bf16(ra1, q.rope[0][1], S.s[0]);
  S.s[1] = mfma16_bf16(ra1, q.rope[1][1], S.s[1]);
  bf16x8 wa = widen8((uint32_t)kr[0][0], (uint32_t)kr[0][1]);  // k-step 0: first half of pair 0
  f32x4 acc[2][2];  // partial scores: [tile parity][head block]
  f32x4 sc = {};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int t = j >> 2, ph = t & 1, tp = t - 1;
    acc[ph][0] = mfma16_bf16(wa, q.lat[0][j], (j & 3) == 0 ? f32x4{} : acc[ph][0]);
    acc[ph][1] = mfma16_bf16(wa, q.lat[1][j], (j & 3) == 0 ? f32x4{} : acc[ph][1]);
    if (j + 1 < 16) {
      const i32x4& n = kr[(j + 1) >> 1];
      wa = (j + 1) & 1 ? widen8((uint32_t)n[2], (uint32_t)n[3]) : widen8((uint32_t)n[0], (uint32_t)n[1]);
    }
    if ((j & 1) && j / 2 + 3 < 8) kr[j / 2 + 3] = *reinterpret_cast<const i32x4*>(kb + 4 * (j / 2 + 3) * kCS);
    if (t >= 1 && (j & 3) == 1) sc = *reinterpret_cast<const f32x4*>(srow + kTT * tp + (sx ^ (8 * (tp & 1))));
    if (t >= 1 && (j & 3) >= 2) {  // scores += scale(token, t - 1) * partial of tile t - 1
      const int hb = (j & 3) - 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) S.s[hb][i] = fmaf(sc[i], acc[tp & 1][hb][i], S.s[hb][i]);
    }
  }
  sc = *reinterpret_cast<const f32x4*>(srow + kTT * 3 + (sx ^ 8));
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) S.s[hb][i] = fmaf(sc[i], acc[1][hb][i], S.s[hb][i]);
  return S;
}

struct SoftmaxState {
  float m_ref[2], m_raw[2], l_run[2];
  float shift[2];  // the power of two folded into m_ref (log2 units)
};

// A reference below this magnitude (log2 units) takes the integer shift exactly; a larger one is
// left unshifted (its products are checked like any other).
constexpr float kExactFold = 1048576.0f;

// Softmax of this lane's scores against each head's reference: probabilities to the heads' rows
// of `pn`, running raw max and sum.  kMask: entries at or past `nin` get p = 0 (only a range's
// last tile can hold such entries).  kExact: the
// reference is the largest rounded product score * cq, and each exponent is that rounded product
// minus the reference, so none exceeds 0 (a fused score * cq - ref exceeds 0 by up to half an ulp
// of the reference: more than 1 once references pass 2^25, an fp32 overflow of p past 2^31), and
// the probabilities handed to the value waves carry c = 2^-e (the sums do not).
template <bool kMask, bool kExact>
__device__ __forceinline__ void softmax_tile(const Scores& S, int tb, int hh, int G, int r, int nin, float cq,
                                             SoftmaxState& st, uint8_t* pn, float c) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    f32x4 t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = !kMask || 16 * tb + 4 * G + i < nin ? S.s[hb][i] : -INFINITY;
      st.m_raw[hb] = __builtin_elementwise_maximum(st.m_raw[hb], v);
      t[i] = fast_exp2(kExact ? rounded_product_minus(v, cq, st.m_ref[hb]) : fmaf(v, cq, -st.m_ref[hb]));
      st.l_run[hb] += t[i];
    }
    if (kExact) t *= c;
    const int row = 32 * hh + 16 * hb + r;
    *reinterpret_cast<f32x4*>(pn + row * kPRow + 16 * (4 * tb + G)) = t;
  }
}

// ---------------------------------------------------------------------------------------------
// Value side

// Raw V^T codes of a tile for value wave v: raw[ks][db] = dims 128v + 32db + (lane & 31) of records
// 16ks + 8(lane >> 5) + 0..7.  Lane group G reads records 16ks + 8(G >> 1) + 0..7 of chunk
// 8v + 2db + (G & 1) through ds_read_b64_tr_b8.
struct VRaw {
  i32x2 raw[2][4];
};
__device__ __forceinline__ void load_vraw(const uint8_t* tile, int v, int lane, VRaw& f) {
  const int G = lane >> 4, a = lane & 15;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int c = 8 * v + 2 * db + (G & 1);
      f.raw[ks][db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (SMLA_LDS i32x2*)(tile + c * kCS + 16 * rpos(c, 16 * ks + 8 * (G >> 1) + (a >> 1)) + 8 * (a & 1)));
    }
}

// Output of tile `tile` over dims 128v .. 128v + 127 for the block's 64 heads, with the tile's raw
// V^T codes `cur` (read a step earlier) and fp32 probabilities `pb` ([head][token]); the codes of
// the next tile are read into `nxt` (from `next_tile`, when non-null) once the MFMAs are under
// way.  O[db][hb]: dims 128v + 32db + 8(i/4) + 4(lane/32) + i%4, head 32hb + (lane & 31).  The
// probabilities and scales are requested first and the first token half's fragments are widened
// while they arrive; then sixteen MFMAs in chunks ci = (ks, hb) = (ci >> 1, ci & 1) of four
// (db = 0..3), beside them the P' operand of the next chunk, the probabilities two chunks ahead,
// and the second token half's fragments, each widened after the last use of the one it replaces.
// (Head rows past the block's heads hold stale probabilities; their output columns are never
// stored.)
__device__ __forceinline__ void value_tile(const uint8_t* tile, const uint8_t* pb, const VRaw& cur, f32x16 (&O)[4][2],
                                           int v, int lane, const uint8_t* next_tile, VRaw& nxt) {
  const int g = lane >> 5, r32 = lane & 31;
  const float* srow = reinterpret_cast<const float*>(tile + kScaleBase) + kTT * v;
  auto pread = [&](int ci, f32x4& p0, f32x4& p1) {  // tokens 16ks + 8g + 0..7 of head 32hb + r32
    const int ks = ci >> 1, row = 32 * (ci & 1) + r32;
    const uint8_t* pr = pb + row * kPRow;
    p0 = *reinterpret_cast<const f32x4*>(pr + 16 * (4 * ks + 2 * g));
    p1 = *reinterpret_cast<const f32x4*>(pr + 16 * (4 * ks + 2 * g + 1));
  };
  auto sread = [&](int ks, f32x4& s0, f32x4& s1) {  // scales of tile v for tokens 16ks + 8g + 0..7
    const int x = (16 * ks + 8 * g) ^ (8 * (v & 1));
    s0 = *reinterpret_cast<const f32x4*>(srow + x);
    s1 = *reinterpret_cast<const f32x4*>(srow + x + 4);
  };
  auto pp4 = [](const f32x4& p, const f32x4& s) {
    return f16x4{(_Float16)(p[0] * s[0]), (_Float16)(p[1] * s[1]), (_Float16)(p[2] * s[2]), (_Float16)(p[3] * s[3])};
  };
  auto join8h = [](const f16x4& lo, const f16x4& hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); };

  f32x4 sv[2][2];
  f32x4 pa[2], pnx[2];
  pread(0, pa[0], pa[1]);
  sread(0, sv[0][0], sv[0][1]);
  pread(1, pnx[0], pnx[1]);
  sread(1, sv[1][0], sv[1][1]);
  f16x8 vt[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) vt[db] = widen8h((uint32_t)cur.raw[0][db][0], (uint32_t)cur.raw[0][db][1]);
  f16x8 pp = join8h(pp4(pa[0], sv[0][0]), pp4(pa[1], sv[0][1]));
  f16x4 nlo, nhi;
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    const int hb = ci & 1, nks = (ci + 1) >> 1;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      O[db][hb] = mfma32_f16(vt[db], pp, O[db][hb]);
      if (ci == 1) vt[db] = widen8h((uint32_t)cur.raw[1][db][0], (uint32_t)cur.raw[1][db][1]);  // second token half
      if (ci < 3 && db == 0) nlo = pp4(pnx[0], sv[nks][0]);
      if (ci < 3 && db == 1) {
        nhi = pp4(pnx[1], sv[nks][1]);
        if (ci < 2) pread(ci + 2, pnx[0], pnx[1]);
      }
      if (ci < 3 && db == 3) pp = join8h(nlo, nhi);
      if (ci == 2 && db == 0 && next_tile) load_vraw(next_tile, v, lane, nxt);
    }
  }
}

// Sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (every lane gets it).
__device__ __forceinline__ float sum4x16(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Staged output rows -> global memory: `rows` rows of the block starting at head row `h0`, from
// sh.stage with pitch kStg32 (fp32) or kStg16 (bf16), 16 bytes per thread and instruction; rows
// past the block's heads are not written.  The stores are non-temporal: nothing reads the output
// again here, and streaming it past L2 leaves the L2 lines of the records to the other head block.
__device__ __forceinline__ void store_staged(const DecodeParams& p, const Block& bk, const RowShared& sh, int h0,
                                             int rows, int tid) {
  if (p.splits > 1 || p.out_fp32) {
    float* base;
    int64_t hstride;
    if (p.splits > 1) {  // this split's unnormalised partial
      base = p.ws_o + ((int64_t)bk.row * p.splits + bk.split) * p.H * kLatent;
      hstride = kLatent;
    } else {
      base = reinterpret_cast<float*>(p.out) + (int64_t)bk.row * p.o_st;
      hstride = p.o_sh;
    }
    constexpr int kChunks = 4 * kLatent / 16;
    for (int c = tid; c < rows * kChunks; c += kRT) {
      const int row = c / kChunks, col = c % kChunks;
      if (h0 + row < bk.nh) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(sh.stage + row * kStg32 + 16 * col);
        __builtin_nontemporal_store(v,
                                    reinterpret_cast<f32x4*>(base + (int64_t)(bk.h_lo + h0 + row) * hstride + 4 * col));
      }
    }
  } else {
    __bf16* base = reinterpret_cast<__bf16*>(p.out) + (int64_t)bk.row * p.o_st;
    constexpr int kChunks = 2 * kLatent / 16;
    for (int c = tid; c < rows * kChunks; c += kRT) {
      const int row = c / kChunks, col = c % kChunks;
      if (h0 + row < bk.nh) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(sh.stage + row * kStg16 + 16 * col);
        __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(base + (int64_t)(bk.h_lo + h0 + row) * p.o_sh + 8 * col));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// The two roles.  Both run the same sequence of workgroup barriers:
//   per pass with tiles: B0 (tile 0 staged), X (first pass only: reference exchange),
//   B1 .. B(ntiles-1) (tile n staged, p(n - 1) published), Blast (p(last) published);
//   per pass: the "over" vote; after a vote for a second pass: two exchange barriers.
//   Then E (sums published) and the output staging rounds.

// One pass of a score wave over the range: scores, softmax and probabilities of every tile.
// kRepeat: a repeated range, whose references are the exact maxima and whose probabilities go to
// the value waves times c.
template <bool kRepeat>
__device__ __forceinline__ void score_pass(const Block& bk, RowShared& sh, const QOps& q, int tb, int hh, int G, int r,
                                           float cq, SoftmaxState& st, float c) {
  if (bk.ntiles == 0) return;
  lds_barrier();  // B0
  const Scores S = score_tile(sh.stage, q, tb, G, r);
  const int nin = min(kTT, bk.total);
  if (!kRepeat) {  // reference: the max of each head over tile 0, from both token halves
    float mx[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      mx[hb] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mx[hb] = __builtin_elementwise_maximum(mx[hb], 16 * tb + 4 * G + i < nin ? S.s[hb][i] : -INFINITY);
      mx[hb] = max4x16(mx[hb]);
      if (G == 0) sh.xch[tb][32 * hh + 16 * hb + r] = mx[hb];
    }
    lds_barrier();  // X
    // p * scale enters the output MFMAs as fp16: the reference also carries 2^e, e the exponent
    // of tile 0's largest record scale (found by the value waves), so the products of the first
    // tile stay below 2^13; the shift cancels in out = O / L and is part of the LSE.  A reference
    // too large to take the integer e exactly keeps e = 0.
    const float e = scale_exponent(sh.smax[0]);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float m = __builtin_elementwise_maximum(mx[hb], sh.xch[tb ^ 1][32 * hh + 16 * hb + r]) * cq;
      st.shift[hb] = __builtin_fabsf(m) < kExactFold ? e : 0.0f;
      st.m_ref[hb] = m + st.shift[hb];
    }
  }
  if (bk.ntiles > 1) softmax_tile<false, kRepeat>(S, tb, hh, G, r, nin, cq, st, sh.pbuf, c);
  else softmax_tile<true, kRepeat>(S, tb, hh, G, r, nin, cq, st, sh.pbuf, c);
  for (int n = 1; n < bk.ntiles; ++n) {
    lds_barrier();  // Bn
    const Scores Sn = score_tile(sh.stage + (n % kStages) * kTileBytes, q, tb, G, r);
    if (n + 1 < bk.ntiles) softmax_tile<false, kRepeat>(Sn, tb, hh, G, r, kTT, cq, st, sh.pbuf + (n & 1) * kPBuf, c);
    else softmax_tile<true, kRepeat>(Sn, tb, hh, G, r, bk.total - n * kTT, cq, st, sh.pbuf + (n & 1) * kPBuf, c);
  }
  lds_barrier();  // Blast
}

__device__ __forceinline__ void score_role(const DecodeParams& p, const Block& bk, RowShared& sh, int s, int lane,
                                           const QOps& q) {
  const int G = lane >> 4, r = lane & 15;
  const int tb = s & 1, hh = s >> 1;
  const float cq = p.scale_log2;
  SoftmaxState st;
  st.m_ref[0] = st.m_ref[1] = -INFINITY;
  st.shift[0] = st.shift[1] = 0.0f;
  float c = 1.0f;  // a repeated range: 2^-e on the probabilities of the output MFMAs
  for (int pass = 0; pass < 2; ++pass) {
    st.m_raw[0] = st.m_raw[1] = -INFINITY;
    st.l_run[0] = st.l_run[1] = 0.0f;
    if (pass == 0) score_pass<false>(bk, sh, q, tb, hh, G, r, cq, st, 1.0f);
    else score_pass<true>(bk, sh, q, tb, hh, G, r, cq, st, c);
    // a second pass, with the exact max as reference, only if some score outgrew the headroom or
    // (the value waves' vote) some fp16 product p * scale overflowed
    float mm[2];
    bool over = false;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      mm[hb] = max4x16(st.m_raw[hb] * cq);
      over = over || mm[hb] > st.m_ref[hb] - st.shift[hb] + kPHeadroom;
    }
    if (!__syncthreads_or(over) || pass == 1) break;  // the value waves vote too: an fp16 product overflowed
    // the repeat: exact maxima as references (p <= 1), and the probabilities of the output MFMAs
    // times 2^-e, e the exponent of the largest scale of every record in range (scan_scales), so
    // that every fp16 product is below 2 however large the references are; the value waves
    // multiply their output by 2^e
    scan_scales(p, bk, sh, s, 64 * s + lane);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      if (G == 0) sh.xch[tb][32 * hh + 16 * hb + r] = mm[hb];
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      st.m_ref[hb] = __builtin_elementwise_maximum(mm[hb], sh.xch[tb ^ 1][32 * hh + 16 * hb + r]);
      st.shift[hb] = 0.0f;
    }
    c = ldexpf(1.0f, -repeat_exponent(sh));
    __syncthreads();  // the exchange slots are free again
  }
  // per-head sums: over the lane groups, then over the two token halves
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float l = sum4x16(st.l_run[hb]);
    if (G == 0) sh.xch[tb][32 * hh + 16 * hb + r] = l;
  }
  __syncthreads();  // E
  if (tb == 0 && G == 0) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hl = 32 * hh + 16 * hb + r;
      if (hl >= bk.nh) continue;
      const float lt = sh.xch[0][hl] + sh.xch[1][hl];
      const int head = bk.h_lo + hl;
      if (p.splits == 1) {
        p.lse[(int64_t)bk.row * p.l_st + (int64_t)head * p.l_sh] =
            lt > 0.0f ? (st.m_ref[hb] + __log2f(lt)) * kLn2 : -INFINITY;
      } else {
        const int64_t pidx = ((int64_t)bk.row * p.splits + bk.split) * p.H + head;
        p.ws_ml[pidx * 2 + 0] = lt > 0.0f ? st.m_ref[hb] : -INFINITY;
        p.ws_ml[pidx * 2 + 1] = lt;
      }
    }
  }
  // output staging rounds: the value waves stage, everyone stores
  const int tid = 64 * s + lane;
  if (p.splits > 1 || p.out_fp32) {
#pragma unroll 1
    for (int hb = 0; hb < 2; ++hb) {
      __syncthreads();  // staged
      store_staged(p, bk, sh, 32 * hb, 32, tid);
      __syncthreads();  // stored
    }
  } else {
    __syncthreads();
    store_staged(p, bk, sh, 0, kRH, tid);
  }
}

__device__ __forceinline__ void value_role(const DecodeParams& p, const Block& bk, RowShared& sh, int v, int lane) {
  f32x16 O[4][2];
  float up = 1.0f;  // 2^e: a repeated range's probabilities carry 2^-e, given back to the output here
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) O[db][hb] = f32x16{};
    if (bk.ntiles > 0) {
      for (int n = 0; n < kAhead && n < bk.ntiles; ++n)
        issue_row_tile(sh.stage + n * kTileBytes, p.kv + (int64_t)copy_slot(sh, n, bk.total, lane) * kRecordBytes, v,
                       lane);
      int next_slot = kAhead < bk.ntiles ? copy_slot(sh, kAhead, bk.total, lane) : 0;
      wait_row_tile(bk.ntiles > 1, v);
      lds_barrier();  // B0
      if (kAhead < bk.ntiles) {
        issue_row_tile(sh.stage + kAhead * kTileBytes, p.kv + (int64_t)next_slot * kRecordBytes, v, lane);
        if (kAhead + 1 < bk.ntiles) next_slot = copy_slot(sh, kAhead + 1, bk.total, lane);
      }
      VRaw va, vb;  // raw V^T codes of the tile output now (va) and of the next one (vb)
      load_vraw(sh.stage, v, lane, vb);
      if (pass == 0) {  // tile 0's largest record scale, for the score waves' reference
        if (v == 0) {
          const float2 s2 = *reinterpret_cast<const float2*>(sh.stage + kScaleBase + 8 * lane);
          const float m = wave_max64(__builtin_elementwise_maximum(s2.x, s2.y));
          if (lane == 0) sh.smax[0] = m;
        }
        lds_barrier();  // X
      }
      for (int n = 1; n < bk.ntiles; ++n) {
        wait_row_tile(n + 1 < bk.ntiles, v);
        lds_barrier();  // Bn: tile n staged; p(n - 1) published; tile n - 2 and p(n - 2) consumed
        if (n + kAhead < bk.ntiles) {
          issue_row_tile(sh.stage + ((n + kAhead) % kStages) * kTileBytes, p.kv + (int64_t)next_slot * kRecordBytes,
                         v, lane);
          if (n + kAhead + 1 < bk.ntiles) next_slot = copy_slot(sh, n + kAhead + 1, bk.total, lane);
        }
        va = vb;
        value_tile(sh.stage + ((n - 1) % kStages) * kTileBytes, sh.pbuf + ((n - 1) & 1) * kPBuf, va, O, v, lane,
                   sh.stage + (n % kStages) * kTileBytes, vb);
      }
      lds_barrier();  // Blast
      const int n = bk.ntiles;
      value_tile(sh.stage + ((n - 1) % kStages) * kTileBytes, sh.pbuf + ((n - 1) & 1) * kPBuf, vb, O, v, lane, nullptr,
                 va);
    }
    // an fp16 product p * scale that overflowed made every output dim of its head inf or NaN (inf
    // times a zero code included), so one accumulator per head tells: repeat the range
    const bool bad = !__builtin_isfinite(O[0][0][0]) || !__builtin_isfinite(O[0][1][0]);
    if (!__syncthreads_or(bad) || pass == 1) break;
    scan_scales(p, bk, sh, 4 + v, 256 + 64 * v + lane);
    __syncthreads();
    up = ldexpf(1.0f, repeat_exponent(sh));
    __syncthreads();
  }
  __syncthreads();  // E: the per-head sums are in sh.xch
  // normalise and stage: dims 128v + 32db + 8qd + 4g + 0..3 of head 32hb + (lane & 31)
  const int g = lane >> 5, r32 = lane & 31;
  float inv[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int hl = 32 * hb + r32;
    const float lt = sh.xch[0][hl] + sh.xch[1][hl];
    inv[hb] = p.splits > 1 ? up : (lt > 0.0f ? up / lt : 0.0f);
  }
  const int tid = 256 + 64 * v + lane;
  if (p.splits > 1 || p.out_fp32) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float* srow = reinterpret_cast<float*>(sh.stage + r32 * kStg32) + 128 * v + 4 * g;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x16& o = O[db][hb];
          *reinterpret_cast<f32x4*>(srow + 32 * db + 8 * qd) =
              f32x4{o[4 * qd], o[4 * qd + 1], o[4 * qd + 2], o[4 * qd + 3]} * inv[hb];
        }
      __syncthreads();  // staged
      store_staged(p, bk, sh, 32 * hb, 32, tid);
      __syncthreads();  // stored
    }
  } else {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      __bf16* srow = reinterpret_cast<__bf16*>(sh.stage + (32 * hb + r32) * kStg16) + 128 * v + 4 * g;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x16& o = O[db][hb];
          *reinterpret_cast<bf16x4*>(srow + 32 * db + 8 * qd) =
              bf16x4{(__bf16)(o[4 * qd] * inv[hb]), (__bf16)(o[4 * qd + 1] * inv[hb]),
                     (__bf16)(o[4 * qd + 2] * inv[hb]), (__bf16)(o[4 * qd + 3] * inv[hb])};
        }
    }
    __syncthreads();
    store_staged(p, bk, sh, 0, kRH, tid);
  }
}

// kFull: the block has 64 heads.  Otherwise q of heads past H is zero (their scores, outputs and
// sums are computed and never stored).
template <bool kFull>
__global__ __launch_bounds__(kRT, 1) void decode_row_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) RowShared sh;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  Block bk;
  if (!block_of<kRH>(p, bk)) return;
  // The row's valid count, its slot entries and (score waves) its q are all requested before any
  // of them is used, so the prologue costs one memory round trip.  A row counted empty reads
  // neither further.
  // (Each role runs its own copy of the compaction, so q is live only in the score waves' code.)
  const int counted = p.valid != nullptr ? p.valid[bk.row] : 1;
  SlotEntries<kRT> se;
  load_slot_entries<kRT>(p, bk, tid, se);
  if (w < 4) {
    QOps q;
    load_q_row<kFull>(p, bk.row, bk.h_lo + 32 * (w >> 1) + (lane & 15), lane >> 4, q);
    if (counted <= 0) {
      write_marked_empty<kRT>(p, bk, tid);
      return;
    }
    bk.total = compact_loaded<RowShared, kRT>(p, bk, sh, w, lane, se);
    bk.ntiles = (bk.total + kTT - 1) / kTT;
    score_role(p, bk, sh, w, lane, q);
  } else {
    if (counted <= 0) {
      write_marked_empty<kRT>(p, bk, tid);
      return;
    }
    bk.total = compact_loaded<RowShared, kRT>(p, bk, sh, w, lane, se);
    bk.ntiles = (bk.total + kTT - 1) / kTT;
    value_role(p, bk, sh, w - 4, lane);
  }
}

}  // namespace

hipError_t launch_decode_row(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream) {
  const unsigned grid = (unsigned)decode_grid(p.T, plan.head_blocks, plan.splits);
  if (p.H % kRH == 0)
    hipLaunchKernelGGL(decode_row_kernel<true>, dim3(grid), dim3(kRT), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_row_kernel<false>, dim3(grid), dim3(kRT), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_split_combine(p, stream);
}

}  // namespace smla
