// Sparse MLA decode with every head of a query row in one workgroup, against the packed
// fp8_ds_mla cache.
//
// Computes, per query row t and head h, softmax attention over the row's own candidate
// records and returns out[t,h,0:512] and lse[t,h] (page "FlashMLA sparse fp8 path gains
// DCP and MTP", "Key source snippets" and "Implementation breakdown" steps 1-3; page
// "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA", "Why").
//
// gfx950 design
//  * A workgroup owns one row, all of its heads (up to 128) and one range of its top-k list,
//    so each record is copied HBM -> LDS once and then read by every head.  Four waves, one
//    per SIMD with up to 512 registers each: wave w computes the scores and softmax of heads
//    32w .. 32w + 31 (its q lives in its registers) and the output of every head over the
//    latent dims 128w .. 128w + 127, i.e. over record scale tile w (its accumulators, 128 dims
//    x 128 heads in fp32, fill the accumulation registers).  The probabilities cross from the
//    score side to the value side through LDS, double-buffered; one workgroup barrier per tile
//    orders that hand-over and the tile ring.
//  * Gather: the row's slot range is compacted in LDS (-1 and out-of-range entries dropped),
//    then tiles of 32 records are copied with global_load_lds, two tiles ahead, by all four
//    waves.  A tile sits chunk-major in LDS: [40 chunk rows][32 records][16 B] for the 512
//    codes and 64 rope values, then the record scales as [4 tiles][32 tokens] fp32.  Odd
//    chunk rows hold record r at position r ^ 8 and odd scale rows token r at r ^ 8, so the
//    transposed value reads of two lane groups fall in different banks.
//  * QK^T on v_mfma_f32_32x32x16_bf16 as S^T = K . q^T (tokens x heads): q is the B operand as
//    given (bf16, in registers), the record codes are widened exactly from e4m3 to bf16 for the
//    A operand.  (The scaled fp8 MFMA sums its products with about 12 bits of precision
//    relative to the largest product, so splitting q into fp8 terms is not exact; the bf16 MFMA
//    accumulates in fp32.)  A 128-dim scale tile is eight k-steps; after them the fp32 record
//    scale multiplies the tile's partial scores.  Rope dims take four more bf16 k-steps with
//    q's rope values read from LDS.  The A-operand row m of the MFMA reads record pi(m) (bits
//    2 and 3 of m swapped), so a lane's sixteen scores are tokens 16(i/8) + 8(lane/32) + i%8
//    of its head: exactly the k-order the value MFMA wants for its probability operand.
//  * Softmax in base 2 against a per-head reference max fixed at the first tile: later
//    probabilities are 2^(s - ref) and may exceed 1, which fp32 accumulators hold; should a
//    score exceed the reference by more than 2^64 the workgroup recomputes the range once with
//    the exact max, so the output accumulators are never rescaled inside the loop.
//  * PV as O^T = V^T . P'^T (dims x heads) on v_mfma_f32_32x32x16_bf16: V^T fragments come
//    from the staged tile through ds_read_b64_tr_b8 and are widened exactly to bf16; P' = p *
//    scale(token, w) is rounded once to bf16 from the fp32 probabilities.
//  * Software pipeline: one loop step runs the scores of tile n and the output of tile n-1,
//    two independent MFMA streams the scheduler interleaves with each other's vector work.
//  * Split-K over the top-k list with an in-kernel combine (last split to arrive merges); a
//    row with no valid entry yields out = 0, lse = -inf.

#include "decode_common.h"

namespace smla {
namespace {

using namespace dec;

constexpr int kRT = 256;                              // four waves, one per SIMD
constexpr int kRH = 128;                              // heads one workgroup covers
constexpr int kTT = 32;                               // records per tile
constexpr int kChunkRows = 40;                        // 32 code + 8 rope chunks of 16 bytes per record
constexpr int kCS = 16 * kTT;                         // bytes per chunk row (512)
constexpr int kScaleBase = kChunkRows * kCS;          // record scales [4][32] fp32 after the chunk rows
constexpr int kTileBytes = kScaleBase + 4 * kTT * 4;  // 20992
constexpr int kStages = 4;                            // tile ring: scores on n, values on n-1,
constexpr int kAhead = 2;                             //   copies in flight for n+1, n+2
constexpr int kPRow = 4 * kTT;                        // fp32 probabilities of one head for one tile
constexpr int kPBuf = kRH * kPRow;                    // 16 KB
constexpr int kQRopeRow = 2 * kRope;                  // 128 bytes: one head's rope q

static_assert(kStages == kAhead + 2, "ring: the tile being scored, the one being valued, the copies");
static_assert(kRH * kMaxSplits * 4 <= kStages * kTileBytes, "split weights fit in the tile ring");

struct RowShared {
  uint8_t stage[kStages * kTileBytes];
  uint8_t pbuf[2 * kPBuf];         // [buffer][head][token] fp32, 16-byte chunks swizzled by head
  uint8_t qrope[kRH * kQRopeRow];  // [head][64] bf16, 16-byte chunks swizzled by head
  int32_t clist[kMaxEntriesPerSplit];
  float ml[2 * kRH];  // per head: (reference max, sum)
  int32_t wave_cnt[kRT / 64];
  int32_t last_flag;
};

// Position of record r in chunk row c of a tile, and of token r in scale row t.
__device__ __forceinline__ int rpos(int c, int r) { return r ^ ((c & 1) << 3); }
// Record read by A-operand row m of the score MFMA: bits 2 and 3 of m swapped.
__device__ __forceinline__ int row_token(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Output accumulators live in the accumulation registers (AGPRs) and only the value MFMAs touch
// them, while the score MFMAs accumulate in ordinary VGPRs that the vector unit reads; the
// compiler picks one register form for every MFMA of a function, so the value MFMAs are written
// here.  Wait states follow the compiler's own for these instructions on gfx950: one after a
// vector write of an A/B operand (s_nop 1 gives two), twelve after an MFMA before any other
// read of its result (the fence below gives 32), none between MFMAs chained on one accumulator.
__device__ __forceinline__ void pv_mfma4(f32x16& o0, f32x16& o1, f32x16& o2, f32x16& o3, const bf16x8& v0,
                                         const bf16x8& v1, const bf16x8& v2, const bf16x8& v3, const bf16x8& pp) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %5, %8, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %6, %8, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %7, %8, %3"
      : "+a"(o0), "+a"(o1), "+a"(o2), "+a"(o3)
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "v"(pp));
}
// An accumulator block set to zero by an MFMA of zero operands (no vector write of an AGPR).
__device__ __forceinline__ void zero_acc(f32x16& o, const bf16x8& zero) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(o) : "v"(zero));
}

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

// Copies per tile and wave: five chunk-row pairs, and one scale row pair for waves 0 and 1.
__device__ __forceinline__ void wait_row_tile(bool newer_in_flight, int w) {
  if (!newer_in_flight) wait_vmcnt<0>();
  else if (w < 2) wait_vmcnt<6>();
  else wait_vmcnt<5>();
}

// HBM -> LDS copy of one tile by wave w.  Load j (0..19) fills chunk rows 2j (lanes 0-31) and
// 2j + 1 (lanes 32-63); wave w issues j = w, w + 4, .., w + 16.  Lane i writes position i & 31 of
// its row, i.e. record (i & 31) ^ 8 (i >> 5), whose bytes start at `rec`.  Chunk c of a record
// starts at byte 16c (codes) or 16c + 16 (rope, after the 16 scale bytes).  Waves 0 and 1 also
// copy scale tiles 2w and 2w + 1 of the same records into the scale rows.
__device__ __forceinline__ void issue_row_tile(uint8_t* tile, const uint8_t* rec, int w, int lane) {
  const uint8_t* src = rec + 16 * (lane >> 5) + 32 * w;
  uint8_t* dst = tile + 1024 * w;
  dma16(src, dst);
  dma16(src + 128, dst + 4096);
  dma16(src + 256, dst + 8192);
  dma16(src + 384, dst + 12288);
  dma16(src + 528, dst + 16384);
  if (w < 2) dma4(rec + kScaleOffset + 8 * w + 4 * (lane >> 5), tile + kScaleBase + 256 * w);
}

// Slot of this lane's copy record in tile n; entries past the end repeat the last one.
__device__ __forceinline__ int copy_slot(const RowShared& sh, int n, int total, int lane) {
  return sh.clist[min(n * kTT + ((lane & 31) ^ ((lane >> 5) << 3)), total - 1)];
}

// q of a score lane (head 32w + (lane & 31), lane group g = lane >> 5) as B operands of the
// latent MFMAs: pair u (dims 32u .. 32u + 31) is two k-steps, lo[u] = dims 32u + 16g + 0..7 and
// hi[u] = dims 32u + 16g + 8..15 (the record operand uses the same dims for the same k-slots).
struct QOps {
  bf16x8 lo[16], hi[16];
};

__device__ __forceinline__ void load_q_row(const DecodeParams& p, int row, int hl, int g, QOps& q) {
  if (hl >= p.H) {
#pragma unroll
    for (int u = 0; u < 16; ++u) q.lo[u] = q.hi[u] = bf16x8{};
    return;
  }
  const uint16_t* qp = p.q + (int64_t)row * p.q_st + (int64_t)hl * p.q_sh + 16 * g;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    q.lo[u] = *reinterpret_cast<const bf16x8*>(qp + 32 * u);
    q.hi[u] = *reinterpret_cast<const bf16x8*>(qp + 32 * u + 8);
  }
}

// Rope q of heads 32w .. 32w + 31 -> LDS rows [head][64] (chunk c of head h at c ^ (h & 7)),
// four global_load_lds_dwordx4 per wave: load k covers heads 32w + 8k .. + 7, lane i writes head
// 32w + 8k + i/8, position i % 8.
__device__ __forceinline__ void load_rope_q(const DecodeParams& p, RowShared& sh, int row, int w, int lane) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int hl = 32 * w + 8 * k + (lane >> 3);
    const int c = (lane & 7) ^ (hl & 7);
    const int h = min(hl, p.H - 1);  // heads past H copy a real row; their scores are never stored
    const uint16_t* src = p.q + (int64_t)row * p.q_st + (int64_t)h * p.q_sh + kLatent + 8 * c;
    dma16(reinterpret_cast<const uint8_t*>(src), sh.qrope + 1024 * (4 * w + k));
  }
}

// ---------------------------------------------------------------------------------------
// Scores of tile `tile` for this wave's heads: S^T (tokens x heads), raw (before the softmax
// scale).  Lane (g, r): head 32w + r, element i <-> token 16(i/8) + 8g + i%8.
__device__ __forceinline__ f32x16 score_tile(const uint8_t* tile, const uint8_t* qrope, const QOps& q, int hl, int g,
                                             int tokA) {
  f32x16 S = {};
#pragma unroll
  for (int s = 0; s < 4; ++s) {  // rope: dims 16s + 8g .. + 7 of both operands
    const int c = 32 + 2 * s + g;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(tile + c * kCS + 16 * rpos(c, tokA));
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(qrope + hl * kQRopeRow + 16 * ((2 * s + g) ^ (hl & 7)));
    S = mfma32_bf16(a, b, S);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x16 acc = {};
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {  // pair u = 4t + uu: chunk 2u + g holds dims 32u + 16g + 0..15
      const int u = 4 * t + uu, c = 2 * u + g;
      const i32x4 raw = *reinterpret_cast<const i32x4*>(tile + c * kCS + 16 * rpos(c, tokA));
      acc = mfma32_bf16(widen8((uint32_t)raw[0], (uint32_t)raw[1]), q.lo[u], acc);
      acc = mfma32_bf16(widen8((uint32_t)raw[2], (uint32_t)raw[3]), q.hi[u], acc);
    }
    // record scales of tile t for tokens 8g + 0..7 and 16 + 8g + 0..7
    const float* srow = reinterpret_cast<const float*>(tile + kScaleBase) + kTT * t;
    const int x = 8 * (g ^ (t & 1));
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(srow + x);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(srow + x + 4);
    const f32x4 s2 = *reinterpret_cast<const f32x4*>(srow + 16 + x);
    const f32x4 s3 = *reinterpret_cast<const f32x4*>(srow + 16 + x + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S[i] = fmaf(s0[i], acc[i], S[i]);
      S[4 + i] = fmaf(s1[i], acc[4 + i], S[4 + i]);
      S[8 + i] = fmaf(s2[i], acc[8 + i], S[8 + i]);
      S[12 + i] = fmaf(s3[i], acc[12 + i], S[12 + i]);
    }
  }
  return S;
}

// Output of tile `tile` over dims 128w .. 128w + 127 for every head, with the tile's fp32
// probabilities `pb` ([head][token]).  O[db][hb]: dims 128w + 32db + 8(i/4) + 4(lane/32) + i%4,
// head 32hb + (lane & 31).
template <bool kFull>
__device__ __forceinline__ void value_tile(const uint8_t* tile, const uint8_t* pb, f32x16 (&O)[4][4], int w,
                                           int lane, int nhb) {
  const int g = lane >> 5, G = lane >> 4, a = lane & 15;
  const float* srow = reinterpret_cast<const float*>(tile + kScaleBase) + kTT * w;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    // record scales of tile w for tokens 16ks + 8g + 0..7
    const int x = (16 * ks + 8 * g) ^ (8 * (w & 1));
    const f32x4 sa = *reinterpret_cast<const f32x4*>(srow + x);
    const f32x4 sb = *reinterpret_cast<const f32x4*>(srow + x + 4);
    // V^T operands: lane group G reads records 16ks + 8(G >> 1) + 0..7 of chunk 8w + 2db + (G & 1)
    bf16x8 vt[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int c = 8 * w + 2 * db + (G & 1);
      const int rec = 16 * ks + 8 * (G >> 1) + (a >> 1);
      const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (SMLA_LDS i32x2*)(tile + c * kCS + 16 * rpos(c, rec) + 8 * (a & 1)));
      vt[db] = widen8((uint32_t)raw[0], (uint32_t)raw[1]);
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      if (!kFull && hb >= nhb) break;  // head blocks past H (wave-uniform)
      const int row = 32 * hb + (lane & 31);
      const uint8_t* pr = pb + row * kPRow;
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(pr + 16 * ((4 * ks + 2 * g) ^ (row & 7)));
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(pr + 16 * ((4 * ks + 2 * g + 1) ^ (row & 7)));
      const bf16x8 pp = {(__bf16)(p0[0] * sa[0]), (__bf16)(p0[1] * sa[1]), (__bf16)(p0[2] * sa[2]),
                         (__bf16)(p0[3] * sa[3]), (__bf16)(p1[0] * sb[0]), (__bf16)(p1[1] * sb[1]),
                         (__bf16)(p1[2] * sb[2]), (__bf16)(p1[3] * sb[3])};
      pv_mfma4(O[0][hb], O[1][hb], O[2][hb], O[3][hb], vt[0], vt[1], vt[2], vt[3], pp);
    }
  }
}

// Probabilities of one tile against the reference, into this wave's rows of `pb`; updates the
// running raw max and sum.  Entries at or past `nin` get p = 0.
__device__ __forceinline__ void softmax_tile(f32x16& S, int nin, int g, float cq, float m_ref, float& m_raw,
                                             float& l_run, uint8_t* pb, int hl) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = 16 * (i >> 3) + 8 * g + (i & 7);
    S[i] = tok < nin ? S[i] : -INFINITY;
    m_raw = __builtin_elementwise_maximum(m_raw, S[i]);
  }
  float l = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    S[i] = fast_exp2(fmaf(S[i], cq, -m_ref));
    l += S[i];
  }
  l_run += l;
  uint8_t* pr = pb + hl * kPRow;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 4 * (k >> 1) + 2 * g + (k & 1);
    *reinterpret_cast<f32x4*>(pr + 16 * (c ^ (hl & 7))) = f32x4{S[4 * k], S[4 * k + 1], S[4 * k + 2], S[4 * k + 3]};
  }
}

// kFull: H = 128, every wave has 32 heads to score and every head block has heads; otherwise
// waves and head blocks past H skip their work (wave-uniform branches).
template <bool kFull>
__global__ __launch_bounds__(kRT, 1) void decode_row_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) RowShared sh;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int hl = 32 * w + (lane & 31);  // this lane's head on the score side
  const int tokA = row_token(lane & 31);
  const bool scores = kFull || 32 * w < p.H;  // this wave has heads to score
  const int nhb = kFull ? 4 : (p.H + 31) / 32;

  Block bk;
  if (!block_of<kRH>(p, bk) || skip_marked_empty<kRT>(p, bk, tid)) return;
  QOps q;  // issued before the slot compaction, so both loads share one memory round trip
  load_q_row(p, bk.row, hl, g, q);
  load_rope_q(p, sh, bk.row, w, lane);
  bk.total = compact_slots<RowShared, kRT>(p, bk, sh, tid, w, lane);
  bk.ntiles = (bk.total + kTT - 1) / kTT;

  const float cq = p.scale_log2;
  f32x16 O[4][4];
  float m_ref = -INFINITY, m_raw = -INFINITY, l_run = 0.0f;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) zero_acc(O[db][hb], bf16x8{});
    m_raw = -INFINITY;
    l_run = 0.0f;
    if (bk.ntiles > 0) {
      for (int n = 0; n < kAhead && n < bk.ntiles; ++n)
        issue_row_tile(sh.stage + n * kTileBytes, p.kv + (int64_t)copy_slot(sh, n, bk.total, lane) * kRecordBytes, w,
                       lane);
      int next_slot = kAhead < bk.ntiles ? copy_slot(sh, kAhead, bk.total, lane) : 0;
      // step 0: scores of tile 0 (and, in the first pass, the reference max)
      wait_row_tile(bk.ntiles > 1, w);
      lds_barrier();
      if (kAhead < bk.ntiles) {
        issue_row_tile(sh.stage + kAhead * kTileBytes, p.kv + (int64_t)next_slot * kRecordBytes, w, lane);
        if (kAhead + 1 < bk.ntiles) next_slot = copy_slot(sh, kAhead + 1, bk.total, lane);
      }
      if (scores) {
        f32x16 S = score_tile(sh.stage, sh.qrope, q, hl, g, tokA);
        const int nin = min(kTT, bk.total);
        if (pass == 0) {
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = 16 * (i >> 3) + 8 * g + (i & 7);
            mx = __builtin_elementwise_maximum(mx, tok < nin ? S[i] : -INFINITY);
          }
          mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32));
          m_ref = mx * cq;
        }
        softmax_tile(S, nin, g, cq, m_ref, m_raw, l_run, sh.pbuf, hl);
      }
      // steady steps: scores of tile n, output of tile n - 1
      for (int n = 1; n < bk.ntiles; ++n) {
        wait_row_tile(n + 1 < bk.ntiles, w);
        lds_barrier();  // tile n staged; p(n-1) written; tile n-2 and p(n-2) consumed
        if (n + kAhead < bk.ntiles) {
          issue_row_tile(sh.stage + ((n + kAhead) % kStages) * kTileBytes, p.kv + (int64_t)next_slot * kRecordBytes,
                         w, lane);
          if (n + kAhead + 1 < bk.ntiles) next_slot = copy_slot(sh, n + kAhead + 1, bk.total, lane);
        }
        const uint8_t* tile = sh.stage + (n % kStages) * kTileBytes;
        const uint8_t* prev = sh.stage + ((n - 1) % kStages) * kTileBytes;
        if (kFull) {
          f32x16 S = score_tile(tile, sh.qrope, q, hl, g, tokA);
          value_tile<kFull>(prev, sh.pbuf + ((n - 1) & 1) * kPBuf, O, w, lane, nhb);
          softmax_tile(S, min(kTT, bk.total - n * kTT), g, cq, m_ref, m_raw, l_run, sh.pbuf + (n & 1) * kPBuf, hl);
        } else {
          if (scores) {
            f32x16 S = score_tile(tile, sh.qrope, q, hl, g, tokA);
            softmax_tile(S, min(kTT, bk.total - n * kTT), g, cq, m_ref, m_raw, l_run, sh.pbuf + (n & 1) * kPBuf, hl);
          }
          value_tile<kFull>(prev, sh.pbuf + ((n - 1) & 1) * kPBuf, O, w, lane, nhb);
        }
      }
      // last step: output of the last tile
      lds_barrier();
      {
        const int n = bk.ntiles;
        value_tile<kFull>(sh.stage + ((n - 1) % kStages) * kTileBytes, sh.pbuf + ((n - 1) & 1) * kPBuf, O, w, lane,
                          nhb);
      }
    }
    // a second pass, with the exact max as reference, only if some score outgrew the headroom
    float m_max = m_raw * cq;
    m_max = __builtin_elementwise_maximum(m_max, __shfl_xor(m_max, 32));
    const bool over = m_max > m_ref + kRefHeadroom;
    if (!__syncthreads_or(over)) break;
    m_ref = m_max;
  }

  // the last value MFMAs have written O before anything reads it
  asm volatile("s_nop 15\n\ts_nop 15"
               : "+a"(O[0][0]), "+a"(O[0][1]), "+a"(O[0][2]), "+a"(O[0][3]), "+a"(O[1][0]), "+a"(O[1][1]),
                 "+a"(O[1][2]), "+a"(O[1][3]), "+a"(O[2][0]), "+a"(O[2][1]), "+a"(O[2][2]), "+a"(O[2][3]),
                 "+a"(O[3][0]), "+a"(O[3][1]), "+a"(O[3][2]), "+a"(O[3][3]));

  // ---- per-head (max, sum): LSE or the split's partial, and the normaliser of the output
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (g == 0 && hl < bk.nh) {
    const float mo = l_tot > 0.0f ? m_ref : -INFINITY;
    sh.ml[2 * hl] = mo;
    sh.ml[2 * hl + 1] = l_tot;
    if (p.splits == 1) {
      p.lse[(int64_t)bk.row * p.l_st + (int64_t)hl * p.l_sh] =
          l_tot > 0.0f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const int64_t pidx = ((int64_t)bk.row * p.splits + bk.split) * p.H + hl;
      p.ws_ml[pidx * 2 + 0] = mo;
      p.ws_ml[pidx * 2 + 1] = l_tot;
    }
  }
  __syncthreads();

  // ---- output rows: dims 128w + 32db + 8qd + 4g + 0..3 of head 32hb + (lane & 31)
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = 32 * hb + (lane & 31);
    if (hb >= nhb) break;
    if (h >= bk.nh) continue;
    float inv = 1.0f;
    if (p.splits == 1) {
      const float lt = sh.ml[2 * h + 1];
      inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    }
    if (p.splits > 1 || p.out_fp32) {
      float* base = p.splits > 1
                        ? p.ws_o + (((int64_t)bk.row * p.splits + bk.split) * p.H + h) * kLatent
                        : reinterpret_cast<float*>(p.out) + (int64_t)bk.row * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x16& o = O[db][hb];
          const f32x4 v = {o[4 * qd] * inv, o[4 * qd + 1] * inv, o[4 * qd + 2] * inv, o[4 * qd + 3] * inv};
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(base + 128 * w + 32 * db + 8 * qd + 4 * g));
        }
    } else {
      __bf16* base = reinterpret_cast<__bf16*>(p.out) + (int64_t)bk.row * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x16& o = O[db][hb];
          const bf16x4 v = {(__bf16)(o[4 * qd] * inv), (__bf16)(o[4 * qd + 1] * inv), (__bf16)(o[4 * qd + 2] * inv),
                            (__bf16)(o[4 * qd + 3] * inv)};
          __builtin_nontemporal_store(__builtin_bit_cast(i32x2, v),
                                      reinterpret_cast<i32x2*>(base + 128 * w + 32 * db + 8 * qd + 4 * g));
        }
    }
  }
  if (p.splits == 1) return;
  if (arrive_last(p, bk, sh, tid))
    combine_splits<RowShared, kRT, kRH>(p, bk, sh, reinterpret_cast<float*>(sh.stage), tid);
}

__global__ void zero_row_counters(int32_t* cnt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) cnt[i] = 0;
}

}  // namespace

hipError_t launch_decode_row(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream) {
  const int64_t items = (int64_t)p.T * plan.head_blocks * plan.splits;
  const unsigned grid = (unsigned)((items + 7) / 8 * 8);
  if (plan.splits > 1) {
    const int64_t n = (int64_t)p.T * plan.head_blocks;
    hipLaunchKernelGGL(zero_row_counters, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p.ws_cnt, n);
  }
  if (p.H == kRH)
    hipLaunchKernelGGL(decode_row_kernel<true>, dim3(grid), dim3(kRT), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_row_kernel<false>, dim3(grid), dim3(kRT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
