// Sparse MLA decode over per-row top-k slot lists against a plain bf16 latent cache: 576
// little-endian bf16 values per token (512 latent, then 64 rope; 1152 bytes), the layout
// page "FlashMLA sparse fp8 path gains DCP and MTP" contrasts with the packed fp8_ds_mla one
// ("Related": 576 against 656; "Risks and impact": the bf16 sparse path).  Same contract as
// the fp8 decode: out[t,h,0:512] and lse[t,h] of softmax attention over the row's own
// candidate records, (0, -inf) for a row without one, split-K merged by split_combine.hip.
//
// gfx950 design (the fp8 kernel's structure, without scales, query split or widening)
//  * A workgroup owns one row, up to 64 heads and one range of the row's top-k list: four
//    score waves (16 heads each) and four value waves (128 output dims each), one of each
//    per SIMD.
//  * Tiles of 16 records, copied HBM -> LDS by the value waves with global_load_lds_dwordx4
//    four tiles ahead (6 tile buffers): one copy moves four 16-byte chunks of the 16 records,
//    so a tile sits chunk-major in LDS ([72 chunks][16 records][16 B]).
//  * QK^T on v_mfma_f32_16x16x32_bf16 over all 576 dims (18 k-steps, two accumulators):
//    the record's bf16 values are the operand as stored, q stays in registers as bf16, and
//    scores come out as heads x tokens (a lane holds one token and four heads), so the max
//    runs per lane with no cross-lane work per tile.  No per-tile scale.
//  * Softmax in base 2 against a per-head reference max fixed at the first tile (a second
//    pass with the exact max if a score ever exceeds it by more than 2^64), so the output
//    accumulators are never rescaled; P = bf16(p) goes to LDS once per tile as swizzled
//    [token][head] rows that the value waves read back transposed (ds_read_b64_tr_b16).
//  * The output leaves through LDS-staged rows, whole rows per store instruction.
//  * PV on v_mfma_f32_32x32x16_bf16: O^T[dim, head] += V^T[dim, token] . P^T[token, head];
//    the V^T operand comes straight from the staged tile through two ds_read_b64_tr_b16 per
//    32-dim block (lane i of a 16-lane group receives dim D0 + i of four consecutive tokens).
//  * One LDS-only barrier per tile; split-K partials merged by the split-merge kernel as in the
//    fp8 kernel.

#include "decode_common.h"

namespace smla {
namespace {

using namespace dec;


constexpr int kRecB = 2 * kHeadDim;          // 1152 bytes per record
constexpr int kTT = 16;                      // records per tile
constexpr int kChunks = kRecB / 16;          // 72 chunks of 16 bytes per record
constexpr int kCS = 16 * kTT;                // 256 bytes per chunk row of a tile
constexpr int kTileBytes = kChunks * kCS;    // 18432
constexpr int kStages = 6;                   // tile buffers: scores on n, values on n-1,
constexpr int kAhead = kStages - 2;          //   loads in flight for n+1 .. n+kAhead
constexpr int kLoads = kChunks / 4;          // 18 global_load_lds per tile, four chunks each
constexpr int kKSteps = kHeadDim / 32;       // 18 QK k-steps of 32 dims
constexpr int kPRow = 2 * kHB;               // bytes per token row of a probability tile
constexpr int kPTile = kTT * kPRow;          // 2 KB
// the probability buffers, sized so that the tile, probability and slot-list buffers together
// hold the output staging rows after the loop
constexpr int kPSpan = 2 * kPTile > kOutStageBytes - kStages * kTileBytes - 4 * kMaxEntriesPerSplit
                           ? 2 * kPTile
                           : kOutStageBytes - kStages * kTileBytes - 4 * kMaxEntriesPerSplit;

static_assert(kRecB % 64 == 0, "a copy moves four whole chunks");
static_assert(kAhead == 4, "load waits below are written for 4 tiles ahead");

struct Shared {
  uint8_t stage[kStages * kTileBytes];  // followed directly by pbuf and clist: the output staging
  uint8_t pbuf[kPSpan];                 // rows span all three once the tile loop is done
  int32_t clist[kMaxEntriesPerSplit];
  float ml[2 * kHB];  // per head of the block: (reference max, sum)
  int32_t wave_cnt[kThreads / 64];
};
static_assert(offsetof(Shared, pbuf) == offsetof(Shared, stage) + sizeof(Shared::stage) &&
                  offsetof(Shared, clist) == offsetof(Shared, pbuf) + sizeof(Shared::pbuf) &&
                  sizeof(Shared::stage) + sizeof(Shared::pbuf) + sizeof(Shared::clist) >= kOutStageBytes,
              "tile, probability and slot-list buffers are contiguous and hold the output staging rows");

__device__ __forceinline__ uint8_t* staging(Shared& sh) { return reinterpret_cast<uint8_t*>(&sh) + offsetof(Shared, stage); }

// Copies value wave b issues per tile: copy j of a tile belongs to wave j % 4.
__device__ __forceinline__ int loads_of_wave(int b) { return b < kLoads % 4 ? kLoads / 4 + 1 : kLoads / 4; }

// Wait until this wave's copies of tile n have landed, given `tiles_newer` later tiles of
// this wave still in flight (wave-uniform).
__device__ __forceinline__ void wait_tile(int tiles_newer, int b) {
  switch (tiles_newer * loads_of_wave(b)) {
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 15: wait_vmcnt<15>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// HBM -> LDS copy of one tile by value wave b (0..3): copy j moves chunks 4j .. 4j+3 of all
// 16 records (lane l: record l % 16, chunk 4j + l / 16) into the contiguous kilobyte j of the
// chunk-major tile.  `rec` is this lane's record plus 16 (l / 16) bytes.
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* rec, int b) {
#pragma unroll
  for (int k = 0; k < (kLoads + 3) / 4; ++k) {
    const int j = b + 4 * k;
    if (j < kLoads) lds_dma16(rec + 64 * j, stage + 1024 * j);
  }
}

// Record of tile entry (lane % 16); entries past the end of the list repeat the last one.
__device__ __forceinline__ const uint8_t* lane_record(const DecodeParams& p, const Shared& sh, int n, int total,
                                                      int lane) {
  const int idx = min(n * kTT + (lane & 15), total - 1);
  return p.kv + (int64_t)sh.clist[idx] * kRecB + 16 * (lane >> 4);
}

// Largest per-lane sum of a pass whose probabilities all stay within the headroom: 2^64 each,
// at most 2^8 tokens per lane (4096 entries over 16 lanes).
constexpr float kMaxLaneSum = 0x1p72f;

template <bool B>
struct PassTag {
  static constexpr bool value = B;
};

// ---------------------------------------------------------------------------------------
// Score wave `sw` (0..3): heads h_lo + 16sw + 0..15.  Query operand: lane holds head
// 16sw + (lane & 15) and dims 32ks + 8g .. +7 of every k-step ks (g = lane >> 4).  Scores
// S = q K^T come out as heads x tokens: lane holds token (lane & 15) and heads 16sw + 4g + r.
__device__ __forceinline__ void score_role(const DecodeParams& p, Shared& sh, const Block& bk, int sw, int lane) {
  const int g = lane >> 4;
  const int hl = 16 * sw + (lane & 15);  // head of this lane's query operand row
  const bool active = 16 * sw < bk.nh;
  bf16x8 qv[kKSteps];
  if (active) {
    const uint16_t* qp = p.q + (int64_t)bk.row * p.q_st + (int64_t)(bk.h_lo + hl) * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qv[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * g);
  } else {
    // an idle score wave (fewer than 64 heads) keeps its heads' probability segments at zero
    for (int i = lane; i < 2 * kTT * 4; i += 64) {
      const int s4 = 4 * sw + (i & 3), j = (i >> 2) % kTT, b = i / (4 * kTT);
      *reinterpret_cast<i32x2*>(sh.pbuf + b * kPTile + j * kPRow + 8 * (s4 ^ pswz(j))) = i32x2{0, 0};
    }
  }
  const float cq = p.scale_log2;
  const int tok = lane & 15;
  const int pseg = (4 * sw + g) ^ pswz(tok);  // P segment of this lane's four heads in token row tok

  float m_ref[4], m_raw[4], l_run[4];  // per output head: reference, running raw max, running sum
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_ref[r] = -INFINITY;
    m_raw[r] = -INFINITY;
    l_run[r] = 0.0f;
  }
  // The tile loop of one pass.  The first pass takes each head's max over the first tile as its
  // reference; a repeated range (kExact) takes the exact max, and rounds each product score * cq
  // before subtracting it, so that no exponent exceeds 0 (a fused product and difference exceeds
  // 0 by up to half an ulp of the reference, which overflows p once references pass 2^31).
  auto tiles = [&](auto exact) {
    constexpr bool kExact = decltype(exact)::value;
    for (int n = 0; n <= bk.ntiles; ++n) {
      lds_barrier();  // tile n staged; P(n-2) consumed by the value waves
      if (!active || n >= bk.ntiles) continue;
      const uint8_t* tile = sh.stage + (n % kStages) * kTileBytes;
      const uint8_t* kr = tile + 16 * tok + g * kCS;
      f32x4 acc0 = {}, acc1 = {};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ks += 2) {
        acc0 = mfma16_bf16(qv[ks], *reinterpret_cast<const bf16x8*>(kr + 4 * ks * kCS), acc0);
        acc1 = mfma16_bf16(qv[ks + 1], *reinterpret_cast<const bf16x8*>(kr + 4 * (ks + 1) * kCS), acc1);
      }
      float pv[4];  // raw scores of heads 4g + r; cq > 0 scales them into log2 units below
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = acc0[r] + acc1[r];
      if (n + 1 == bk.ntiles && tok >= bk.total - n * kTT) {  // tail tile: entries past the list end get p = 0
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) m_raw[r] = __builtin_elementwise_maximum(m_raw[r], pv[r]);
      if (!kExact && n == 0) {
        // the reference of the first pass: each head's max over the first tile (scaling by
        // cq > 0 commutes with the max)
#pragma unroll
        for (int r = 0; r < 4; ++r) m_ref[r] = max16(m_raw[r]) * cq;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = fast_exp2(kExact ? rounded_product_minus(pv[r], cq, m_ref[r]) : fmaf(pv[r], cq, -m_ref[r]));
        l_run[r] += pv[r];
      }
      // P = bf16(p) as [token][head]: this lane's heads 16sw + 4g .. +3 of token tok
      *reinterpret_cast<bf16x4*>(sh.pbuf + (n & 1) * kPTile + tok * kPRow + 8 * pseg) =
          bf16x4{(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
    }
  };
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 0) tiles(PassTag<false>{});
    else tiles(PassTag<true>{});
    // a second pass, with the exact max as reference, only if some score outgrew the headroom or
    // some probability overflowed (a score of the first tile may exceed its own rounded product,
    // the reference, by half an ulp: past 2^31 that alone is more than 2^128)
    bool over = false;
    float m_max[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_max[r] = active ? max16(m_raw[r]) * cq : -INFINITY;
      over |= m_max[r] > m_ref[r] + kRefHeadroom || !(l_run[r] <= kMaxLaneSum);
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
// Value wave `vw` (0..3): output dims 128vw .. +127 of every head of the block; also the
// loader of the tiles.
__device__ __forceinline__ void value_role(const DecodeParams& p, Shared& sh, const Block& bk, int vw, int lane) {
  // O^T blocks o[db][hg]: dims 128vw + 32db + 8(r/4) + 4(lane/32) + r%4, head 32hg + lane%32
  f32x16 o[4][2];
  // P^T operand of head block hg (heads 32hg + lane%32, tokens 8(lane/32) .. +7) as two
  // transposed reads: in its 16-lane group G the lane a addresses token 8(G/2) + a/4 (then
  // + 4) and heads H0 + 4(a%4) .. +3 (H0 = 32hg + 16(G%2)), and receives head H0 + a of the
  // four tokens.  Offsets within a probability tile.
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
      issue_tile(sh.stage + n * kTileBytes, lane_record(p, sh, n, bk.total, lane), vw);
    for (int n = 0; n <= bk.ntiles; ++n) {
      wait_tile(min(kAhead - 1, max(bk.ntiles - 1 - n, 0)), vw);  // tile n is in
      lds_barrier();  // tile n staged; P(n-1) written; tile n-2 and P(n-2) consumed
      if (n + kAhead < bk.ntiles)
        issue_tile(sh.stage + ((n + kAhead) % kStages) * kTileBytes, lane_record(p, sh, n + kAhead, bk.total, lane),
                   vw);
      if (n == 0) continue;
      // ---- O^T += V^T P^T for tile n-1 (tokens past the end carry P = 0 against real records)
      const int m = n - 1;
      const uint8_t* tile = sh.stage + (m % kStages) * kTileBytes;
      const uint8_t* pb = sh.pbuf + (m & 1) * kPTile;
      bf16x8 pf[2];
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) {
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS i16x4*)(pb + poff[hg][0]));
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS i16x4*)(pb + poff[hg][1]));
        pf[hg] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      // tr16 source of this lane a (in its 16-lane group G = lane / 16): token 8(G/2) + a/4 (+4 for
      // the second read), dims D0 + 4(a%4) .. +3 with D0 = 128vw + 32db + 16(G%2)
      const int a = lane & 15, G = lane >> 4;
      const int dl = 16 * (G & 1) + 4 * (a & 3);  // dim within the 32-dim block, a multiple of 4
      const uint8_t* vsrc = tile + 16 * (8 * (G >> 1) + (a >> 2)) + 2 * (dl & 7) + (dl >> 3) * kCS;
      bf16x8 va[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint8_t* base = vsrc + (4 * (4 * vw + db)) * kCS;  // chunk of dim 128vw + 32db
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS i16x4*)(base));
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS i16x4*)(base + 4 * 16));
        va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int hg = 0; hg < 2; ++hg) o[db][hg] = mfma32_bf16(va[db], pf[hg], o[db][hg]);
    }
    if (!__syncthreads_or(false)) break;
  }
  __syncthreads();  // the score waves' (max, sum) are in LDS
  stage_output(p, sh.ml, staging(sh), o, vw, lane);
}

__global__ __launch_bounds__(kThreads, 1) void decode_bf16_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) Shared sh;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  Block bk;
  if (!block_of(p, bk) || skip_marked_empty<kThreads>(p, bk, tid)) return;
  bk.total = compact_slots(p, bk, sh, tid, wave, lane);
  bk.ntiles = (bk.total + kTT - 1) / kTT;

  // The two roles run the same number of workgroup barriers, one per loop step.
  if (wave < 4)
    score_role(p, sh, bk, wave, lane);
  else
    value_role(p, sh, bk, wave - 4, lane);
  __syncthreads();  // output rows staged
  store_rows(p, bk, staging(sh), tid);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream) {
  const unsigned grid = (unsigned)decode_grid(p.T, plan.head_blocks, plan.splits);
  hipLaunchKernelGGL(decode_bf16_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_split_combine(p, stream);
}

}  // namespace smla
