// Sparse MLA decode over per-row top-k slot lists against a packed fp8_ds_mla cache.
//
// Computes, per query row t and head h, softmax attention over the row's own candidate
// records and returns out[t,h,0:512] and lse[t,h] (page "FlashMLA sparse fp8 path gains
// DCP and MTP", "Key source snippets" and "Implementation breakdown" steps 1-3; page
// "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA", "Why").
//
// gfx950 design
//  * A workgroup owns one row, up to 128 heads (NW waves x 32) and one range of the row's
//    top-k list, with one wave per SIMD.  Every gathered record feeds all heads of the row.
//  * Work split inside the workgroup: wave w computes scores, softmax and probabilities for
//    its 32 heads over all 576 dims; the probabilities go to LDS; wave w then accumulates
//    output dims [w*512/NW, (w+1)*512/NW) for ALL heads of the workgroup.  No softmax is
//    duplicated and every value operand is widened by exactly one wave.
//  * Gather: the row's slot range is compacted in LDS (-1 and out-of-range entries are
//    skipped; no front-pack on the host), then tiles of TT records are copied HBM -> LDS
//    with global_load_lds_dwordx4 (no register staging), double-buffered.  Lane r of a load
//    carries record r of the tile and load j moves 16-byte chunk j of every record, so the
//    tile sits in LDS chunk-major ([41 chunks][TT records][16 B]): one base address per
//    lane, and every MFMA operand read below is a contiguous LDS access.
//  * QK^T latent part on fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales): the raw
//    e4m3 codes are the A operand as stored, and q is split exactly into two e4m3 terms,
//    q * 2^e_h = hi + lo (hi = rne(q * 2^e_h), lo = rne(q * 2^e_h - hi), e_h a per-head power
//    of two putting max|q| just under 448), so two fp8 MFMAs give the bf16-exact product at
//    the cost of one bf16 MFMA and no operand widening.  Each 128-dim fp32 record scale
//    multiplies the fp32 partial dot product of its tile.  Rope dims (bf16) run on
//    v_mfma_f32_32x32x16_bf16.  S^T (tokens x heads) puts one head per lane, so softmax row
//    reductions are in-lane plus one cross-half swap.
//  * Softmax in base 2 against a per-head reference max fixed at the first tile: later
//    probabilities are 2^(s - ref) and may exceed 1, which fp32 accumulators and bf16
//    probabilities hold without loss.  Should a score ever exceed the reference by more
//    than 2^64 the workgroup recomputes the row once with the exact max as reference, so
//    the accumulators are never rescaled inside the loop.
//  * PV: O^T[dim, head] += V^T[dim, token] . P'^T[token, head] on bf16 MFMA with
//    P' = p * scale(token, tile) rounded once to bf16 (written to LDS per scale tile); V^T
//    fragments come from the tile through ds_read_b64_tr_b8 and are widened exactly.
//  * Split-K over the top-k list with an in-kernel combine: every split writes its
//    unnormalised partial (O, max, sum) to the workspace; the last split to arrive (device
//    scope counter, zeroed by a small kernel before the decode kernel) merges them.
//  * A row with no valid entry yields out = 0, lse = -inf.

#include "smla_internal.h"

#include <math.h>

namespace smla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
#define SMLA_LDS __attribute__((address_space(3)))

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRefHeadroom = 64.0f;  // log2 units a score may exceed the reference by
constexpr int kUnitScale = 127;       // E8M0 encoding of 2^0 for the scaled fp8 MFMA

__device__ __forceinline__ bf16x8 widen_fp8x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kUnitScale, 0, kUnitScale);
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// HBM -> LDS copy of one tile: lane r < TT carries record r (records past the end of the
// list repeat the last valid one) and load j moves chunk j of every record.  Wave w issues
// chunks w, w + NW, ...
template <int NW, int TT>
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* rec, int wave, int lane) {
  if (lane < TT) {
#pragma unroll
    for (int k = 0; k < (41 + NW - 1) / NW; ++k) {
      const int j = k * NW + wave;
      if (j < 41) __builtin_amdgcn_global_load_lds(rec + 16 * j, (SMLA_LDS void*)(stage + j * 16 * TT), 16, 0, 0);
    }
  }
}

template <int NW, int TT>
__global__ __launch_bounds__(NW * 64, 1) void decode_kernel(DecodeParams p) {
  constexpr int NT = NW * 64;
  constexpr int NB = TT / 32;        // 32-token blocks per tile
  constexpr int CS = 16 * TT;        // bytes per chunk row of a tile
  constexpr int DPW = kLatent / NW;  // output dims per wave
  constexpr int NDB = DPW / 32;      // 32-dim output blocks per wave
  constexpr int TPW = 4 / NW;        // scale tiles per wave
  constexpr int HPB = 32 * NW;       // heads per workgroup
  constexpr int PS = 2 * TT;         // bytes per head row of a probability tile
  constexpr int GM = TT / 8 - 1;     // 16-byte granules of a row are XOR-swizzled by head & GM
  constexpr int PT = HPB * PS;       // bytes per scale tile of probabilities
  __shared__ __attribute__((aligned(16))) uint8_t stage0[41 * CS];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[41 * CS];
  __shared__ __attribute__((aligned(16))) float sct[4 * TT];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[4 * PT];
  __shared__ float linv_s[HPB];
  __shared__ int32_t clist[kMaxEntriesPerSplit];
  __shared__ int32_t wave_cnt[NW];
  __shared__ int32_t last_flag;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int h32 = lane & 31;
  const int hh = lane >> 5;

  // Consecutive blocks are dispatched round-robin over the 8 XCDs; give every XCD a
  // contiguous range of work items so the splits of a row run side by side on one XCD.
  const int per_xcd = (int)((gridDim.x + 7) / 8);
  const int wg = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (wg >= p.T * p.head_blocks * p.splits) return;
  const int split = wg % p.splits;
  const int rest = wg / p.splits;
  const int hb = rest % p.head_blocks;
  const int row = rest / p.head_blocks;
  const int h_lo = hb * HPB;
  const int qhead = h_lo + wave * 32 + h32;  // head whose scores this lane computes
  const bool q_ok = qhead < p.H;

  // ---- query: latent as exact e4m3 pairs (dims 128t + 64kk + 32hh + i <-> byte i), rope bf16
  i32x8 qh[4][2], ql[4][2];
  bf16x8 qr[4];
  float qexp_inv;  // 2^-e_h (the rope fragments carry the same 2^e_h)
  {
    const uint16_t* qp = p.q + (int64_t)row * p.q_st + (int64_t)(q_ok ? qhead : 0) * p.q_sh + 32 * hh;
    // pass 1: per-head max |q| over the latent dims (lanes h32 and h32 + 32 hold one head)
    float amax = 0.0f;
    if (q_ok) {
#pragma unroll 4
      for (int c = 0; c < 32; ++c) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 64 * (c >> 2) + 8 * (c & 3));
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)v[i]));
      }
    }
    if (q_ok) {
      const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(qp - 32 * hh + kLatent + 32 * hh);
      const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(qp - 32 * hh + kLatent + 32 * hh + 8);
      const bf16x8 v2 = *reinterpret_cast<const bf16x8*>(qp - 32 * hh + kLatent + 32 * hh + 16);
      const bf16x8 v3 = *reinterpret_cast<const bf16x8*>(qp - 32 * hh + kLatent + 32 * hh + 24);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf((float)v0[i]), fabsf((float)v1[i])),
                                 fmaxf(fabsf((float)v2[i]), fabsf((float)v3[i]))));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int e = 0;
    if (amax > 0.0f) {
      e = (int)floorf(__log2f(448.0f / amax));
      if (ldexpf(amax, e) > 448.0f) --e;
      e = max(-100, min(100, e));
    }
    qexp_inv = ldexpf(1.0f, -e);
    // pass 2: q * 2^e = hi + lo, both e4m3 (exact for |q * 2^e| >= 2^-2, see the design notes)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 v = q_ok ? *reinterpret_cast<const bf16x8*>(qp + 128 * t + 64 * kk + 8 * c) : bf16x8{};
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            int hi, lo;
            split_e4m3(ldexpf((float)v[4 * g], e), ldexpf((float)v[4 * g + 1], e), ldexpf((float)v[4 * g + 2], e),
                       ldexpf((float)v[4 * g + 3], e), hi, lo);
            qh[t][kk][2 * c + g] = hi;
            ql[t][kk][2 * c + g] = lo;
          }
        }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 v = q_ok ? *reinterpret_cast<const bf16x8*>(qp - 32 * hh + kLatent + 16 * kk + 8 * hh) : bf16x8{};
      bf16x8 w;
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = (__bf16)ldexpf((float)v[i], e);  // exact: |q * 2^e| <= 448
      qr[kk] = w;
    }
  }

  // ---- compact this split's slot entries (valid = within [0, num_slots))
  const int e0 = split * p.entries_per_split;
  const int e1 = min(p.K, e0 + p.entries_per_split);
  const int32_t* srow = p.slots + (int64_t)row * p.slots_ld;
  int total = 0;
  for (int base = e0; base < e1; base += NT * 8) {
    int vals[8];
    int wcount = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = base + i * NT + tid;
      const int v = e < e1 ? srow[e] : -1;
      const bool ok = v >= 0 && (int64_t)v < p.num_slots;
      vals[i] = ok ? v : -1;
      wcount += __popcll(__ballot(ok));
    }
    if (lane == 0) wave_cnt[wave] = wcount;
    __syncthreads();
    int off = total, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = wave_cnt[w];
      off += w < wave ? c : 0;
      all += c;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = vals[i] >= 0;
      const unsigned long long b = __ballot(ok);
      if (ok) clist[off + __popcll(b & below)] = vals[i];
      off += __popcll(b);
    }
    total += all;
    __syncthreads();
  }

  // ---- state: O^T accumulators o[db][hg] = dims wave*DPW + 32db + 8(r/4) + 4hh + r%4, head h_lo + 32hg + h32
  f32x16 o[NDB][NW];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int hg = 0; hg < NW; ++hg) o[db][hg] = f32x16{};
  float m_ref = -INFINITY;  // reference max of head qhead (log2 units), same in lanes h32 and h32+32
  float m_max = -INFINITY;  // exact running max of head qhead
  float l_run = 0.0f;       // this lane's share of the softmax sum of head qhead

  const float sl_lat = p.scale_log2 * qexp_inv;

  const int ntiles = (total + TT - 1) / TT;
  for (int pass = 0; pass < 2; ++pass) {
  bool over = false;  // a score exceeded the reference by more than the headroom
  if (ntiles > 0) issue_tile<NW, TT>(stage0, p.kv + (int64_t)clist[min(lane, total - 1)] * kRecordBytes, wave, lane);
  for (int it = 0; it < ntiles; ++it) {
    uint8_t* tile = (it & 1) ? stage1 : stage0;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of tile `it`
    __syncthreads();  // tile `it` in LDS; every wave is done with tile it-1 (its probabilities included)
    if (it + 1 < ntiles) {
      const int idx = min((it + 1) * TT + lane, total - 1);
      issue_tile<NW, TT>((it & 1) ? stage0 : stage1, p.kv + (int64_t)clist[idx] * kRecordBytes, wave, lane);
    }
    // scale chunk (chunk 32) is [record][4 fp32]; transpose it to [tile][record]
    for (int i = tid; i < 4 * TT; i += NT) {
      const int tok = i >> 2, t = i & 3;
      sct[t * TT + tok] = *reinterpret_cast<const float*>(tile + 32 * CS + 16 * tok + 4 * t);
    }
    __syncthreads();
    const int nin = min(TT, total - it * TT);

    // ---- per 32-token block: scores of this wave's 32 heads, softmax numerators, P'
    // s[r] <-> token 32b + 8(r/4) + 4hh + r%4 of the tile; lane = head qhead
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));  // recompute lane-derived addresses here instead of hoisting them
    const int l32 = lane_o & 31, lhh = lane_o >> 5;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (32 * b >= nin) break;
      const uint8_t* krow = tile + 16 * (32 * b + l32);
      // rope dims 16kk + 8hh .. +7 (bf16, both operands scaled by 2^e_h): chunk 33 + 2kk + hh
      f32x16 s = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s = mfma_bf16(*reinterpret_cast<const bf16x8*>(krow + (33 + 2 * kk + lhh) * CS), qr[kk], s);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int c0 = 8 * t + 4 * kk + 2 * lhh;  // dims 128t + 64kk + 32hh .. +31
          const i32x4 a0 = *reinterpret_cast<const i32x4*>(krow + c0 * CS);
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(krow + (c0 + 1) * CS);
          const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          acc = mfma_fp8(a, qh[t][kk], acc);
          acc = mfma_fp8(a, ql[t][kk], acc);
        }
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 sc = *reinterpret_cast<const f32x4*>(sct + t * TT + 32 * b + 8 * qd + 4 * lhh);
#pragma unroll
          for (int i = 0; i < 4; ++i) s[4 * qd + i] += sc[i] * acc[4 * qd + i];
        }
      }
      s *= sl_lat;
      if (nin - 32 * b < 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * lhh + (r & 3) >= nin - 32 * b) s[r] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_max = fmaxf(m_max, mx);
      if (m_ref == -INFINITY) m_ref = mx;
      over |= mx > m_ref + kRefHeadroom;
      const float mref = m_ref == -INFINITY ? 0.0f : m_ref;
      float lsum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(s[r] - mref);
        lsum += s[r];
      }
      l_run += lsum;
      // P'_t = bf16(p * scale(token, t)) as [t][head][token]; granule tok/8 = 4b + qd, byte 8hh inside it
      const int ph = wave * 32 + l32;
      uint8_t* prow = pbuf + ph * PS + 8 * lhh;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 sc = *reinterpret_cast<const f32x4*>(sct + t * TT + 32 * b + 8 * qd + 4 * lhh);
          const bf16x4 v = {(__bf16)(s[4 * qd] * sc[0]), (__bf16)(s[4 * qd + 1] * sc[1]),
                            (__bf16)(s[4 * qd + 2] * sc[2]), (__bf16)(s[4 * qd + 3] * sc[3])};
          *reinterpret_cast<bf16x4*>(prow + t * PT + 16 * ((4 * b + qd) ^ (ph & GM))) = v;
        }
    }
    __syncthreads();

    // ---- O^T += V^T P'^T for this wave's dims and every head of the workgroup
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
      if (16 * ks < nin) {
        bf16x8 bq[TPW][NW];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
          for (int hg = 0; hg < NW; ++hg)
            bq[tt][hg] = *reinterpret_cast<const bf16x8*>(pbuf + (wave * TPW + tt) * PT + (32 * hg + l32) * PS +
                                                          16 * ((2 * ks + lhh) ^ ((32 * hg + l32) & GM)));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int mbg = wave * NDB + db;  // global 32-dim block: chunks 2mbg, 2mbg+1
          const int vrow = 16 * (8 * ((lane_o >> 4) >> 1) + ((lane_o & 15) >> 1)) + 8 * (lane_o & 1) +
                           ((lane_o >> 4) & 1) * CS;  // tr8 row of this lane
          const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (SMLA_LDS i32x2*)(tile + 2 * mbg * CS + 16 * 16 * ks + vrow));
          const bf16x8 va = widen_fp8x8((uint32_t)raw[0], (uint32_t)raw[1]);
          const int tt = db / 4;  // 4 dim blocks per scale tile
#pragma unroll
          for (int hg = 0; hg < NW; ++hg) o[db][hg] = mfma_bf16(va, bq[tt][hg], o[db][hg]);
        }
      }
    }
  }

  // a second pass, with the exact max as reference, only if some score outgrew the headroom
  if (!__syncthreads_or(over)) break;
  m_ref = m_max;
  l_run = 0.0f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int hg = 0; hg < NW; ++hg) o[db][hg] = f32x16{};
  }  // pass

  // ---- epilogue: per-head sums from the score waves, normalisation by the value waves
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  __syncthreads();  // every wave is done reading pbuf
  if (hh == 0) linv_s[wave * 32 + h32] = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (p.splits == 1 && q_ok && hh == 0)
    p.lse[(int64_t)row * p.l_st + (int64_t)qhead * p.l_sh] =
        l_tot > 0.0f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (p.splits > 1 && q_ok && hh == 0) {
    const int64_t pidx = ((int64_t)row * p.splits + split) * p.H + qhead;
    p.ws_ml[pidx * 2 + 0] = l_tot > 0.0f ? m_ref : -INFINITY;
    p.ws_ml[pidx * 2 + 1] = l_tot;
  }
  __syncthreads();
  const int dbase = wave * DPW + 4 * hh;  // + 32db + 8qd
  if (p.splits == 1) {
#pragma unroll
    for (int hg = 0; hg < NW; ++hg) {
      const int head = h_lo + 32 * hg + h32;
      if (head >= p.H) continue;
      const float inv = linv_s[32 * hg + h32];
      if (p.out_fp32) {
        float* orow = reinterpret_cast<float*>(p.out) + (int64_t)row * p.o_st + (int64_t)head * p.o_sh + dbase;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * qd) =
                f32x4{o[db][hg][4 * qd], o[db][hg][4 * qd + 1], o[db][hg][4 * qd + 2], o[db][hg][4 * qd + 3]} * inv;
      } else {
        __bf16* orow = reinterpret_cast<__bf16*>(p.out) + (int64_t)row * p.o_st + (int64_t)head * p.o_sh + dbase;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * qd) =
                bf16x4{(__bf16)(o[db][hg][4 * qd] * inv), (__bf16)(o[db][hg][4 * qd + 1] * inv),
                       (__bf16)(o[db][hg][4 * qd + 2] * inv), (__bf16)(o[db][hg][4 * qd + 3] * inv)};
      }
    }
    return;
  }

  // ---- split-K: publish this split's unnormalised partial, the last arrival combines
#pragma unroll
  for (int hg = 0; hg < NW; ++hg) {
    const int head = h_lo + 32 * hg + h32;
    if (head >= p.H) continue;
    float* po = p.ws_o + (((int64_t)row * p.splits + split) * p.H + head) * kLatent + dbase;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * qd) =
            f32x4{o[db][hg][4 * qd], o[db][hg][4 * qd + 1], o[db][hg][4 * qd + 2], o[db][hg][4 * qd + 3]};
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(p.ws_cnt + (int64_t)row * p.head_blocks + hb, 1, __ATOMIC_ACQ_REL,
                                           __HIP_MEMORY_SCOPE_AGENT);
    last_flag = old == p.splits - 1;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();

  const int nh = min(HPB, p.H - h_lo);
  for (int item = tid; item < nh * (kLatent / 4); item += NT) {
    const int hrel = item / (kLatent / 4);
    const int d4 = item - hrel * (kLatent / 4);
    const int h = h_lo + hrel;
    const float* ml = p.ws_ml + ((int64_t)row * p.splits * p.H + h) * 2;  // split sp at + sp * H * 2
    float M = -INFINITY;
    for (int sp = 0; sp < p.splits; ++sp) M = fmaxf(M, __builtin_nontemporal_load(ml + (int64_t)sp * p.H * 2));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.0f;
    if (M != -INFINITY) {
      for (int sp = 0; sp < p.splits; ++sp) {
        const float ms = __builtin_nontemporal_load(ml + (int64_t)sp * p.H * 2);
        if (ms == -INFINITY) continue;
        const float w = fast_exp2(ms - M);
        L += w * __builtin_nontemporal_load(ml + (int64_t)sp * p.H * 2 + 1);
        const int64_t pidx = ((int64_t)row * p.splits + sp) * p.H + h;
        acc += w * __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.ws_o + pidx * kLatent) + d4);
      }
    }
    const bool empty = !(L > 0.0f);
    acc *= empty ? 0.0f : 1.0f / L;
    if (p.out_fp32) {
      float* orow = reinterpret_cast<float*>(p.out) + (int64_t)row * p.o_st + (int64_t)h * p.o_sh;
      *reinterpret_cast<f32x4*>(orow + 4 * d4) = acc;
    } else {
      __bf16* orow = reinterpret_cast<__bf16*>(p.out) + (int64_t)row * p.o_st + (int64_t)h * p.o_sh;
      *reinterpret_cast<bf16x4*>(orow + 4 * d4) = bf16x4{(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
    }
    if (d4 == 0) p.lse[(int64_t)row * p.l_st + (int64_t)h * p.l_sh] = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
  }
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
  switch (plan.waves) {
    case 1:
      hipLaunchKernelGGL((decode_kernel<1, 32>), dim3(grid), dim3(64), 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((decode_kernel<2, 32>), dim3(grid), dim3(128), 0, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL((decode_kernel<4, 64>), dim3(grid), dim3(256), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
