// Sparse MLA decode over per-row top-k slot lists against a packed fp8_ds_mla cache.
//
// Computes, per query row t and head h, softmax attention over the row's own candidate
// records and returns out[t,h,0:512] and lse[t,h] (page "FlashMLA sparse fp8 path gains
// DCP and MTP", "Key source snippets" and "Implementation breakdown" steps 1-3; page
// "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA", "Why").
//
// gfx950 design
//  * A workgroup owns one row, up to 64 heads and one range of the row's top-k list.  It
//    has one wave per SIMD.  Waves come in pairs; a pair owns 32 heads.  Wave half p of a
//    pair computes the partial scores over latent dims 256p..256p+255 and rope dims
//    32p..32p+31, the two halves swap partial scores through LDS, and wave p then
//    accumulates output dims 256p..256p+255.  Per wave that keeps 72 registers of query
//    and 128 accumulator registers, while every LDS operand byte still feeds 32 heads.
//  * Gather: the row's slot range is compacted in LDS (-1 and out-of-range entries are
//    skipped in place of a front-pack on the host), then tiles of 64 records are copied
//    HBM -> LDS with global_load_lds_dwordx4 (no register staging), double-buffered so the
//    next tile is in flight while the current one is computed.  Lane r of a load carries
//    record r of the tile and load j moves 16-byte chunk j of every record, so the tile
//    sits in LDS chunk-major ([41 chunks][64 records][16 B]): one base address per lane,
//    and every MFMA operand read below is a contiguous LDS access.
//  * QK^T: S^T[token, head] = K[token, :] . Q^T on v_mfma_f32_32x32x16_bf16.  The fp8
//    codes are widened to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1), so the
//    products are exact; each 128-dim fp32 scale multiplies the fp32 partial dot product
//    of its tile, and the bf16 rope dims are added unscaled.
//  * Online softmax in base 2 with a lazy reference max: the accumulators are rescaled
//    only when the running max grows by more than 8 (probabilities stay <= 2^8).  The
//    S^T layout puts one head per lane, so row reductions are in-lane plus one swap.
//  * PV: O^T[dim, head] += V^T[dim, token] . P'^T[token, head] on the same MFMA, with
//    P' = p * scale(token, tile) rounded once to bf16; V^T fragments come straight from
//    the tile with ds_read_b64_tr_b8 and are widened to bf16 exactly.
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
typedef __attribute__((ext_vector_type(2))) int i32x2;
#define SMLA_LDS __attribute__((address_space(3)))

constexpr int TT = 64;       // records per gathered tile
constexpr int CS = 16 * TT;  // bytes per chunk row of a tile
constexpr int kStageBytes = 41 * CS;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLazyRescale = 8.0f;  // log2 units

__device__ __forceinline__ bf16x8 widen_fp8x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-lane state of one wave: 32 heads, its 256 output dims.
struct WaveState {
  f32x16 o[8];  // O^T block mb: dims 256*half + 32*mb + 8*(r/4) + 4*(lane/32) + r%4
  float m_run;  // reference max (log2 units); identical in both waves of a pair
  float l_run;  // this lane's share of the softmax sum (its 16 tokens of each block)
};

// One 32-token block: partial QK^T, score swap with the partner wave, softmax update, PV.
__device__ __forceinline__ void block_compute(const uint8_t* __restrict__ tile, const float* __restrict__ sct,
                                              float* __restrict__ xs_mine, const float* __restrict__ xs_peer,
                                              int blk, int nvalid, const bf16x8 (&qr)[18], WaveState& st,
                                              float scale_log2, int half, int lane) {
  const int h32 = lane & 31;
  const int hh = lane >> 5;

  // ---- partial S^T over latent tiles 2*half, 2*half+1 and rope dims 32*half..+31
  f32x16 s = {};
  const uint8_t* krow = tile + 16 * (32 * blk + h32) + 8 * hh;  // chunk c at + c * CS
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 2 * half + tt;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint2 raw = *reinterpret_cast<const uint2*>(krow + (8 * t + kk) * CS);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen_fp8x8(raw.x, raw.y), qr[8 * tt + kk], acc, 0, 0, 0);
    }
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(sct + t * TT + 32 * blk + 8 * qd + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * qd + i] += sc[i] * acc[4 * qd + i];
    }
  }
  {
    // rope dims 32*half + 16*kk + 8*hh .. +7 are bytes 528 + 64*half + 32*kk + 16*hh
    const uint8_t* rrow = tile + 16 * (32 * blk + h32) + (33 + 4 * half + hh) * CS;
    f32x16 rp = {};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(rrow + 2 * kk * CS);
      rp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[16 + kk], rp, 0, 0, 0);
    }
    s += rp;
  }

  // ---- swap partial scores with the partner wave (same lane layout on both sides)
#pragma unroll
  for (int qd = 0; qd < 4; ++qd)
    *reinterpret_cast<f32x4*>(xs_mine + 16 * lane + 4 * qd) =
        f32x4{s[4 * qd], s[4 * qd + 1], s[4 * qd + 2], s[4 * qd + 3]};
  __syncthreads();
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(xs_peer + 16 * lane + 4 * qd);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * qd + i] += v[i];  // a + b == b + a: both waves agree bit for bit
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tok = 8 * (r >> 2) + 4 * hh + (r & 3);
    s[r] = tok < nvalid ? s[r] * scale_log2 : -INFINITY;
  }

  // ---- online softmax (lane = one head, 16 of the block's tokens)
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m_run, mx);
  const bool need = m_new > st.m_run + kLazyRescale;
  if (__any(need && st.m_run != -INFINITY)) {
    const float alpha = need ? fast_exp2(st.m_run - m_new) : 1.0f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) st.o[mb] *= alpha;
    st.l_run *= alpha;
  }
  if (need) st.m_run = m_new;
  const float mref = st.m_run == -INFINITY ? 0.0f : st.m_run;
  float lsum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = fast_exp2(s[r] - mref);
    lsum += s[r];
  }
  st.l_run += lsum;

  // ---- O^T += V^T P'^T over this wave's latent tiles
  // tr8 row of lane (G = lane/16, rho = lane%16): token tau(ks, G/2, rho/2) and dims
  // 128t + 32mb + 16(G%2) + 8(rho%2) .. +7, i.e. chunk 8t + 2mb + G%2 at byte 8(rho%2).
  const int G = lane >> 4, rho = lane & 15, jj = rho >> 1;
  const int tok0 = 8 * (jj >> 2) + 4 * (G >> 1) + (jj & 3);
  const uint8_t* vbase = tile + 16 * (32 * blk + tok0) + (G & 1) * CS + 8 * (rho & 1);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 2 * half + tt;
    f32x4 sc[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      sc[qd] = *reinterpret_cast<const f32x4*>(sct + t * TT + 32 * blk + 8 * qd + 4 * hh);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 b;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = (__bf16)(s[8 * ks + j] * sc[2 * ks + (j >> 2)][j & 3]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const uint8_t* vp = vbase + 16 * 16 * ks + (8 * t + 2 * mb) * CS;
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SMLA_LDS i32x2*)(vp));
        st.o[4 * tt + mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            widen_fp8x8((uint32_t)raw[0], (uint32_t)raw[1]), b, st.o[4 * tt + mb], 0, 0, 0);
      }
    }
  }
}

// HBM -> LDS copy of one tile: lane r carries record r (records past the end of the list
// repeat the last valid one) and load j moves chunk j of every record.  Wave w issues
// chunks w, w + NW, ...
template <int NW>
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint8_t* rec, int wave) {
#pragma unroll
  for (int k = 0; k < (41 + NW - 1) / NW; ++k) {
    const int j = k * NW + wave;
    if (j < 41) __builtin_amdgcn_global_load_lds(rec + 16 * j, (SMLA_LDS void*)(stage + j * CS), 16, 0, 0);
  }
}

template <int NP>
__global__ __launch_bounds__(NP * 128, 1) void decode_kernel(DecodeParams p) {
  constexpr int NW = 2 * NP;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStageBytes];
  __shared__ __attribute__((aligned(16))) float sct[4 * TT];
  __shared__ __attribute__((aligned(16))) float xs[2][NW][64 * 16];
  __shared__ int32_t clist[kMaxEntriesPerSplit];
  __shared__ int32_t wave_cnt[NW];
  __shared__ int32_t last_flag;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int h32 = lane & 31;
  const int hh = lane >> 5;
  const int pair = wave >> 1;
  const int half = wave & 1;

  // Consecutive blocks are dispatched round-robin over the 8 XCDs; give every XCD a
  // contiguous range of work items so that the head blocks and splits of a row, which
  // gather the same records, run side by side on one XCD and share its L2.
  const int per_xcd = (int)((gridDim.x + 7) / 8);
  const int wg = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (wg >= p.T * p.head_blocks * p.splits) return;
  const int split = wg % p.splits;
  const int rest = wg / p.splits;
  const int hb = rest % p.head_blocks;
  const int row = rest / p.head_blocks;
  const int head = hb * p.heads_per_block + pair * kHeadsPerWave + h32;
  const bool head_ok = head < p.H && (pair * kHeadsPerWave + h32) < p.heads_per_block;

  // ---- query fragments: latent dims 256*half + 16k + 8*hh (k < 16), rope dims 32*half + 16k + 8*hh
  bf16x8 qr[18];
  {
    const int hc = head_ok ? head : 0;
    const uint16_t* qp = p.q + (int64_t)row * p.q_st + (int64_t)hc * p.q_sh + 8 * hh;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 256 * half + 16 * k);
      qr[k] = head_ok ? v : bf16x8{};
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + kLatent + 32 * half + 16 * k);
      qr[16 + k] = head_ok ? v : bf16x8{};
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

  // ---- main loop over gathered tiles
  WaveState st;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) st.o[mb] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.0f;

  const int ntiles = (total + TT - 1) / TT;
  int xbuf = 0;
  if (ntiles > 0) issue_tile<NW>(stage0, p.kv + (int64_t)clist[min(lane, total - 1)] * kRecordBytes, wave);
  for (int it = 0; it < ntiles; ++it) {
    uint8_t* cur = (it & 1) ? stage1 : stage0;
    // the loads of tile `it` are this wave's only ones in flight
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile `it` is in LDS and every wave is done with tile it-1
    if (it + 1 < ntiles) {
      const int idx = min((it + 1) * TT + lane, total - 1);
      issue_tile<NW>((it & 1) ? stage0 : stage1, p.kv + (int64_t)clist[idx] * kRecordBytes, wave);
    }
    // scale chunk (chunk 32) is [record][4 fp32]; transpose it to [tile][record]
    for (int i = tid; i < 4 * TT; i += NT) {
      const int tok = i >> 2, t = i & 3;
      sct[t * TT + tok] = *reinterpret_cast<const float*>(cur + 32 * CS + 16 * tok + 4 * t);
    }
    __syncthreads();
    const int nin = min(TT, total - it * TT);
#pragma unroll
    for (int b = 0; b < TT / 32; ++b) {
      if (32 * b < nin) {
        block_compute(cur, sct, xs[xbuf][wave], xs[xbuf][wave ^ 1], b, nin - 32 * b, qr, st, p.scale_log2, half,
                      lane);
        xbuf ^= 1;
      }
    }
  }

  // ---- epilogue
  const float l_tot = st.l_run + __shfl_xor(st.l_run, 32);
  const int dbase = 256 * half + 4 * hh;  // + 32*mb + 8*qd
  if (p.splits == 1) {
    if (!head_ok) return;
    const bool empty = !(l_tot > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / l_tot;
    if (p.out_fp32) {
      float* orow = reinterpret_cast<float*>(p.out) + (int64_t)row * p.o_st + (int64_t)head * p.o_sh + dbase;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<f32x4*>(orow + 32 * mb + 8 * qd) =
              f32x4{st.o[mb][4 * qd], st.o[mb][4 * qd + 1], st.o[mb][4 * qd + 2], st.o[mb][4 * qd + 3]} * inv;
    } else {
      __bf16* orow = reinterpret_cast<__bf16*>(p.out) + (int64_t)row * p.o_st + (int64_t)head * p.o_sh + dbase;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<bf16x4*>(orow + 32 * mb + 8 * qd) =
              bf16x4{(__bf16)(st.o[mb][4 * qd] * inv), (__bf16)(st.o[mb][4 * qd + 1] * inv),
                     (__bf16)(st.o[mb][4 * qd + 2] * inv), (__bf16)(st.o[mb][4 * qd + 3] * inv)};
    }
    if (half == 0 && hh == 0)
      p.lse[(int64_t)row * p.l_st + (int64_t)head * p.l_sh] = empty ? -INFINITY : (st.m_run + __log2f(l_tot)) * kLn2;
    return;
  }

  // ---- split-K: publish this split's partial, the last arrival combines
  if (head_ok) {
    const int64_t pidx = ((int64_t)row * p.splits + split) * p.H + head;
    float* po = p.ws_o + pidx * kLatent + dbase;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<f32x4*>(po + 32 * mb + 8 * qd) =
            f32x4{st.o[mb][4 * qd], st.o[mb][4 * qd + 1], st.o[mb][4 * qd + 2], st.o[mb][4 * qd + 3]};
    if (half == 0 && hh == 0) {
      p.ws_ml[pidx * 2 + 0] = l_tot > 0.0f ? st.m_run : -INFINITY;
      p.ws_ml[pidx * 2 + 1] = l_tot;
    }
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

  const int h_lo = hb * p.heads_per_block;
  const int nh = min(p.heads_per_block, p.H - h_lo);
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
      *reinterpret_cast<bf16x4*>(orow + 4 * d4) =
          bf16x4{(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
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
    case 2:
      hipLaunchKernelGGL((decode_kernel<1>), dim3(grid), dim3(128), 0, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL((decode_kernel<2>), dim3(grid), dim3(256), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
