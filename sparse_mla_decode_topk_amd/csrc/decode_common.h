// Device helpers shared by the decode kernels of both record layouts (fp8_ds_mla and plain
// bf16): workgroup-to-work mapping, slot-list compaction, LDS-only barriers, HBM -> LDS
// copies, MFMA wrappers and output staging.  Each kernel keeps its own tile
// layout, roles and main loop.

#pragma once

#include "smla_internal.h"

#include <math.h>
#include <stddef.h>

namespace smla {
namespace dec {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
#define SMLA_LDS __attribute__((address_space(3)))

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRefHeadroom = 64.0f;  // log2 units a score may exceed the reference by
constexpr int kThreads = 512;          // 4 score waves + 4 value waves
constexpr int kHB = kHeadsPerBlock;    // 64 heads per workgroup

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x * c rounded to fp32, then minus m (two roundings: never fused into one fma).  A repeated
// range's exponents take this form against the largest rounded product, so none exceeds 0; a
// fused x * c - m exceeds 0 by up to half an ulp of m.
__device__ __forceinline__ float rounded_product_minus(float x, float c, float m) {
#pragma clang fp contract(off)
  return x * c - m;
}

__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Range exponent of a block of q values with largest magnitude amax: the largest e with
// amax * 2^e <= 448 (the e4m3 maximum), clamped to [-100, 100]; 0 for an all-zero block.
__device__ __forceinline__ int range_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = (int)floorf(__log2f(448.0f / amax));
  if (ldexpf(amax, e) > 448.0f) --e;
  return max(-100, min(100, e));
}

// 2^e as a float for |e| <= 126 (exact).
__device__ __forceinline__ float exp2_int(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global memory, which
// makes every wave drain its in-flight HBM -> LDS copies at each barrier; the copies are
// instead waited for explicitly by the waves that issued them.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// max of a value over lanes l, l^16, l^32, l^48 (every lane gets it), on the VALU
__device__ __forceinline__ float max4x16(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane i's 16 bytes land at
// LDS address lds + 16 i.  Issued as inline assembly so the compiler does not treat every
// later LDS read as a possible alias of the copy and drain all copies in flight before it;
// the waves wait for their own copies explicitly before the barrier that publishes a tile.
// M0 (the LDS base of the copy) is written right before each copy; the kernels have no
// other M0 user.
__device__ __forceinline__ void lds_dma16(const uint8_t* src, const uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(SMLA_LDS void*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
}

struct Block {
  int row, hb, split, h_lo, nh, total, ntiles;
};

// Work item of this workgroup: (row, head block of HB heads, split), or false when the grid slot
// holds none.  Rows go to the 8 XCDs in groups of kRowGroup consecutive rows, group g to XCD
// g % 8 (workgroup b runs on XCD b % 8), so the items of a group (every head block and split of
// its rows: the MTP rows of a request share records) run side by side on one XCD and share its
// L2, while rows whose work grows or shrinks along the batch (prefill rows at increasing
// positions) spread evenly over the XCDs.  The grid is decode_grid() slots.
template <int HB = kHB>
__device__ __forceinline__ bool block_of(const DecodeParams& p, Block& bk) {
  const int per_group = kRowGroup * p.head_blocks * p.splits;
  const int k = (int)(blockIdx.x / 8);
  const int group = (int)(blockIdx.x % 8) + 8 * (k / per_group);
  const int64_t wg = (int64_t)group * per_group + k % per_group;
  if (wg >= (int64_t)p.T * p.head_blocks * p.splits) return false;
  bk.split = (int)(wg % p.splits);
  const int rest = (int)(wg / p.splits);
  bk.hb = rest % p.head_blocks;
  bk.row = rest / p.head_blocks;
  bk.h_lo = bk.hb * HB;
  bk.nh = min(HB, p.H - bk.h_lo);  // a multiple of 16
  return true;
}

// A row the caller marks empty through its valid count (<= 0): neither q nor the slot list is
// read.  Unsplit, the workgroup writes out = 0 and lse = -inf for the block's heads; split, it
// does nothing (the split merge writes the row).  Returns true when the workgroup is done.
template <int NT>
__device__ __forceinline__ void write_marked_empty(const DecodeParams& p, const Block& bk, int tid);

template <int NT>
__device__ __forceinline__ bool skip_marked_empty(const DecodeParams& p, const Block& bk, int tid) {
  if (p.valid == nullptr || p.valid[bk.row] > 0) return false;
  write_marked_empty<NT>(p, bk, tid);
  return true;
}

// The output of a row marked empty: out = 0 and lse = -inf for the block's heads when the call
// has one split (with several, the split merge writes the row).
template <int NT>
__device__ __forceinline__ void write_marked_empty(const DecodeParams& p, const Block& bk, int tid) {
  if (p.splits > 1) return;
  const int per_row = p.out_fp32 ? 4 * kLatent / 16 : 2 * kLatent / 16;  // 16-byte pieces of one head
  for (int c = tid; c < bk.nh * per_row; c += NT) {
    const int h = bk.h_lo + c / per_row, col = c % per_row;
    uint8_t* row = reinterpret_cast<uint8_t*>(p.out) +
                   ((int64_t)bk.row * p.o_st + (int64_t)h * p.o_sh) * (p.out_fp32 ? 4 : 2);
    *reinterpret_cast<i32x4*>(row + 16 * col) = i32x4{0, 0, 0, 0};
  }
  if (tid < bk.nh) p.lse[(int64_t)bk.row * p.l_st + (int64_t)(bk.h_lo + tid) * p.l_sh] = -INFINITY;
}

// Probability tiles are [token][head] rows of 64 bf16 values (128 bytes) in 8-byte segments of
// four heads; segment s of token j sits at segment s ^ pswz(j).  pswz swaps the two 2-bit
// fields of j's low four bits, so both the score waves' stores (sixteen tokens, one segment
// each) and the value waves' transposed reads (four tokens x four segments per 16-lane
// group) touch sixteen distinct segments: no bank conflicts either way.
__device__ __forceinline__ int pswz(int j) { return ((j & 3) << 2) | ((j >> 2) & 3); }

// Max and sum over the 16 lanes of a lane group (lanes 16g .. 16g + 15); every lane of the
// group gets the same result.
__device__ __forceinline__ float max16(float x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Output staging rows after a decode kernel's tile loop: 16 bytes of padding put consecutive
// rows four banks apart, so the value waves' row-strided writes do not conflict.
constexpr int kOutPitch32 = 4 * kLatent + 16;  // fp32 rows
constexpr int kOutPitch16 = 2 * kLatent + 16;  // bf16 rows
constexpr int kOutStageBytes = kHB * kOutPitch32;  // LDS span a kernel provides after its loop

// Value wave vw's O^T blocks (o[db][hg]: dims 128vw + 32db + 8(r/4) + 4(lane/32) + r%4, head
// 32hg + lane%32), normalised by the head's sum when the call has one split, into the staging
// rows [head][dim] at stg: fp32 for split partials and fp32 outputs, bf16 otherwise.
__device__ __forceinline__ void stage_output(const DecodeParams& p, const float* ml, uint8_t* stg,
                                             const f32x16 (&o)[4][2], int vw, int lane) {
  const bool f32out = p.splits > 1 || p.out_fp32;
  const int h32 = lane & 31;
  const int dbase = 128 * vw + 4 * (lane >> 5);  // + 32db + 8qd
#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    const int hl = 32 * hg + h32;
    float inv = 1.0f;
    if (p.splits == 1) {
      const float lt = ml[2 * hl + 1];
      inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    }
    if (f32out) {
      float* r = reinterpret_cast<float*>(stg + hl * kOutPitch32) + dbase;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<f32x4*>(r + 32 * db + 8 * qd) =
              f32x4{o[db][hg][4 * qd], o[db][hg][4 * qd + 1], o[db][hg][4 * qd + 2], o[db][hg][4 * qd + 3]} * inv;
    } else {
      __bf16* r = reinterpret_cast<__bf16*>(stg + hl * kOutPitch16) + dbase;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<bf16x4*>(r + 32 * db + 8 * qd) =
              bf16x4{(__bf16)(o[db][hg][4 * qd] * inv), (__bf16)(o[db][hg][4 * qd + 1] * inv),
                     (__bf16)(o[db][hg][4 * qd + 2] * inv), (__bf16)(o[db][hg][4 * qd + 3] * inv)};
    }
  }
}

// Staged output rows -> global memory, 16 bytes per thread and 1 KB of one row per wave and
// instruction (a direct store from the MFMA layout would touch 32 rows per instruction).
// Rows of heads past the block's last head are not written.  The stores are non-temporal:
// nothing in the kernel reads the output again, and streaming it past L2 leaves the L2
// lines of the records to the other head block of the row.
__device__ __forceinline__ void store_rows(const DecodeParams& p, const Block& bk, const uint8_t* stg, int tid) {
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
    constexpr int kChunksPerRow = 4 * kLatent / 16;  // 128
#pragma unroll
    for (int k = 0; k < kHB * kChunksPerRow / kThreads; ++k) {
      const int c = tid + kThreads * k;
      const int hl = c / kChunksPerRow, col = c % kChunksPerRow;
      if (hl < bk.nh) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + hl * kOutPitch32 + 16 * col);
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(base + (int64_t)(bk.h_lo + hl) * hstride + 4 * col));
      }
    }
  } else {
    __bf16* base = reinterpret_cast<__bf16*>(p.out) + (int64_t)bk.row * p.o_st;
    constexpr int kChunksPerRow = 2 * kLatent / 16;  // 64
#pragma unroll
    for (int k = 0; k < kHB * kChunksPerRow / kThreads; ++k) {
      const int c = tid + kThreads * k;
      const int hl = c / kChunksPerRow, col = c % kChunksPerRow;
      if (hl < bk.nh) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(stg + hl * kOutPitch16 + 16 * col);
        __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(base + (int64_t)(bk.h_lo + hl) * p.o_sh + 8 * col));
      }
    }
  }
}

// This split's slot entries, as loaded by one thread before compaction: at most
// kMaxEntriesPerSplit / NT of them, in groups of four; -1 past the split's end.
template <int NT>
struct SlotEntries {
  static constexpr int kPer = ((kMaxEntriesPerSplit + NT - 1) / NT + 3) / 4 * 4;
  int v[kPer];
};

// Issues every load of this thread's slot entries (the whole list costs one memory round trip).
template <int NT>
__device__ __forceinline__ void load_slot_entries(const DecodeParams& p, const Block& bk, int tid,
                                                  SlotEntries<NT>& se) {
  const int e0 = bk.split * p.entries_per_split;
  const int e1 = min(p.K, e0 + p.entries_per_split);
  const int32_t* srow = p.slots + (int64_t)bk.row * p.slots_ld;
#pragma unroll
  for (int i = 0; i < SlotEntries<NT>::kPer; ++i) {
    const int e = e0 + i * NT + tid;
    se.v[i] = e < e1 ? srow[e] : -1;
  }
}

// Compacts the loaded entries that lie in [0, num_slots) into sh.clist, in a fixed order
// (attention sums over the set); returns their number.  No front-pack is needed upstream.
// Groups of 4 * NT entries are placed in order, two barriers per group.
template <class SH, int NT>
__device__ __forceinline__ int compact_loaded(const DecodeParams& p, const Block& bk, SH& sh, int wave, int lane,
                                              SlotEntries<NT>& se) {
  constexpr int kPer = SlotEntries<NT>::kPer;
  const int e0 = bk.split * p.entries_per_split;
  const int e1 = min(p.K, e0 + p.entries_per_split);
  int total = 0;
#pragma unroll
  for (int grp = 0; grp < kPer / 4; ++grp) {
    if (e0 + grp * 4 * NT >= e1) break;  // uniform across the workgroup
    int wcount = 0;
#pragma unroll
    for (int i = 4 * grp; i < 4 * grp + 4; ++i) {
      const bool ok = se.v[i] >= 0 && (int64_t)se.v[i] < p.num_slots;
      se.v[i] = ok ? se.v[i] : -1;
      wcount += __popcll(__ballot(ok));
    }
    if (lane == 0) sh.wave_cnt[wave] = wcount;
    __syncthreads();
    int off = total, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      const int c = sh.wave_cnt[w];
      off += w < wave ? c : 0;
      all += c;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 4 * grp; i < 4 * grp + 4; ++i) {
      const bool ok = se.v[i] >= 0;
      const unsigned long long bm = __ballot(ok);
      if (ok) sh.clist[off + __popcll(bm & below)] = se.v[i];
      off += __popcll(bm);
    }
    total += all;
    __syncthreads();
  }
  return total;
}

// Loads and compacts this split's slot entries (see load_slot_entries and compact_loaded).
template <class SH, int NT = kThreads>
__device__ __forceinline__ int compact_slots(const DecodeParams& p, const Block& bk, SH& sh, int tid, int wave,
                                             int lane) {
  SlotEntries<NT> se;
  load_slot_entries<NT>(p, bk, tid, se);
  return compact_loaded<SH, NT>(p, bk, sh, wave, lane, se);
}

}  // namespace dec
}  // namespace smla
