// Achievable-peak microbenchmarks for the units the sparse MLA decode relies on, on gfx950:
// streaming HBM copy and read, dense bf16 and fp8 MFMA chains (and the latency of dependent
// ones), the e4m3 -> bf16 widening
// conversion, and an MFMA stream with independent vector work beside it in the same wave.
// Built into a library of its own (libsmla_peak.so): measurement, not part of the decode path.
//
// Every kernel is a plain loop of a fixed instruction pattern; the caller times a launch with
// events on `stream` and converts with the work figures each entry point documents.  Results
// that would otherwise be dead are written to `sink` (one value per thread), so the compiler
// keeps the loops.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

// ---- HBM streams -------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_copy(const i32x4* __restrict__ src, i32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void k_read(const i32x4* __restrict__ src, int64_t n, int* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const i32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x7fffffff) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// ---- MFMA chains ----------------------------------------------------------------------------
// Eight independent accumulators per wave, each advanced once per iteration.  The MFMAs are
// written out so the pattern is exactly as stated.  Wait states: the operands pass through an
// empty asm statement with five wait states after their last vector write, consecutive MFMAs on
// one accumulator need none, and a 48-state fence holding the accumulators follows the loop.
#define SMLA_SETTLE(a, b) asm volatile("s_nop 4" : "+v"(a), "+v"(b))

template <int KIND>  // 0: 32x32x16 bf16, 1: 16x16x32 bf16
__global__ __launch_bounds__(512) void k_mfma_bf16(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  i32x4 a = {lane, lane + 1, lane + 2, lane + 3};
  i32x4 b = {lane * 3, lane ^ 5, 7, lane + 9};
  a &= 0x3f803f80;  // small normal bf16 values
  b &= 0x3f803f80;
  SMLA_SETTLE(a, b);
  float r = 0.0f;
  if (KIND == 0) {
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
    for (int it = 0; it < iters; ++it) {
      asm volatile(
          "v_mfma_f32_32x32x16_bf16 %0, %8, %9, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %8, %9, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %8, %9, %2\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %8, %9, %3\n\t"
          "v_mfma_f32_32x32x16_bf16 %4, %8, %9, %4\n\t"
          "v_mfma_f32_32x32x16_bf16 %5, %8, %9, %5\n\t"
          "v_mfma_f32_32x32x16_bf16 %6, %8, %9, %6\n\t"
          "v_mfma_f32_32x32x16_bf16 %7, %8, %9, %7"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
          : "v"(a), "v"(b));
    }
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15"
                 : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7));
    r = c0[0] + c1[1] + c2[2] + c3[3] + c4[4] + c5[5] + c6[6] + c7[7];
  } else {
    f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
    for (int it = 0; it < iters; ++it) {
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
          "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
          "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
          "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
          "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
          : "v"(a), "v"(b));
    }
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15"
                 : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7));
    r = c0[0] + c1[1] + c2[2] + c3[3] + c4[0] + c5[1] + c6[2] + c7[3];
  }
  if (r == 1234.5f) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// C dependent chains of 16x16x32 bf16 MFMAs per wave (C = 1, 2, 4 or 8), each advanced once per
// iteration: with few chains every MFMA waits for the result of the one before it on its
// accumulator, so the time per MFMA against C gives the dependent-issue latency.
template <int C>
__global__ __launch_bounds__(512) void k_mfma_chain(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  i32x4 ai = {lane, lane + 1, lane + 2, lane + 3};
  i32x4 bi = {lane * 3, lane ^ 5, 7, lane + 9};
  ai &= 0x3f803f80;  // small normal bf16 values
  bi &= 0x3f803f80;
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  const bf16x8 a = __builtin_bit_cast(bf16x8, ai), b = __builtin_bit_cast(bf16x8, bi);
  f32x4 c[C];
#pragma unroll
  for (int k = 0; k < C; ++k) c[k] = f32x4{0.0f, 0.0f, 0.0f, (float)k};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < C; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float r = 0.0f;
#pragma unroll
  for (int k = 0; k < C; ++k) r += c[k][0] + c[k][3];
  if (r == 1234.5f) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// fp8 (e4m3 x e4m3) 32x32x64 MFMA chains, eight accumulators.
__global__ __launch_bounds__(512) void k_mfma_fp8(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (lane * 7 + i) & 0x38383838;  // small normal e4m3 codes
    b[i] = (lane * 5 + 3 * i) & 0x38383838;
  }
  SMLA_SETTLE(a, b);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_32x32x64_f8f6f4 %0, %8, %9, %0\n\t"
        "v_mfma_f32_32x32x64_f8f6f4 %1, %8, %9, %1\n\t"
        "v_mfma_f32_32x32x64_f8f6f4 %2, %8, %9, %2\n\t"
        "v_mfma_f32_32x32x64_f8f6f4 %3, %8, %9, %3\n\t"
        "v_mfma_f32_32x32x64_f8f6f4 %4, %8, %9, %4\n\t"
        "v_mfma_f32_32x32x64_f8f6f4 %5, %8, %9, %5\n\t"
        "v_mfma_f32_32x32x64_f8f6f4 %6, %8, %9, %6\n\t"
        "v_mfma_f32_32x32x64_f8f6f4 %7, %8, %9, %7"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b));
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15"
               : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7));
  const float r = c0[0] + c1[1] + c2[2] + c3[3] + c4[4] + c5[5] + c6[6] + c7[7];
  if (r == 1234.5f) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// ---- MFMA with vector work beside it -------------------------------------------------------
// Per iteration: four 32x32x16 bf16 MFMAs on independent accumulators (128 MFMA cycles at the
// published rate) and NV independent fp32 FMAs on registers no MFMA touches, in one wave.  The
// time per iteration against NV shows how much vector work a wave hides under its own MFMAs.
template <int NV>
__global__ __launch_bounds__(512) void k_mix(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  i32x4 a = {lane, lane + 1, lane + 2, lane + 3};
  i32x4 b = {lane * 3, lane ^ 5, 7, lane + 9};
  a &= 0x3f803f80;
  b &= 0x3f803f80;
  SMLA_SETTLE(a, b);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[NV > 0 ? NV : 1];
#pragma unroll
  for (int i = 0; i < (NV > 0 ? NV : 1); ++i) x[i] = (float)(lane + i) * 1e-3f;
  const float y = 0.999f, z = 1e-4f;
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
        "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
        "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
        : "v"(a), "v"(b));
#pragma unroll
    for (int i = 0; i < NV; ++i) x[i] = fmaf(x[i], y, z);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
  float r = c0[0] + c1[1] + c2[2] + c3[3];
#pragma unroll
  for (int i = 0; i < NV; ++i) r += x[i];
  if (r == 1234.5f) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// The same work with the vector instructions spread between the MFMAs: four blocks of one MFMA
// and NV / 4 FMAs, so the wave issues vector work while each MFMA runs.
template <int NV>
__global__ __launch_bounds__(512) void k_mixi(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  i32x4 a = {lane, lane + 1, lane + 2, lane + 3};
  i32x4 b = {lane * 3, lane ^ 5, 7, lane + 9};
  a &= 0x3f803f80;
  b &= 0x3f803f80;
  SMLA_SETTLE(a, b);
  f32x16 c[4] = {};
  float x[NV > 0 ? NV : 1];
#pragma unroll
  for (int i = 0; i < (NV > 0 ? NV : 1); ++i) x[i] = (float)(lane + i) * 1e-3f;
  const float y = 0.999f, z = 1e-4f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c[m]) : "v"(a), "v"(b));
#pragma unroll
      for (int i = m * NV / 4; i < (m + 1) * NV / 4; ++i) x[i] = fmaf(x[i], y, z);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]));
  float r = c[0][0] + c[1][1] + c[2][2] + c[3][3];
#pragma unroll
  for (int i = 0; i < NV; ++i) r += x[i];
  if (r == 1234.5f) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// ---- one MFMA wave and one vector wave per SIMD ------------------------------------------------
// Waves 0-3 run `iters` iterations of four independent 32x32x16 bf16 MFMAs (when mfma != 0); waves
// 4-7 run `iters` iterations of 16 e4m3 -> bf16 conversions (when valu != 0).  With both, the
// time against either alone shows how far a SIMD overlaps one wave's MFMAs with another's vector
// work.
__global__ __launch_bounds__(512) void k_dual(int iters, int mfma, int valu, float* sink) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float r = 0.0f;
  if (w < 4) {
    if (!mfma) return;
    i32x4 a = {lane, lane + 1, lane + 2, lane + 3};
    i32x4 b = {lane * 3, lane ^ 5, 7, lane + 9};
    a &= 0x3f803f80;
    b &= 0x3f803f80;
    SMLA_SETTLE(a, b);
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      asm volatile(
          "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
          : "v"(a), "v"(b));
    }
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
    r = c0[0] + c1[1] + c2[2] + c3[3];
  } else {
    if (!valu) return;
    uint32_t s0 = 0x3a3b3c3du ^ (uint32_t)lane, s2 = 0x3f800000u;
    asm volatile("" : "+v"(s0), "+v"(s2));
    uint32_t d[8];
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int rep = 0; rep < 2; ++rep) {
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2" : "=v"(d[i]) : "v"(s0), "v"(s2));
        asm volatile("" ::"v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5]), "v"(d[6]), "v"(d[7]));
      }
    }
    r = (float)(d[0] ^ d[7]);
  }
  if (r == 1234.5f) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// ---- vector instruction issue rates ------------------------------------------------------------
// Per iteration 32 independent instances of one vector instruction (sources fixed, results kept
// live through an empty asm statement every eight): 0 v_fma_f32, 1 v_cvt_scalef32_pk_bf16_fp8,
// 2 v_cvt_pk_f32_fp8, 3 v_perm_b32, 4 v_exp_f32, 5 v_cvt_pk_bf16_f32, 6 v_and_or_b32.
template <int OP>
__global__ __launch_bounds__(512) void k_valu(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  uint32_t s0 = 0x3a3b3c3du ^ (uint32_t)lane, s1 = 0x01234567u + (uint32_t)lane, s2 = 0x3f800000u;
  asm volatile("" : "+v"(s0), "+v"(s1), "+v"(s2));
  uint32_t d[8];
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (OP == 0) asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(d[i]) : "v"(s0), "v"(s1), "v"(s2));
        if (OP == 1) asm volatile("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2" : "=v"(d[i]) : "v"(s0), "v"(s2));
        if (OP == 2) asm volatile("v_cvt_pk_f32_fp8 %0, %1" : "=v"(*reinterpret_cast<uint64_t*>(&d[i & 6])) : "v"(s0));
        if (OP == 3) asm volatile("v_perm_b32 %0, %1, %2, %3" : "=v"(d[i]) : "v"(s0), "v"(s1), "v"(s2));
        if (OP == 4) asm volatile("v_exp_f32 %0, %1" : "=v"(d[i]) : "v"(s1));
        if (OP == 5) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(d[i]) : "v"(s1), "v"(s2));
        if (OP == 6) asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(d[i]) : "v"(s0), "v"(s1), "v"(s2));
      }
      asm volatile("" ::"v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5]), "v"(d[6]), "v"(d[7]));
    }
  }
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) r ^= d[i];
  if (r == 0x12345u) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)r;
}

// ---- LDS throughput -----------------------------------------------------------------------------
// Per iteration 16 LDS instructions per wave on conflict-free addresses in the first 64 KB of a
// 96 KB buffer (so one workgroup holds a CU):
// 0 ds_read_b128 (lane i: 16 bytes at 16 i), 1 ds_read_b64 (8 bytes at 8 i), 2 ds_read_b64_tr_b8
// (8 bytes at 8 i), 3 ds_write_b128 (16 bytes at 16 i).  Waves w and w + 4 share a window; no
// access leaves the buffer.
template <int OP>
__global__ __launch_bounds__(512) void k_lds(int iters, float* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[98304];  // over half the CU's LDS: one workgroup per CU
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 65536 / 16; i += blockDim.x) reinterpret_cast<i32x4*>(buf)[i] = i32x4{i, i, i, i};
  __syncthreads();
  const int step = OP == 0 || OP == 3 ? 16 : 8;
  // byte address in LDS: window of wave w & 3 (1 KB apart) + lane offset; the largest access ends
  // at 3072 + 1008 + 16 + 28672 + 32768 = 65536
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)buf + 1024 * (w & 3) + step * lane;
  i32x4 acc = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t a = base + 4096 * (k & 7) + 32768 * (k >> 3);
      if (OP == 0) {
        i32x4 v;
        asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
        acc ^= v;
      } else if (OP == 1 || OP == 2) {
        typedef __attribute__((ext_vector_type(2))) int i32x2;
        i32x2 v;
        if (OP == 1) asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(a));
        else asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(v) : "v"(a));
        acc[0] ^= v[0];
        acc[1] ^= v[1];
      } else {
        asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(acc) : "memory");
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if (acc[0] == 0x12345 && acc[1] == 7) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)acc[2];
}

// ---- e4m3 -> bf16 widening ---------------------------------------------------------------------
// Per iteration 16 v_cvt_scalef32_pk_bf16_fp8 (two codes each) and 16 bit operations, on 8
// independent source words.
__global__ __launch_bounds__(512) void k_cvt(int iters, const uint32_t seed, float* sink) {
  const int lane = threadIdx.x & 63;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = (seed * (lane + 1) + 0x9e3779b9u * i) & 0x3f3f3f3fu;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = bf16x2{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x2 p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
      const bf16x2 q = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
      // fold into the source word so each conversion depends on the previous iteration
      w[i] ^= __builtin_bit_cast(uint32_t, p) ^ __builtin_bit_cast(uint32_t, q);
      w[i] &= 0x3f3f3f3fu;
      acc[i] = p;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r += (float)acc[i][0] + (float)w[i];
  if (r == 1234.5f) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// Shader clock under MFMA load: one wave per workgroup runs 32x32x16 bf16 MFMAs and records the
// shader cycle counter and the constant 100 MHz real-time counter at both ends of its loop.
__global__ __launch_bounds__(64) void k_clock(int iters, unsigned long long* out) {
  const int lane = threadIdx.x & 63;
  i32x4 a = {lane, lane + 1, lane + 2, lane + 3};
  a &= 0x3f803f80;
  i32x4 b = a;
  SMLA_SETTLE(a, b);
  f32x16 c0 = {}, c1 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %2, %3, %1"
        : "+v"(c0), "+v"(c1)
        : "v"(a), "v"(b));
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(c0), "+v"(c1));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[4 * blockIdx.x + 0] = t0;
    out[4 * blockIdx.x + 1] = t1;
    out[4 * blockIdx.x + 2] = r0;
    out[4 * blockIdx.x + 3] = r1;
  }
  if (c0[0] + c1[1] == 1234.5f) out[4 * blockIdx.x] = 0;
}

}  // namespace

extern "C" {

// Streaming copy of n16 16-byte words from src to dst (device pointers, 16-byte aligned):
// 32 n16 bytes of HBM traffic.  grid: workgroups of 256 threads.
int smla_peak_copy(const void* src, void* dst, int64_t n16, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, stream, static_cast<const i32x4*>(src), static_cast<i32x4*>(dst),
                     n16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Streaming read of n16 16-byte words: 16 n16 bytes.  sink: grid * 256 ints (never written in
// practice).
int smla_peak_read(const void* src, int64_t n16, int grid, int* sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, stream, static_cast<const i32x4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// MFMA chains: kind 0 = 32x32x16 bf16 (32768 flops each), 1 = 16x16x32 bf16 (16384), 2 = 32x32x64
// fp8 (131072).  Each wave issues 8 * iters MFMAs.  Workgroups of 64 * waves_per_wg threads;
// sink: grid * 64 * waves_per_wg floats.
int smla_peak_mfma(int kind, int iters, int grid, int waves_per_wg, float* sink, hipStream_t stream) {
  if (waves_per_wg < 1 || waves_per_wg > 8) return 1;
  const dim3 blk(64 * waves_per_wg);
  if (kind == 0) hipLaunchKernelGGL(k_mfma_bf16<0>, dim3(grid), blk, 0, stream, iters, sink);
  else if (kind == 1) hipLaunchKernelGGL(k_mfma_bf16<1>, dim3(grid), blk, 0, stream, iters, sink);
  else if (kind == 2) hipLaunchKernelGGL(k_mfma_fp8, dim3(grid), blk, 0, stream, iters, sink);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// `chains` (1, 2, 4 or 8) dependent 16x16x32 bf16 MFMA chains per wave, `iters` MFMAs each.
int smla_peak_chain(int chains, int iters, int grid, int waves_per_wg, float* sink, hipStream_t stream) {
  if (waves_per_wg < 1 || waves_per_wg > 8) return 1;
  const dim3 blk(64 * waves_per_wg);
  switch (chains) {
    case 1: hipLaunchKernelGGL(k_mfma_chain<1>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 2: hipLaunchKernelGGL(k_mfma_chain<2>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 4: hipLaunchKernelGGL(k_mfma_chain<4>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 8: hipLaunchKernelGGL(k_mfma_chain<8>, dim3(grid), blk, 0, stream, iters, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Four 32x32x16 bf16 MFMAs and nv (0, 16, 32, 64 or 128) fp32 FMAs per iteration and wave.
int smla_peak_mix(int nv, int iters, int grid, int waves_per_wg, float* sink, hipStream_t stream) {
  if (waves_per_wg < 1 || waves_per_wg > 8) return 1;
  const dim3 blk(64 * waves_per_wg);
  switch (nv) {
    case 0: hipLaunchKernelGGL(k_mix<0>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 16: hipLaunchKernelGGL(k_mix<16>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 32: hipLaunchKernelGGL(k_mix<32>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 64: hipLaunchKernelGGL(k_mix<64>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 128: hipLaunchKernelGGL(k_mix<128>, dim3(grid), blk, 0, stream, iters, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// MFMA with interleaved vector work (nv = 0, 16, 32, 64 or 128), as smla_peak_mix.
int smla_peak_mixi(int nv, int iters, int grid, int waves_per_wg, float* sink, hipStream_t stream) {
  if (waves_per_wg < 1 || waves_per_wg > 8) return 1;
  const dim3 blk(64 * waves_per_wg);
  switch (nv) {
    case 0: hipLaunchKernelGGL(k_mixi<0>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 16: hipLaunchKernelGGL(k_mixi<16>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 32: hipLaunchKernelGGL(k_mixi<32>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 64: hipLaunchKernelGGL(k_mixi<64>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 128: hipLaunchKernelGGL(k_mixi<128>, dim3(grid), blk, 0, stream, iters, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// 32 independent instances of vector instruction `op` (0..6, see k_valu) per iteration and wave.
int smla_peak_valu(int op, int iters, int grid, int waves_per_wg, float* sink, hipStream_t stream) {
  if (waves_per_wg < 1 || waves_per_wg > 8) return 1;
  const dim3 blk(64 * waves_per_wg);
  switch (op) {
    case 0: hipLaunchKernelGGL(k_valu<0>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 1: hipLaunchKernelGGL(k_valu<1>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 2: hipLaunchKernelGGL(k_valu<2>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 3: hipLaunchKernelGGL(k_valu<3>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 4: hipLaunchKernelGGL(k_valu<4>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 5: hipLaunchKernelGGL(k_valu<5>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 6: hipLaunchKernelGGL(k_valu<6>, dim3(grid), blk, 0, stream, iters, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// One MFMA wave (four 32x32x16 bf16 per iteration) and one conversion wave (16 per iteration) per
// SIMD; mfma / valu switch each side on.  One workgroup of 8 waves per CU.
int smla_peak_dual(int iters, int mfma, int valu, int grid, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_dual, dim3(grid), dim3(512), 0, stream, iters, mfma, valu, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// 16 LDS instructions (op 0..3, see k_lds) per iteration and wave; one workgroup per CU.
int smla_peak_lds(int op, int iters, int grid, int waves_per_wg, float* sink, hipStream_t stream) {
  if (waves_per_wg < 1 || waves_per_wg > 8) return 1;
  const dim3 blk(64 * waves_per_wg);
  switch (op) {
    case 0: hipLaunchKernelGGL(k_lds<0>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 1: hipLaunchKernelGGL(k_lds<1>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 2: hipLaunchKernelGGL(k_lds<2>, dim3(grid), blk, 0, stream, iters, sink); break;
    case 3: hipLaunchKernelGGL(k_lds<3>, dim3(grid), blk, 0, stream, iters, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// 16 widening conversions (32 codes) plus 16 bit operations per iteration and wave.
int smla_peak_cvt(int iters, int grid, int waves_per_wg, float* sink, hipStream_t stream) {
  if (waves_per_wg < 1 || waves_per_wg > 8) return 1;
  hipLaunchKernelGGL(k_cvt, dim3(grid), dim3(64 * waves_per_wg), 0, stream, iters, 12345u, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Shader-cycle and 100 MHz real-time stamps around 2 * iters dependent-free MFMAs in each of grid
// single-wave workgroups: out[4 i + 0..3] = cycles at start, at end, real time at start, at end.
int smla_peak_clock(int iters, int grid, unsigned long long* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_clock, dim3(grid), dim3(64), 0, stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
