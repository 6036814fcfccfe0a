// Split-K merge of one decode call: the second kernel of a decode whose top-k lists were split
// over several workgroups per row.
//
// Each split s of row t left, per head h, its unnormalised output O_s (sum over its entries of
// 2^(score - m_s) v) and (m_s, l_s): its reference maximum in log2 units and its sum of
// 2^(score - m_s).  Over the whole list the softmax output is
//     out = sum_s 2^(m_s - M) O_s / L,   L = sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// and lse = (M + log2 L) ln 2: the rescaling the online softmax applies tile by tile, and the
// same merge of (out, lse) pairs over disjoint key sets that combines DCP shards (page
// "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown" step 3); the
// partials live in an fp32 slab per (row, head) like the softmax-stats slab of page
// "[Bugfix][Attention] Stabilize sparse-MLA DCP for GLM PCP evals", "FlashInfer sparse-MLA DCP
// workspace".  A row with no valid entry (every m_s = -inf, or a row its valid count marks
// empty) yields out = 0 and lse = -inf.
//
// One wave per (row, head): lane s < splits reads split s's (m, l), the wave reduces them to
// M and L and keeps split s's weight 2^(m_s - M) / L in lane s; then every lane owns 8 of the
// 512 dims and adds the splits' partial rows, eight splits' loads in flight at a time (the first
// eight issued beside the (max, sum) loads).  A
// separate kernel rather than an in-kernel "last split to arrive" merge: the kernel boundary
// publishes the partials to every XCD without a device-scope release and acquire in each
// workgroup (each of which writes back and invalidates the L2 of its XCD), and the merge
// spreads over T * H waves instead of one workgroup per row.

#include "smla_internal.h"

namespace smla {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kWaves = 4;  // heads per workgroup, one wave each
constexpr float kLn2f = 0.69314718055994530942f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__global__ __launch_bounds__(64 * kWaves) void split_combine_kernel(DecodeParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int per_row = (p.H + kWaves - 1) / kWaves;
  const int row = blockIdx.x / per_row;
  const int h = (blockIdx.x % per_row) * kWaves + wave;
  if (row >= p.T || h >= p.H) return;  // wave-uniform
  const bool marked_empty = p.valid != nullptr && p.valid[row] <= 0;

  // The first eight splits' partial rows are requested together with the (max, sum) pairs (one
  // memory round trip for both); a split whose weight turns out zero is skipped when adding, so
  // rows never written by this call (a row marked empty) are read but never used.
  const f32x4* base = reinterpret_cast<const f32x4*>(p.ws_o + ((int64_t)row * p.splits * p.H + h) * kLatent) + 2 * lane;
  const int64_t sstride = (int64_t)p.H * kLatent / 4;  // one split further, in 16-byte units
  f32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < p.splits) {
      a[i] = __builtin_nontemporal_load(base + i * sstride);
      b[i] = __builtin_nontemporal_load(base + i * sstride + 1);
    }
  }
  float m = -INFINITY, l = 0.0f;
  if (!marked_empty && lane < p.splits) {
    const float* ml = p.ws_ml + (((int64_t)row * p.splits + lane) * p.H + h) * 2;
    m = __builtin_nontemporal_load(ml);
    l = __builtin_nontemporal_load(ml + 1);
  }
  const float M = wave_max(m);
  float w = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
  const float L = wave_sum(w * l);
  const bool empty = !(L > 0.0f);  // wave-uniform
  w = empty ? 0.0f : w / L;
  if (lane == 0) p.lse[(int64_t)row * p.l_st + (int64_t)h * p.l_sh] = empty ? -INFINITY : (M + __log2f(L)) * kLn2f;

  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll 1
  for (int s0 = 0; s0 < p.splits; s0 += 8) {
    if (s0 > 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (s0 + i < p.splits) {
          a[i] = __builtin_nontemporal_load(base + (s0 + i) * sstride);
          b[i] = __builtin_nontemporal_load(base + (s0 + i) * sstride + 1);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s0 + i < p.splits) {
        const float ws = lane_value(w, s0 + i);
        if (ws != 0.0f) {  // a zero-weight split adds nothing (and its row may hold no finite values)
          acc0 += ws * a[i];
          acc1 += ws * b[i];
        }
      }
    }
  }
  if (p.out_fp32) {
    f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + (int64_t)row * p.o_st + (int64_t)h * p.o_sh) +
               2 * lane;
    o[0] = acc0;
    o[1] = acc1;
  } else {
    bf16x8* o = reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(p.out) + (int64_t)row * p.o_st +
                                          (int64_t)h * p.o_sh) + lane;
    *o = bf16x8{(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
                (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
  }
}

}  // namespace

hipError_t launch_split_combine(const DecodeParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.T * ((p.H + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(split_combine_kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
