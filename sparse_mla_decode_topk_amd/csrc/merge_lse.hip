// LSE merge of S partial attention results over disjoint KV shards.
//
// lse = ln sum_s exp(lse_s), out = sum_s exp(lse_s - lse) * out_s; an entry whose partials
// are all -inf is (0, -inf), the merge identity (page "FlashMLA sparse fp8 path gains DCP
// and MTP", "Implementation breakdown" steps 1 and 3; page "[eldritch] attention: support
// DCP in SM120 FlashInfer sparse MLA", "Why").
//
// HBM-bound: each (row, head) pair reads S partial rows of 512 values and writes one.  A
// wave handles one (row, head) pair: the S weights are computed once per pair, every lane
// moves 8 consecutive dims with 16- or 32-byte accesses.  Up to 8 shards the partial rows of
// a pair are all in flight together.

#include "smla_internal.h"

#include <math.h>

namespace smla {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kMergeWaves = 4;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ void load8(const void* base, bool fp32, int64_t off, float (&v)[8]) {
  if (fp32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
    const f32x4 a = p[0], b = p[1];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(base) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
  }
}

__device__ __forceinline__ void store_out(const MergeParams& p, int t, int h, int lane, const float (&acc)[8],
                                          float lse) {
  if (p.out_fp32) {
    f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + t * p.o_st + h * p.o_sh + 8 * lane);
    o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (__bf16)acc[i];
    *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(p.out) + t * p.o_st + h * p.o_sh + 8 * lane) = b;
  }
  if (p.lse != nullptr && lane == 0) p.lse[t * p.l_st + h * p.l_sh] = lse;
}

// SM > 0: S <= SM, and every partial LSE, then every partial row, is loaded in one batch so
// a wave waits for two memory round trips in all.  SM == 0: any S, one partial at a time.
template <int SM>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (pair >= (int64_t)p.T * p.H) return;
  const int t = (int)(pair / p.H);
  const int h = (int)(pair - (int64_t)t * p.H);
  const float* lrow = p.lparts + t * p.lp_st + h * p.lp_sh;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;

  if constexpr (SM > 0) {
    float ls[SM];
#pragma unroll
    for (int s = 0; s < SM; ++s) ls[s] = s < p.S ? lrow[s * p.lp_ss] : -INFINITY;
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < SM; ++s) m = fmaxf(m, ls[s]);
    if (m != -INFINITY) {
      float tot = 0.0f;
#pragma unroll
      for (int s = 0; s < SM; ++s) tot += s < p.S ? exp2f((ls[s] - m) * kLog2e) : 0.0f;
      lse = m + logf(tot);
      float v[SM][8];
#pragma unroll
      for (int s = 0; s < SM; ++s) {
        if (ls[s] != -INFINITY) {  // an empty partial contributes nothing and is not read
          load8(p.parts, p.part_fp32, s * p.p_ss + t * p.p_st + h * p.p_sh + 8 * lane, v[s]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[s][i] = 0.0f;
        }
      }
#pragma unroll
      for (int s = 0; s < SM; ++s) {
        if (ls[s] == -INFINITY) continue;
        const float w = exp2f((ls[s] - lse) * kLog2e);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += w * v[s][i];
      }
    }
  } else {
    float m = -INFINITY;
    for (int s = 0; s < p.S; ++s) m = fmaxf(m, lrow[s * p.lp_ss]);
    if (m != -INFINITY) {
      float tot = 0.0f;
      for (int s = 0; s < p.S; ++s) tot += exp2f((lrow[s * p.lp_ss] - m) * kLog2e);
      lse = m + logf(tot);
      for (int s = 0; s < p.S; ++s) {
        const float ls = lrow[s * p.lp_ss];
        if (ls == -INFINITY) continue;  // an empty partial contributes nothing
        const float w = exp2f((ls - lse) * kLog2e);
        float v[8];
        load8(p.parts, p.part_fp32, s * p.p_ss + t * p.p_st + h * p.p_sh + 8 * lane, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += w * v[i];
      }
    }
  }
  store_out(p, t, h, lane, acc, lse);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t pairs = (int64_t)p.T * p.H;
  const unsigned grid = (unsigned)((pairs + kMergeWaves - 1) / kMergeWaves);
  const dim3 g(grid), b(kMergeWaves * 64);
  if (p.S <= 2)
    hipLaunchKernelGGL(merge_kernel<2>, g, b, 0, stream, p);
  else if (p.S <= 4)
    hipLaunchKernelGGL(merge_kernel<4>, g, b, 0, stream, p);
  else if (p.S <= 8)
    hipLaunchKernelGGL(merge_kernel<8>, g, b, 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<0>, g, b, 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
