// New tokens -> fp8_ds_mla records at their DCP-local cache slots, and per-request local
// sequence lengths under DCP.
//
// Placement: page "FlashMLA sparse fp8 path gains DCP and MTP", "Review highlights", item 2
// (the slot mapping of a new token must follow the DCP ownership that reads use, not
// ctx_pos // block_size) and "Implementation breakdown" step 2 (ownership and local
// position of an id under DCP).  Local lengths: page "[Bugfix][Attention] Stabilize
// sparse-MLA DCP for GLM PCP evals", "Root causes and fixes", subsection "DCP decode rank
// scalar" (get_dcp_local_seq_lens; the rank arrives here as a kernel argument, so nothing is
// built on the device per call).  The record's quantiser is not on the pages: per 128-value
// tile the scale is fp32(amax / 448) (1.0 when that is not positive), each value becomes the
// nearest e4m3fn value to fp32(x / scale) (ties to even, saturating at 448, sign kept), rope
// is rounded to bf16.
//
// Eight waves per workgroup, one wave per two tokens: lane l quantises latent dims 8l .. 8l+7 (scale tile l / 16, its
// amax a reduction over 16 lanes) and rope dim l of each, and writes its 8 code bytes, its
// rope value and, for the first lane of a tile, the tile's scale.  The input rows, positions
// and requests of both tokens are loaded before the block-table lookups, so a wave waits for
// two memory round trips.  Per value the correctly rounded quotient costs one multiply and two
// fused multiply-adds against a per-tile reciprocal, and the e4m3 rounding is the hardware
// convert.  1152 B (bf16 in) or 2304 B (fp32 in) read and 656 B written per token.

#include "smla_internal.h"

#include <math.h>

namespace smla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kCwWaves = 8;
constexpr int kTokPerWave = 2;  // tokens per wave, their loads in flight together

// fp32(x / s) for s > 0 from the correctly rounded reciprocal r = fp32(1 / s): q0 = fp32(x r)
// lies within an ulp of x / s, the fused residual x - q0 s is exact, and one fused correction
// step then gives the correctly rounded quotient (Markstein's theorem; r must be the rounded
// reciprocal and s not so small that 1 / s overflows -- the caller divides directly then).
// The sign is restored for x = +-0, where the residual step would return +0.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
}

// Four quotients -> four e4m3fn codes (v_cvt_pk_fp8_f32: nearest, ties to even, sign kept).
// The quotients of a tile never exceed 448 (1 + 2^-23), which rounds to 448, so no
// saturation is needed.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Nearest-even bf16 bits of a finite fp32 value.
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// Where this rank writes the token at position `pos` of request `b`: returns the offset in
// its local block and sets blk_out to the block-table column of that block (the caller loads
// the entry), or returns -1 with blk_out = -1 when the rank does not write the token.
__device__ __forceinline__ int64_t token_slot(const CacheWriteParams& p, int pos, int b, int& blk_out) {
  blk_out = -1;
  if (pos < 0 || b < 0 || b >= p.bt_rows) return -1;
  const int D = p.dcp_size, I = p.interleave, B = p.block_size;
  int local = pos;
  if (D > 1) {
    const int g = p.lg_interleave >= 0 ? pos >> p.lg_interleave : pos / I;
    const int gd = p.lg_dcp >= 0 ? g >> p.lg_dcp : g / D;
    if (g - gd * D != p.dcp_rank) return -1;
    local = gd * I + (pos - g * I);
  }
  const int blk = p.lg_block >= 0 ? local >> p.lg_block : local / B;
  if (blk >= p.bt_width) return -1;
  blk_out = blk;
  return local - blk * B;  // offset in the block
}

__global__ __launch_bounds__(kCwWaves * 64) void cache_write_kernel(CacheWriteParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t i0 = ((int64_t)blockIdx.x * kCwWaves + (threadIdx.x >> 6)) * kTokPerWave;
  if (i0 >= p.N) return;

  // ---- every load that does not depend on the slot first: position, request, latent dims
  // 8 lane .. 8 lane + 7 and rope dim `lane` of each of the wave's tokens
  int pos[kTokPerWave], req[kTokPerWave];
  float x[kTokPerWave][8], rope[kTokPerWave];
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    const int64_t i = i0 + j < p.N ? i0 + j : i0;  // a missing second token re-reads the first
    pos[j] = i0 + j < p.N ? p.pos[i] : -1;
    req[j] = p.req[i];
    if (p.in_fp32) {
      const float* lp = reinterpret_cast<const float*>(p.latent) + i * p.latent_st + 8 * lane;
      const f32x4 a = *reinterpret_cast<const f32x4*>(lp), c = *reinterpret_cast<const f32x4*>(lp + 4);
      x[j][0] = a[0]; x[j][1] = a[1]; x[j][2] = a[2]; x[j][3] = a[3];
      x[j][4] = c[0]; x[j][5] = c[1]; x[j][6] = c[2]; x[j][7] = c[3];
      rope[j] = reinterpret_cast<const float*>(p.rope)[i * p.rope_st + lane];
    } else {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p.latent) +
                                                        i * p.latent_st + 8 * lane);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[j][k] = (float)v[k];
      rope[j] = (float)reinterpret_cast<const __bf16*>(p.rope)[i * p.rope_st + lane];
    }
  }
  // ---- this rank's slots (the id-to-slot rule of the reads): one block-table load each
  int64_t slot[kTokPerWave];
  int phys[kTokPerWave];
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    int blk;
    slot[j] = token_slot(p, pos[j], req[j], blk);
    phys[j] = blk >= 0 ? p.bt[(int64_t)req[j] * p.bt_ld + blk] : -1;
  }
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    if (i0 + j >= p.N) break;
    int64_t s = -1;
    if (phys[j] >= 0) {
      s = (int64_t)phys[j] * p.block_size + slot[j];
      if (s >= p.num_slots) s = -1;
    }
    if (p.slot_mapping != nullptr && lane == 0) p.slot_mapping[i0 + j] = (int32_t)s;
    if (s < 0) continue;

    // ---- tile scale: amax over the 16 lanes of the tile
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(x[j][k]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
    float scale = am / 448.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    float y[8];
    if (scale >= 0x1p-100f) {
      const float r = 1.0f / scale;
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = div_by_scale(x[j][k], scale, r);
    } else {  // 1 / scale could overflow: divide directly (only for denormal-sized tiles)
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = x[j][k] / scale;
    }
    const uint32_t lo = pack_e4m3x4(y[0], y[1], y[2], y[3]);
    const uint32_t hi = pack_e4m3x4(y[4], y[5], y[6], y[7]);

    uint8_t* rec = p.cache + s * kRecordBytes;
    // streaming stores: the records are not read again by this kernel
    __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(rec + 8 * lane));
    if ((lane & 15) == 0)
      __builtin_nontemporal_store(scale, reinterpret_cast<float*>(rec + kScaleOffset + 4 * (lane >> 4)));
    __builtin_nontemporal_store(bf16_bits(rope[j]), reinterpret_cast<uint16_t*>(rec + kRopeOffset + 2 * lane));
  }
}

__global__ void local_lens_kernel(const int32_t* seq_lens, int32_t R, int32_t D, int32_t r, int32_t I,
                                  int32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= R) return;
  const int64_t L = seq_lens[i];
  int64_t n = 0;
  if (L > 0) {
    const int64_t cyc = (int64_t)I * D;  // one round of I positions per rank
    const int64_t rem = L % cyc - (int64_t)r * I;
    n = (L / cyc) * I + (rem < 0 ? 0 : (rem > I ? I : rem));
  }
  out[i] = (int32_t)n;
}

int log2_exact(int v) {
  if (v < 1 || (v & (v - 1)) != 0) return -1;
  int lg = 0;
  while ((1 << lg) < v) ++lg;
  return lg;
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p_in, hipStream_t stream) {
  CacheWriteParams p = p_in;
  p.lg_block = log2_exact(p.block_size);
  p.lg_dcp = log2_exact(p.dcp_size);
  p.lg_interleave = log2_exact(p.interleave);
  const int64_t per_wg = (int64_t)kCwWaves * kTokPerWave;
  const unsigned grid = (unsigned)((p.N + per_wg - 1) / per_wg);
  hipLaunchKernelGGL(cache_write_kernel, dim3(grid), dim3(kCwWaves * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_local_lens(const int32_t* seq_lens, int32_t R, int32_t D, int32_t r, int32_t I, int32_t* out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(local_lens_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, stream, seq_lens, R, D, r, I,
                     out);
  return hipGetLastError();
}

}  // namespace smla
