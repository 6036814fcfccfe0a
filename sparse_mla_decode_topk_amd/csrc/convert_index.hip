// Global top-k token ids -> physical (or DCP shard-local) cache slots.
//
// Page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown" step 2 and
// "Key source snippets": without DCP each id goes through its request's block table; under
// DCP ids owned by other ranks become -1 in place (no front compaction) and owned ids become
// slots of the rank's local cache.  Page "[eldritch] attention: support DCP in SM120
// FlashInfer sparse MLA", "Summary": the per-row valid counts are produced alongside.
//
// One workgroup per row; consecutive lanes take consecutive entries (coalesced int32
// traffic).  Each thread handles PER entries per pass with all of their id loads in flight
// together, then all of their block-table loads, so a row costs two dependent memory round
// trips instead of two per entry.  A batch of up to 1024 rows runs 1024 threads per row (two
// entries each for top-k 2048: the few workgroups then keep more loads in flight per CU); a
// larger one runs 256 (eight each), which measured faster once the rows fill the GPU several
// times over.  Power-of-two block size, DCP size and interleave (the
// usual case) take shifts and masks instead of integer division.  The row's valid count is
// a workgroup reduction, so no atomics and no pre-zeroed output are needed.

#include "smla_internal.h"

namespace smla {
namespace {

// x / d and x % d for x >= 0, d >= 1; `lg` is log2(d) when d is a power of two, else -1.
__device__ __forceinline__ int div_pos(int x, int d, int lg) { return lg >= 0 ? x >> lg : x / d; }
__device__ __forceinline__ int mod_pos(int x, int d, int lg) { return lg >= 0 ? x & (d - 1) : x % d; }

template <int NT, int PER>
__global__ __launch_bounds__(NT) void convert_kernel(ConvertParams p) {
  __shared__ int wsum[NT / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* ids = p.ids + (int64_t)t * p.ids_ld;
  int32_t* out = p.slots + (int64_t)t * p.slots_ld;
  const int b = p.K > 0 ? p.req[t] : -1;  // with no entries nothing but the count is written
  const bool req_ok = b >= 0 && b < p.bt_rows;
  const int32_t* btrow = p.bt + (int64_t)(req_ok ? b : 0) * p.bt_ld;
  const int D = p.dcp_size, I = p.interleave, r = p.dcp_rank, B = p.block_size;
  int count = 0;
  for (int base = 0; base < p.K; base += NT * PER) {
    int id[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = base + i * NT + tid;
      id[i] = j < p.K ? ids[j] : -1;
    }
    int blk[PER], off[PER];  // block-table column and offset in the block; blk = -1: no slot
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      blk[i] = -1;
      off[i] = 0;
      const int x = id[i];
      if (x >= 0 && req_ok) {
        bool own = true;
        int pos = x;
        if (D > 1) {
          const int g = div_pos(x, I, p.lg_interleave);
          own = mod_pos(g, D, p.lg_dcp) == r;
          pos = div_pos(g, D, p.lg_dcp) * I + (x - g * I);
        }
        const int bi = div_pos(pos, B, p.lg_block);
        if (own && bi < p.bt_width) {
          blk[i] = bi;
          off[i] = pos - bi * B;
        }
      }
    }
    int phys[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) phys[i] = blk[i] >= 0 ? btrow[blk[i]] : -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = base + i * NT + tid;
      int slot = -1;
      if (phys[i] >= 0) {
        const int64_t s = (int64_t)phys[i] * B + off[i];
        slot = s <= 0x7fffffffLL ? (int)s : -1;
      }
      if (j < p.K) out[j] = slot;
      count += slot >= 0;
    }
  }
  if (p.valid == nullptr) return;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) count += __shfl_xor(count, o);
  if ((tid & 63) == 0) wsum[tid >> 6] = count;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += wsum[w];
    p.valid[t] = s;
  }
}

int log2_exact(int v) {
  if (v < 1 || (v & (v - 1)) != 0) return -1;
  int lg = 0;
  while ((1 << lg) < v) ++lg;
  return lg;
}

}  // namespace

hipError_t launch_convert(const ConvertParams& p_in, hipStream_t stream) {
  ConvertParams p = p_in;
  p.lg_block = log2_exact(p.block_size);
  p.lg_dcp = log2_exact(p.dcp_size);
  p.lg_interleave = log2_exact(p.interleave);
  if (p.T <= 1024)
    hipLaunchKernelGGL((convert_kernel<1024, 2>), dim3(p.T), dim3(1024), 0, stream, p);
  else
    hipLaunchKernelGGL((convert_kernel<256, 8>), dim3(p.T), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
