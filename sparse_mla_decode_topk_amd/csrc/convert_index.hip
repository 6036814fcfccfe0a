// Global top-k token ids -> physical (or DCP shard-local) cache slots.
//
// Page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown" step 2 and
// "Key source snippets": without DCP each id goes through its request's block table; under
// DCP ids owned by other ranks become -1 in place (no front compaction) and owned ids become
// slots of the rank's local cache.  Page "[eldritch] attention: support DCP in SM120
// FlashInfer sparse MLA", "Summary": the per-row valid counts are produced alongside.
//
// One workgroup per row; consecutive lanes take consecutive entries (coalesced int32
// traffic), the row's valid count is a workgroup reduction, so no atomics and no pre-zeroed
// output are needed.

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kConvThreads = 256;

__global__ __launch_bounds__(kConvThreads) void convert_kernel(ConvertParams p) {
  __shared__ int wsum[kConvThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* ids = p.ids + (int64_t)t * p.ids_ld;
  int32_t* out = p.slots + (int64_t)t * p.slots_ld;
  const int b = p.K > 0 ? p.req[t] : -1;  // with no entries nothing but the count is written
  const bool req_ok = b >= 0 && b < p.bt_rows;
  const int32_t* btrow = p.bt + (int64_t)(req_ok ? b : 0) * p.bt_ld;
  const int D = p.dcp_size, I = p.interleave, r = p.dcp_rank, B = p.block_size;
  int count = 0;
  for (int j = tid; j < p.K; j += kConvThreads) {
    const int id = ids[j];
    int slot = -1;
    if (id >= 0 && req_ok) {
      bool own = true;
      int pos = id;
      if (D > 1) {
        const int g = id / I;
        own = (g % D) == r;
        pos = (g / D) * I + (id - g * I);
      }
      if (own) {
        const int blk = pos / B;
        if (blk < p.bt_width) {
          const int phys = btrow[blk];
          if (phys >= 0) {
            const int64_t s = (int64_t)phys * B + (pos - blk * B);
            slot = s <= 0x7fffffffLL ? (int)s : -1;
          }
        }
      }
    }
    out[j] = slot;
    count += slot >= 0;
  }
  if (p.valid == nullptr) return;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) count += __shfl_xor(count, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = count;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kConvThreads / 64; ++w) s += wsum[w];
    p.valid[t] = s;
  }
}

}  // namespace

hipError_t launch_convert(const ConvertParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(convert_kernel, dim3(p.T), dim3(kConvThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
