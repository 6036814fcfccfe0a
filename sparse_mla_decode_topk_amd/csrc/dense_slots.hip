// Slot lists of whole-context (dense) MLA decode rows, for the top-k decode kernel.
//
// Page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation breakdown" step 5 and
// the flashmla.py forward_mqa snippet: the dense path attends over a request's whole paged
// context, with seq_len query tokens per request under speculative decode, and the DCP merge
// consumes its LSE as [batch * seq_len, heads] rows.  Here row b * S + s is query token s of
// request b, at position seq_lens[b] - S + s; it sees every position up to its own, and on a
// DCP rank the positions of that range the rank owns, which are the rank's first n local
// positions (n = its local length of position + 1).  This kernel writes those n local slots
// (block table walk) followed by -1 up to the list width; the top-k decode kernel then runs
// on the lists unchanged, and its (T, H) LSE rows are already the flattened layout.
//
// One workgroup per row, consecutive lanes on consecutive list entries (coalesced int32
// stores); the block table row is read from L2.

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kSlotThreads = 256;

// Positions below L that DCP rank r owns (interleave I): (L / (I D)) I + clamp(L % (I D) - r I, 0, I).
__device__ __forceinline__ int64_t owned_below(int64_t L, int D, int r, int I) {
  if (L <= 0) return 0;
  if (D == 1) return L;
  const int64_t cyc = (int64_t)I * D;
  const int64_t rem = L % cyc - (int64_t)r * I;
  return (L / cyc) * I + (rem < 0 ? 0 : (rem > I ? I : rem));
}

__global__ __launch_bounds__(kSlotThreads) void dense_slots_kernel(DenseSlotParams p) {
  const int t = blockIdx.x;
  const int b = t / p.S;
  const int s = t - b * p.S;
  int32_t* out = p.slots + (int64_t)t * p.K;
  int64_t n = 0;
  if (b < p.bt_rows) {
    const int64_t pos = (int64_t)p.seq_lens[b] - p.S + s;  // this query token's position
    n = owned_below(pos + 1, p.dcp_size, p.dcp_rank, p.interleave);
    if (n > p.K) n = p.K;  // contexts beyond the stated maximum are cut there
  }
  const int32_t* btrow = p.bt + (int64_t)(b < p.bt_rows ? b : 0) * p.bt_ld;
  const int B = p.block_size;
  for (int j = threadIdx.x; j < p.K; j += kSlotThreads) {
    int slot = -1;
    if (j < n) {
      const int blk = j / B;
      if (blk < p.bt_width) {
        const int phys = btrow[blk];
        if (phys >= 0) {
          const int64_t v = (int64_t)phys * B + (j - blk * B);
          slot = v <= 0x7fffffffLL ? (int)v : -1;
        }
      }
    }
    out[j] = slot;
  }
}

}  // namespace

int64_t dense_list_width(int64_t max_seq_len, int dcp_size, int interleave) {
  // rank 0 owns the most positions below any length
  if (max_seq_len <= 0) return 1;
  if (dcp_size == 1) return max_seq_len;
  const int64_t cyc = (int64_t)interleave * dcp_size;
  const int64_t rem = max_seq_len % cyc;
  const int64_t n = (max_seq_len / cyc) * interleave + (rem > interleave ? interleave : rem);
  return n > 0 ? n : 1;
}

hipError_t launch_dense_slots(const DenseSlotParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(dense_slots_kernel, dim3((unsigned)p.T), dim3(kSlotThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
