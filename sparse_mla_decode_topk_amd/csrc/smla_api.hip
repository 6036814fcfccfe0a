// C-ABI entry points of libsmla: argument validation, split planning and kernel launches.
// Declared and documented in include/smla.h.  Nothing here allocates, copies or synchronises.

#include "../../include/smla.h"
#include "smla_internal.h"

#include <atomic>
#include <math.h>

using namespace smla;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device (cached; 256 if the runtime cannot say).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Split plan for a decode call whose workgroups cover `hpb` heads of a row (kRowHeads for the
// fp8_ds_mla decode, kHeadsPerBlock for the bf16-record decode).  Either allows one workgroup
// per CU.  Rows are cut into top-k ranges only when (row, head
// block) pairs cannot cover every CU of the device.
DecodePlan make_plan(int32_t T, int32_t H, int32_t K, int32_t num_splits, int cus, int hpb) {
  DecodePlan pl{};
  pl.head_blocks = (H + hpb - 1) / hpb;
  const int min_splits = K > 0 ? (K + kMaxEntriesPerSplit - 1) / kMaxEntriesPerSplit : 1;
  int splits;
  if (num_splits > 0) {
    splits = num_splits;
  } else {
    const int64_t wgs = (int64_t)T * pl.head_blocks;
    const int64_t slots = (int64_t)cus;
    splits = 1;
    if (wgs > 0 && wgs < slots) {
      const int64_t want = (slots + wgs - 1) / wgs;
      const int64_t cap = K / 256 > 1 ? K / 256 : 1;  // keep >= 256 entries (8 tiles) per split
      splits = (int)(want < cap ? want : cap);
    }
    if (splits < min_splits) splits = min_splits;
    if (splits > kMaxSplits) splits = kMaxSplits;
  }
  pl.splits = splits;
  pl.entries_per_split = K > 0 ? (K + splits - 1) / splits : 1;
  if (splits > 1) {
    pl.ws_o_bytes = round_up((size_t)T * splits * H * kLatent * sizeof(float), 256);
    pl.ws_ml_bytes = round_up((size_t)T * splits * H * 2 * sizeof(float), 256);
  }
  pl.ws_total = pl.ws_o_bytes + pl.ws_ml_bytes;
  return pl;
}

// Workspace that covers a decode call of either record layout for these sizes.
size_t decode_workspace(int32_t T, int32_t H, int32_t K, int32_t num_splits, int cus) {
  const size_t a = make_plan(T, H, K, num_splits, cus, kRowHeads).ws_total;
  const size_t b = make_plan(T, H, K, num_splits, cus, kHeadsPerBlock).ws_total;
  return a > b ? a : b;
}

}  // namespace

extern "C" {

int smla_abi_version(void) { return SMLA_ABI_VERSION; }

const char* smla_status_string(int status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or stride, bad dtype)";
    case SMLA_ERR_UNSUPPORTED: return "unsupported size or mode";
    case SMLA_ERR_WORKSPACE: return "workspace missing or smaller than sparse_mla_decode_workspace_size()";
    case SMLA_ERR_MISALIGNED: return "pointer or stride breaks the required alignment";
    case SMLA_ERR_HIP: return "HIP runtime error while launching";
    default: return "unknown status";
  }
}

int sparse_mla_convert_index(const int32_t* topk_ids, int64_t ids_ld, const int32_t* req_id_per_token,
                             const int32_t* block_table, int64_t bt_ld, int32_t bt_rows, int32_t bt_width,
                             int32_t T, int32_t K, int32_t block_size, int32_t dcp_size, int32_t dcp_rank,
                             int32_t interleave, int32_t* slots, int64_t slots_ld, int32_t* valid_count,
                             hipStream_t stream) {
  if (T < 0 || K < 0) return SMLA_ERR_INVALID_ARG;
  if (block_size < 1 || dcp_size < 1 || dcp_rank < 0 || interleave < 1) return SMLA_ERR_INVALID_ARG;
  if (bt_rows < 1 || bt_width < 1 || bt_ld < bt_width || ids_ld < K || slots_ld < K) return SMLA_ERR_INVALID_ARG;
  if (dcp_rank >= dcp_size) return SMLA_ERR_UNSUPPORTED;
  if (T == 0) return SMLA_OK;
  if (K > 0 && (!topk_ids || !req_id_per_token || !block_table || !slots)) return SMLA_ERR_INVALID_ARG;
  if (K > 0 && reinterpret_cast<const void*>(slots) == reinterpret_cast<const void*>(topk_ids) && slots_ld != ids_ld)
    return SMLA_ERR_INVALID_ARG;
  if (!aligned(topk_ids, 4) || !aligned(req_id_per_token, 4) || !aligned(block_table, 4) || !aligned(slots, 4) ||
      (valid_count && !aligned(valid_count, 4)))
    return SMLA_ERR_MISALIGNED;
  if (K == 0 && valid_count == nullptr) return SMLA_OK;
  ConvertParams p{};
  p.ids = topk_ids;
  p.ids_ld = ids_ld;
  p.req = req_id_per_token;
  p.bt = block_table;
  p.bt_ld = bt_ld;
  p.bt_rows = bt_rows;
  p.bt_width = bt_width;
  p.T = T;
  p.K = K;
  p.block_size = block_size;
  p.dcp_size = dcp_size;
  p.dcp_rank = dcp_rank;
  p.interleave = interleave;
  p.slots = slots;
  p.slots_ld = slots_ld;
  p.valid = valid_count;
  return launch_convert(p, stream) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

size_t sparse_mla_decode_workspace_size(int32_t T, int32_t H, int32_t K, int32_t num_splits) {
  if (T <= 0 || H < 1 || K < 0 || num_splits < 0 || num_splits > kMaxSplits) return 0;
  return decode_workspace(T, H, K, num_splits, num_splits > 0 ? 256 : device_cus());
}

}  // extern "C"

namespace {

// Validation and launch parameters of a decode call; nothing is launched.  Shared by the
// top-k decode and the whole-context decode (which builds its slot lists first).
int prepare_decode(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache, int64_t num_slots,
                   const int32_t* slots, int64_t slots_ld, const int32_t* valid_count, int32_t T, int32_t H, int32_t K, float softmax_scale,
                   void* out, int32_t out_dtype, int64_t out_stride_t, int64_t out_stride_h, float* lse,
                   int64_t lse_stride_t, int64_t lse_stride_h, int32_t num_splits, void* workspace,
                   size_t workspace_bytes, int hpb, DecodeParams& p, DecodePlan& plan) {
  if (T < 0 || H < 1 || K < 0 || num_slots < 0) return SMLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return SMLA_ERR_INVALID_ARG;
  if (out_dtype != SMLA_BF16 && out_dtype != SMLA_FP32) return SMLA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > kMaxSplits) return SMLA_ERR_INVALID_ARG;
  if (q_stride_t < 0 || q_stride_h < 0 || out_stride_t < 0 || out_stride_h < 0 || lse_stride_t < 0 ||
      lse_stride_h < 0 || slots_ld < K)
    return SMLA_ERR_INVALID_ARG;
  if (H > 128 || H % 16 != 0) return SMLA_ERR_UNSUPPORTED;
  if (T == 0) return SMLA_OK;
  if (!q || !out || !lse || (K > 0 && !slots) || (num_slots > 0 && !kv_cache)) return SMLA_ERR_INVALID_ARG;
  if (num_slots > 0x7fffffffLL) return SMLA_ERR_UNSUPPORTED;  // slots are int32
  const int64_t ovec = out_dtype == SMLA_FP32 ? 4 : 8;  // elements per 16 bytes
  if (!aligned(q, 16) || q_stride_t % 8 != 0 || q_stride_h % 8 != 0 || (kv_cache && !aligned(kv_cache, 16)) ||
      (slots && !aligned(slots, 4)) || (valid_count && !aligned(valid_count, 4)) || !aligned(out, 16) || out_stride_t % ovec != 0 ||
      out_stride_h % ovec != 0 || !aligned(lse, 4))
    return SMLA_ERR_MISALIGNED;
  const int cus = num_splits > 0 ? 256 : device_cus();
  plan = make_plan(T, H, K, num_splits, cus, hpb);
  if ((int64_t)K > (int64_t)plan.splits * kMaxEntriesPerSplit) return SMLA_ERR_UNSUPPORTED;
  if (decode_grid(T, plan.head_blocks, plan.splits) > 0x7fffffffLL) return SMLA_ERR_UNSUPPORTED;
  if (plan.ws_total > 0) {
    if (!workspace || workspace_bytes < plan.ws_total) return SMLA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SMLA_ERR_MISALIGNED;
  }
  p = DecodeParams{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_st = q_stride_t;
  p.q_sh = q_stride_h;
  p.kv = kv_cache;
  p.num_slots = num_slots;
  p.slots = slots;
  p.slots_ld = slots_ld;
  p.valid = valid_count;
  p.T = T;
  p.H = H;
  p.K = K;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.out = out;
  p.out_fp32 = out_dtype == SMLA_FP32;
  p.o_st = out_stride_t;
  p.o_sh = out_stride_h;
  p.lse = lse;
  p.l_st = lse_stride_t;
  p.l_sh = lse_stride_h;
  p.splits = plan.splits;
  p.entries_per_split = plan.entries_per_split;
  p.head_blocks = plan.head_blocks;
  p.heads_per_block = hpb;
  if (plan.ws_total > 0) {
    char* ws = static_cast<char*>(workspace);
    p.ws_ml = reinterpret_cast<float*>(ws);
    p.ws_o = reinterpret_cast<float*>(ws + plan.ws_ml_bytes);
  }
  return SMLA_OK;
}

// Bytes of the slot lists a whole-context decode keeps at the front of its workspace.
size_t dense_slots_bytes(int64_t T, int64_t K) { return round_up((size_t)T * (size_t)K * sizeof(int32_t), 256); }

// Workspace of sparse_mla_decode_noalloc: one copy per device, held until the process ends.  In
// host code `scratch` names a host-side stand-in, not the device memory: the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[SMLA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, or null if the runtime cannot give it.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  g_scratch[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" {

int sparse_mla_decode(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                      int64_t num_slots, const int32_t* slots, int64_t slots_ld, const int32_t* valid_count,
                      int32_t T, int32_t H,
                      int32_t K, float softmax_scale, void* out, int32_t out_dtype, int64_t out_stride_t,
                      int64_t out_stride_h, float* lse, int64_t lse_stride_t, int64_t lse_stride_h,
                      int32_t num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodeParams p;
  DecodePlan plan;
  const int st = prepare_decode(q, q_stride_t, q_stride_h, kv_cache, num_slots, slots, slots_ld, valid_count, T, H, K,
                                softmax_scale, out, out_dtype, out_stride_t, out_stride_h, lse, lse_stride_t,
                                lse_stride_h, num_splits, workspace, workspace_bytes, kRowHeads, p, plan);
  if (st != SMLA_OK || T == 0) return st;
  return launch_decode_row(p, plan, stream) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

int sparse_mla_decode_noalloc(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                              int64_t num_slots, const int32_t* slots, int64_t slots_ld, const int32_t* valid_count,
                              int32_t T, int32_t H, int32_t K, float softmax_scale, void* out, int32_t out_dtype,
                              int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                              int64_t lse_stride_h, int32_t num_splits, hipStream_t stream) {
  void* ws = scratch_address();
  if (!ws) return SMLA_ERR_HIP;
  DecodeParams p;
  DecodePlan plan;
  const int st = prepare_decode(q, q_stride_t, q_stride_h, kv_cache, num_slots, slots, slots_ld, valid_count, T, H, K,
                                softmax_scale, out, out_dtype, out_stride_t, out_stride_h, lse, lse_stride_t,
                                lse_stride_h, num_splits, ws, SMLA_NOALLOC_SCRATCH_BYTES, kRowHeads, p, plan);
  if (st != SMLA_OK || T == 0) return st;
  return launch_decode_row(p, plan, stream) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

int sparse_mla_decode_bf16(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                      int64_t num_slots, const int32_t* slots, int64_t slots_ld, const int32_t* valid_count,
                      int32_t T, int32_t H,
                           int32_t K, float softmax_scale, void* out, int32_t out_dtype, int64_t out_stride_t,
                           int64_t out_stride_h, float* lse, int64_t lse_stride_t, int64_t lse_stride_h,
                           int32_t num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodeParams p;
  DecodePlan plan;
  const int st = prepare_decode(q, q_stride_t, q_stride_h, kv_cache, num_slots, slots, slots_ld, valid_count, T, H, K,
                                softmax_scale, out, out_dtype, out_stride_t, out_stride_h, lse, lse_stride_t,
                                lse_stride_h, num_splits, workspace, workspace_bytes, kHeadsPerBlock, p, plan);
  if (st != SMLA_OK || T == 0) return st;
  return launch_decode_bf16(p, plan, stream) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

size_t sparse_mla_dense_decode_workspace_size(int32_t B, int32_t S, int32_t H, int32_t max_seq_len,
                                              int32_t dcp_size, int32_t interleave) {
  if (B <= 0 || S < 1 || H < 1 || max_seq_len < 0 || dcp_size < 1 || interleave < 1) return 0;
  if ((int64_t)dcp_size * interleave > (1 << 30) || (int64_t)B * S > 0x7fffffffLL) return 0;
  const int64_t T = (int64_t)B * S;
  const int64_t K = dense_list_width(max_seq_len, dcp_size, interleave);
  if (K > (int64_t)kMaxSplits * kMaxEntriesPerSplit) return 0;
  return dense_slots_bytes(T, K) + make_plan((int32_t)T, H, (int32_t)K, 0, device_cus(), kRowHeads).ws_total;
}

int sparse_mla_dense_decode(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                            int64_t num_slots, const int32_t* block_table, int64_t bt_ld, int32_t bt_rows,
                            int32_t bt_width, const int32_t* seq_lens, int32_t B, int32_t S, int32_t H,
                            int32_t block_size, int32_t dcp_size, int32_t dcp_rank, int32_t interleave,
                            int32_t max_seq_len, float softmax_scale, void* out, int32_t out_dtype,
                            int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                            int64_t lse_stride_h, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || S < 1 || H < 1 || max_seq_len < 0 || block_size < 1) return SMLA_ERR_INVALID_ARG;
  if (dcp_size < 1 || dcp_rank < 0 || interleave < 1) return SMLA_ERR_INVALID_ARG;
  if (bt_rows < 1 || bt_width < 1 || bt_ld < bt_width) return SMLA_ERR_INVALID_ARG;
  if (dcp_rank >= dcp_size) return SMLA_ERR_UNSUPPORTED;
  if ((int64_t)dcp_size * interleave > (1 << 30) || (int64_t)B * S > 0x7fffffffLL) return SMLA_ERR_UNSUPPORTED;
  const int64_t T = (int64_t)B * S;
  const int64_t K = dense_list_width(max_seq_len, dcp_size, interleave);
  if (K > (int64_t)kMaxSplits * kMaxEntriesPerSplit) return SMLA_ERR_UNSUPPORTED;
  if (T == 0) return SMLA_OK;
  if (!seq_lens || !block_table) return SMLA_ERR_INVALID_ARG;
  if (!aligned(seq_lens, 4) || !aligned(block_table, 4)) return SMLA_ERR_MISALIGNED;
  if (!workspace) return SMLA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return SMLA_ERR_MISALIGNED;
  const size_t lists = dense_slots_bytes(T, K);
  if (workspace_bytes < lists) return SMLA_ERR_WORKSPACE;
  int32_t* slots = static_cast<int32_t*>(workspace);
  DecodeParams p;
  DecodePlan plan;
  const int st = prepare_decode(q, q_stride_t, q_stride_h, kv_cache, num_slots, slots, K, nullptr, (int32_t)T, H,
                                (int32_t)K, softmax_scale, out, out_dtype, out_stride_t, out_stride_h, lse,
                                lse_stride_t, lse_stride_h, 0, static_cast<char*>(workspace) + lists,
                                workspace_bytes - lists, kRowHeads, p, plan);
  if (st != SMLA_OK) return st;
  DenseSlotParams d{};
  d.seq_lens = seq_lens;
  d.bt = block_table;
  d.bt_ld = bt_ld;
  d.bt_rows = bt_rows;
  d.bt_width = bt_width;
  d.T = (int32_t)T;
  d.S = S;
  d.K = (int32_t)K;
  d.block_size = block_size;
  d.dcp_size = dcp_size;
  d.dcp_rank = dcp_rank;
  d.interleave = interleave;
  d.slots = slots;
  if (launch_dense_slots(d, stream) != hipSuccess) return SMLA_ERR_HIP;
  return launch_decode_row(p, plan, stream) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

int sparse_mla_merge_lse(const void* out_parts, int32_t part_dtype, int64_t p_stride_s, int64_t p_stride_t,
                         int64_t p_stride_h, const float* lse_parts, int64_t lp_stride_s, int64_t lp_stride_t,
                         int64_t lp_stride_h, int32_t S, int32_t T, int32_t H, void* out, int32_t out_dtype,
                         int64_t o_stride_t, int64_t o_stride_h, float* lse, int64_t l_stride_t,
                         int64_t l_stride_h, hipStream_t stream) {
  if (S < 1 || T < 0 || H < 1) return SMLA_ERR_INVALID_ARG;
  if (S > kMaxSplits) return SMLA_ERR_UNSUPPORTED;
  if ((part_dtype != SMLA_BF16 && part_dtype != SMLA_FP32) || (out_dtype != SMLA_BF16 && out_dtype != SMLA_FP32))
    return SMLA_ERR_INVALID_ARG;
  if (p_stride_s < 0 || p_stride_t < 0 || p_stride_h < 0 || lp_stride_s < 0 || lp_stride_t < 0 || lp_stride_h < 0 ||
      o_stride_t < 0 || o_stride_h < 0 || l_stride_t < 0 || l_stride_h < 0)
    return SMLA_ERR_INVALID_ARG;
  if (T == 0) return SMLA_OK;
  if (!out_parts || !lse_parts || !out) return SMLA_ERR_INVALID_ARG;
  const int64_t pvec = part_dtype == SMLA_FP32 ? 4 : 8, ovec = out_dtype == SMLA_FP32 ? 4 : 8;
  if (!aligned(out_parts, 16) || p_stride_s % pvec || p_stride_t % pvec || p_stride_h % pvec ||
      !aligned(lse_parts, 4) || !aligned(out, 16) || o_stride_t % ovec || o_stride_h % ovec ||
      (lse && !aligned(lse, 4)))
    return SMLA_ERR_MISALIGNED;
  MergeParams p{};
  p.parts = out_parts;
  p.part_fp32 = part_dtype == SMLA_FP32;
  p.p_ss = p_stride_s;
  p.p_st = p_stride_t;
  p.p_sh = p_stride_h;
  p.lparts = lse_parts;
  p.lp_ss = lp_stride_s;
  p.lp_st = lp_stride_t;
  p.lp_sh = lp_stride_h;
  p.S = S;
  p.T = T;
  p.H = H;
  p.out = out;
  p.out_fp32 = out_dtype == SMLA_FP32;
  p.o_st = o_stride_t;
  p.o_sh = o_stride_h;
  p.lse = lse;
  p.l_st = l_stride_t;
  p.l_sh = l_stride_h;
  return launch_merge(p, stream) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

int sparse_mla_cache_write(const void* latent, int64_t latent_stride, const void* rope, int64_t rope_stride,
                           int32_t in_dtype, const int32_t* positions, const int32_t* req_id,
                           const int32_t* block_table, int64_t bt_ld, int32_t bt_rows, int32_t bt_width, int32_t N,
                           int32_t block_size, int32_t dcp_size, int32_t dcp_rank, int32_t interleave,
                           uint8_t* kv_cache, int64_t num_slots, int32_t* slot_mapping, hipStream_t stream) {
  if (N < 0 || num_slots < 0 || latent_stride < 0 || rope_stride < 0) return SMLA_ERR_INVALID_ARG;
  if (in_dtype != SMLA_BF16 && in_dtype != SMLA_FP32) return SMLA_ERR_INVALID_ARG;
  if (block_size < 1 || dcp_size < 1 || dcp_rank < 0 || interleave < 1) return SMLA_ERR_INVALID_ARG;
  if (bt_rows < 1 || bt_width < 1 || bt_ld < bt_width) return SMLA_ERR_INVALID_ARG;
  if (dcp_rank >= dcp_size || (int64_t)dcp_size * interleave > (1 << 30)) return SMLA_ERR_UNSUPPORTED;
  if (N == 0) return SMLA_OK;
  if (!latent || !rope || !positions || !req_id || !block_table || (num_slots > 0 && !kv_cache))
    return SMLA_ERR_INVALID_ARG;
  if (N > 1 && (latent_stride < kLatent || rope_stride < kRope)) return SMLA_ERR_INVALID_ARG;
  const int64_t lvec = in_dtype == SMLA_FP32 ? 4 : 8;  // elements per 16 bytes
  const int64_t esz = in_dtype == SMLA_FP32 ? 4 : 2;
  if (!aligned(latent, 16) || latent_stride % lvec != 0 || !aligned(rope, esz) || !aligned(positions, 4) ||
      !aligned(req_id, 4) || !aligned(block_table, 4) || (kv_cache && !aligned(kv_cache, 16)) ||
      (slot_mapping && !aligned(slot_mapping, 4)))
    return SMLA_ERR_MISALIGNED;
  CacheWriteParams p{};
  p.latent = latent;
  p.rope = rope;
  p.latent_st = latent_stride;
  p.rope_st = rope_stride;
  p.in_fp32 = in_dtype == SMLA_FP32;
  p.pos = positions;
  p.req = req_id;
  p.bt = block_table;
  p.bt_ld = bt_ld;
  p.bt_rows = bt_rows;
  p.bt_width = bt_width;
  p.N = N;
  p.block_size = block_size;
  p.dcp_size = dcp_size;
  p.dcp_rank = dcp_rank;
  p.interleave = interleave;
  p.cache = kv_cache;
  p.num_slots = num_slots;
  p.slot_mapping = slot_mapping;
  return launch_cache_write(p, stream) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

int sparse_mla_dcp_local_seq_lens(const int32_t* seq_lens, int32_t R, int32_t dcp_size, int32_t dcp_rank,
                                  int32_t interleave, int32_t* local_seq_lens, hipStream_t stream) {
  if (R < 0 || dcp_size < 1 || dcp_rank < 0 || interleave < 1) return SMLA_ERR_INVALID_ARG;
  if (dcp_rank >= dcp_size || (int64_t)dcp_size * interleave > (1 << 30)) return SMLA_ERR_UNSUPPORTED;
  if (R == 0) return SMLA_OK;
  if (!seq_lens || !local_seq_lens) return SMLA_ERR_INVALID_ARG;
  if (!aligned(seq_lens, 4) || !aligned(local_seq_lens, 4)) return SMLA_ERR_MISALIGNED;
  return launch_local_lens(seq_lens, R, dcp_size, dcp_rank, interleave, local_seq_lens, stream) == hipSuccess
             ? SMLA_OK
             : SMLA_ERR_HIP;
}

}  // extern "C"
