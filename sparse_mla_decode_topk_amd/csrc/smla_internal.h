// Internal declarations shared by the HIP sources of libsmla (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kHeadDim = kLatent + kRope;  // 576
constexpr int kRecordBytes = 656;          // 512 e4m3 codes + 4 fp32 scales + 64 bf16 rope
constexpr int kScaleOffset = 512;
constexpr int kRopeOffset = 528;
constexpr int kMaxEntriesPerSplit = 4096;  // slot entries one decode workgroup compacts
constexpr int kMaxSplits = 64;
constexpr int kHeadsPerBlock = 64;           // heads one workgroup of the bf16-record decode covers
constexpr int kRowHeads = 64;                // heads one workgroup of the fp8_ds_mla decode covers
constexpr int kRowGroup = 4;                 // consecutive rows whose decode work items share an XCD

// Workgroups of a decode launch: the work items of groups of kRowGroup rows, the groups dealt
// round-robin to the 8 XCDs (see block_of); slots past the last item stay idle.
inline int64_t decode_grid(int64_t T, int64_t head_blocks, int64_t splits) {
  const int64_t per_group = kRowGroup * head_blocks * splits;
  const int64_t groups = (T + kRowGroup - 1) / kRowGroup;
  return 8 * ((groups + 7) / 8) * per_group;
}

struct ConvertParams {
  const int32_t* ids;
  int64_t ids_ld;
  const int32_t* req;
  const int32_t* bt;
  int64_t bt_ld;
  int32_t bt_rows, bt_width;
  int32_t T, K, block_size, dcp_size, dcp_rank, interleave;
  int32_t* slots;
  int64_t slots_ld;
  int32_t* valid;
  int32_t lg_block, lg_dcp, lg_interleave;  // log2 of block_size, dcp_size, interleave; -1: not a power of two
};

struct DecodeParams {
  const uint16_t* q;
  int64_t q_st, q_sh;
  const uint8_t* kv;
  int64_t num_slots;
  const int32_t* slots;
  int64_t slots_ld;
  const int32_t* valid;  // [T] optional: a row whose count is <= 0 is empty and its list is not read
  int32_t T, H, K;
  float scale_log2;  // softmax_scale * log2(e)
  void* out;
  int32_t out_fp32;
  int64_t o_st, o_sh;
  float* lse;
  int64_t l_st, l_sh;
  int32_t splits, entries_per_split, head_blocks, heads_per_block;
  float* ws_o;    // [T, splits, H, 512] unnormalised partial outputs
  float* ws_ml;   // [T, splits, H, 2]   (running max in log2 units, sum)
};

struct MergeParams {
  const void* parts;
  int32_t part_fp32;
  int64_t p_ss, p_st, p_sh;
  const float* lparts;
  int64_t lp_ss, lp_st, lp_sh;
  int32_t S, T, H;
  void* out;
  int32_t out_fp32;
  int64_t o_st, o_sh;
  float* lse;
  int64_t l_st, l_sh;
};

struct CacheWriteParams {
  const void* latent;  // [N, 512] bf16 or fp32, row stride latent_st elements
  const void* rope;    // [N, 64] same dtype, row stride rope_st elements
  int64_t latent_st, rope_st;
  int32_t in_fp32;
  const int32_t* pos;  // [N] position of the token in its request
  const int32_t* req;  // [N] request of the token
  const int32_t* bt;
  int64_t bt_ld;
  int32_t bt_rows, bt_width;
  int32_t N, block_size, dcp_size, dcp_rank, interleave;
  uint8_t* cache;
  int64_t num_slots;
  int32_t* slot_mapping;  // [N] optional
  int32_t lg_block, lg_dcp, lg_interleave;  // log2 of block_size, dcp_size, interleave; -1: not a power of two
};

struct DenseSlotParams {
  const int32_t* seq_lens;  // [B] context length of each request
  const int32_t* bt;
  int64_t bt_ld;
  int32_t bt_rows, bt_width;
  int32_t T, S, K, block_size, dcp_size, dcp_rank, interleave;
  int32_t* slots;  // [T, K] out
};

struct DecodePlan {
  int32_t head_blocks;  // workgroups per row along heads
  int32_t splits;       // top-k ranges per row
  int32_t entries_per_split;
  size_t ws_o_bytes, ws_ml_bytes, ws_total;
};

hipError_t launch_convert(const ConvertParams& p, hipStream_t stream);
hipError_t launch_decode_row(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream);
// The merge of a split decode's partials (p.splits > 1) into out and lse.
hipError_t launch_split_combine(const DecodeParams& p, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream);
hipError_t launch_dense_slots(const DenseSlotParams& p, hipStream_t stream);
int64_t dense_list_width(int64_t max_seq_len, int dcp_size, int interleave);
hipError_t launch_local_lens(const int32_t* seq_lens, int32_t R, int32_t D, int32_t r, int32_t I, int32_t* out,
                             hipStream_t stream);

}  // namespace smla
