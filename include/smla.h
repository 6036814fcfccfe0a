/*
 * smla.h - sparse MLA decode over indexer top-k ids against a packed fp8_ds_mla
 * latent KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources: the operations below are the hot path described on three pages:
 *   [P-FlashMLA] "FlashMLA sparse fp8 path gains DCP and MTP" (prhub.com.cn
 *                summary of vLLM pull request 46514)
 *   [P-SM120]    "[eldritch] attention: support DCP in SM120 FlashInfer sparse MLA"
 *                (local-inference-lab/vllm pull request 60)
 *   [P-Stab]     "[Bugfix][Attention] Stabilize sparse-MLA DCP for GLM PCP evals"
 *                (vllm-project/vllm pull request 55879)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees, copies to or from the host, or synchronises: each call
 *    validates its scalar arguments on the host, enqueues kernels on `stream`, and
 *    returns before the work is done.  Scalars travel by value as kernel arguments,
 *    so no per-call host-to-device copy exists ([P-Stab] "Root causes and fixes",
 *    "DCP decode rank scalar"), and calls may be captured in a HIP graph.
 *  - Strides are in ELEMENTS of the pointed-to type.
 *  - Errors are found from the arguments alone, before anything is launched; a call
 *    that returns an error has enqueued nothing ("fail closed", [P-FlashMLA]
 *    "Executive summary").  SMLA_ERR_HIP reports a launch failure.
 *  - T = 0 is a no-op that returns SMLA_OK ([P-Stab] "Root causes and fixes",
 *    "Zero-local-sequence DCP warmup rank").
 *  - fp8_ds_mla record (656 bytes per token; [P-FlashMLA] "Related" gives the
 *    656-byte size, [P-SM120] "Scope / Limitations" the packed fp8 layout):
 *      bytes [0,512)   512 latent values, OCP e4m3fn codes
 *      bytes [512,528) 4 little-endian fp32 scales; scale i covers dims 128i..128i+127
 *      bytes [528,656) 64 rope values, little-endian bf16
 *    Record s starts at kv_cache + 656*s.  The latent value of dim d is
 *    e4m3(code[d]) * scale[d/128]; the key is [latent | rope] (576 wide), the value
 *    is the latent (512 wide).  The pages give only the size, not the byte order;
 *    this order is this library's own.
 */
#ifndef SMLA_H_
#define SMLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 3

/* Bytes of the per-device scratch array behind sparse_mla_decode_noalloc (32 MiB). */
#define SMLA_NOALLOC_SCRATCH_BYTES (32u << 20)

enum smla_status {
  SMLA_OK = 0,
  SMLA_ERR_INVALID_ARG = 1, /* null required pointer, negative size or stride        */
  SMLA_ERR_UNSUPPORTED = 2, /* a size or mode outside what the kernels implement      */
  SMLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the queried size     */
  SMLA_ERR_MISALIGNED = 4,  /* a pointer or stride breaks the alignment stated below  */
  SMLA_ERR_HIP = 5          /* the HIP runtime refused a launch                       */
};

enum smla_dtype { SMLA_BF16 = 0, SMLA_FP32 = 1 };

/* ABI version of the loaded library (SMLA_ABI_VERSION). */
int smla_abi_version(void);

/* Static text for a status code; never NULL. */
const char* smla_status_string(int status);

/*
 * sparse_mla_convert_index - global top-k token ids -> physical cache slots.
 *
 * [P-FlashMLA] "Implementation breakdown" step 2 and "Key source snippets"
 * (_forward_fp8_kv_mixed_batch); [P-SM120] "Summary" and "Implementation Notes"
 * (global ids converted to this DCP rank's local physical KV slots, valid counts
 * passed on as per-token sequence lengths).
 *
 * For every row t < T and entry j < K, with id = topk_ids[t*ids_ld + j]:
 *   - id < 0 -> -1.
 *   - dcp_size == 1: pos = id.  dcp_size = D > 1 with interleave I: the id is kept
 *     only if (id / I) % D == dcp_rank, and then pos = (id / (I*D)) * I + id % I
 *     (the shard-local token position); ids of other ranks become -1 IN PLACE, the
 *     valid entries are not moved to the front.
 *   - b = req_id_per_token[t]; blk = pos / block_size.  If b < 0, b >= bt_rows,
 *     blk >= bt_width or block_table[b*bt_ld + blk] < 0 the entry is -1; otherwise
 *     slots[t*slots_ld + j] = block_table[b*bt_ld + blk] * block_size + pos % block_size.
 *   valid_count[t] (optional, may be NULL) = number of entries of row t that are not -1.
 *
 * topk_ids [T, >=K] int32; req_id_per_token [T] int32 (the first T rows);
 * block_table [bt_rows, bt_ld] int32 (the shard's own table when dcp_size > 1);
 * slots [T, >=K] int32 output; slots may be topk_ids itself when slots_ld == ids_ld.
 * With K = 0 the index pointers may be NULL; only valid_count (zeros) is written.
 * Requirements: T, K >= 0; block_size >= 1; dcp_size >= 1; dcp_rank >= 0; interleave >= 1;
 * ids_ld, slots_ld >= K; bt_ld >= bt_width >= 1; bt_rows >= 1 (else SMLA_ERR_INVALID_ARG);
 * dcp_rank < dcp_size (else SMLA_ERR_UNSUPPORTED: no such rank in the group);
 * int32 pointers 4-byte aligned (packed index arrays may be only 4-byte aligned,
 * [P-Stab] "Root causes and fixes", "PCP+DCP first-request JIT keys").
 */
int sparse_mla_convert_index(const int32_t* topk_ids, int64_t ids_ld, const int32_t* req_id_per_token,
                             const int32_t* block_table, int64_t bt_ld, int32_t bt_rows, int32_t bt_width,
                             int32_t T, int32_t K, int32_t block_size, int32_t dcp_size, int32_t dcp_rank,
                             int32_t interleave, int32_t* slots, int64_t slots_ld, int32_t* valid_count,
                             hipStream_t stream);

/*
 * sparse_mla_decode_workspace_size - bytes of workspace sparse_mla_decode needs for
 * these sizes and split count (num_splits = 0: the automatic plan on the current
 * device).  0 means the call needs no workspace.  [P-SM120] "Implementation Notes"
 * (scratch per device, allocated up front, not lazily on the first decode);
 * [P-Stab] "Root causes and fixes", "FlashInfer sparse-MLA DCP workspace" (the
 * softmax-stats slab grows with gathered heads and scheduled tokens).
 */
size_t sparse_mla_decode_workspace_size(int32_t T, int32_t H, int32_t K, int32_t num_splits);

/*
 * sparse_mla_decode - softmax attention of each query row over its own top-k
 * candidate records, returning the output and the log-sum-exp.
 *
 * [P-FlashMLA] "Key source snippets" (the fp8 kernel returns out and LSE; -1 slots
 * are masked natively) and "Implementation breakdown" steps 1 and 3 (LSE returned
 * for the cross-rank merge; rows without a candidate are neutralised to out = 0,
 * lse = -inf, the merge identity); [P-SM120] "Why" (decode must return the LSE so
 * DCP partials can be merged) and "Implementation Notes" (the head count comes from
 * the runtime query tensor).
 *
 * For row t and head h, with J = the entries of slots[t*slots_ld + 0..K) that lie
 * in [0, num_slots) (every other entry, -1 included, is skipped; each kept entry is
 * its own term):  s_j = softmax_scale * <q[t,h,:], key_j>,
 *   lse[t,h] = ln sum_j exp(s_j),  out[t,h,:] = sum_j exp(s_j - lse[t,h]) * value_j.
 * A row with no kept entry gives out = 0 and lse = -inf.
 *
 * q        bf16 [T, H, 576] at q + t*q_stride_t + h*q_stride_h (dims contiguous);
 *          q, q_stride_t and q_stride_h*2 bytes must keep every head 16-byte aligned.
 * kv_cache [num_slots, 656] bytes, 16-byte aligned.
 * slots    int32 [T, >=K], 4-byte aligned (output of sparse_mla_convert_index).
 * valid_count  int32 [T] or NULL, 4-byte aligned: the per-row counts sparse_mla_convert_index
 *          returns ([P-SM120] "Summary": valid counts passed to the launcher as per-token
 *          lengths).  A row whose count is <= 0 is written as out = 0, lse = -inf without
 *          reading its q or its slots (the empty-row mask taken from the conversion,
 *          [P-FlashMLA] "Review highlights"); any other count is not used, the slots decide.
 * out      [T, H, 512] bf16 (out_dtype SMLA_BF16) or fp32 (SMLA_FP32) at
 *          out + t*out_stride_t + h*out_stride_h, dims contiguous, 16-byte aligned rows.
 * lse      fp32 at lse + t*lse_stride_t + h*lse_stride_h: (T,H) layout with strides
 *          (H,1), or the kernel-native (H,T) layout with strides (1,T) ([P-FlashMLA]
 *          "Implementation breakdown" step 1).
 * num_splits  0 = automatic; otherwise the number of top-k ranges each row is cut
 *          into (1..64).  With more than one, the decode kernel leaves fp32 partials
 *          in the workspace and a second kernel on the same stream merges them.
 * workspace   device memory of at least sparse_mla_decode_workspace_size(T,H,K,
 *          num_splits) bytes, 256-byte aligned, any contents (every byte read is
 *          written first by the same call); may be NULL when the size is 0.
 *          Calls that share a workspace must be ordered (same stream); concurrent
 *          ones race.
 * Supported: 1 <= H <= 128, H % 16 == 0; K <= 4096 * num_splits (automatic splits
 * always satisfy this); softmax_scale finite and > 0.
 */
int sparse_mla_decode(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                      int64_t num_slots, const int32_t* slots, int64_t slots_ld, const int32_t* valid_count,
                      int32_t T, int32_t H, int32_t K, float softmax_scale, void* out, int32_t out_dtype,
                      int64_t out_stride_t,
                      int64_t out_stride_h, float* lse, int64_t lse_stride_t, int64_t lse_stride_h,
                      int32_t num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_mla_decode_noalloc - sparse_mla_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The call allocates nothing and calls no allocating routine; its split
 * partials live in a scratch array the library holds on each device it runs on
 * (SMLA_NOALLOC_SCRATCH_BYTES, kept until the process ends).
 *
 * Arguments, layouts, results and errors are those of sparse_mla_decode (same kernels, same
 * split plan), except: the workspace is the library's scratch array; a call whose split plan
 * needs more than SMLA_NOALLOC_SCRATCH_BYTES (see sparse_mla_decode_workspace_size) returns
 * SMLA_ERR_WORKSPACE and launches nothing; SMLA_ERR_HIP if the runtime cannot give the scratch
 * array's device address.  Every call on one device shares that device's array (each call
 * writes every byte of it that it reads), so calls on one device must not overlap in time
 * (calls on different streams of one device race).
 */
int sparse_mla_decode_noalloc(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                              int64_t num_slots, const int32_t* slots, int64_t slots_ld, const int32_t* valid_count,
                              int32_t T, int32_t H, int32_t K, float softmax_scale, void* out, int32_t out_dtype,
                              int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                              int64_t lse_stride_h, int32_t num_splits, hipStream_t stream);

/*
 * sparse_mla_decode_bf16 - sparse_mla_decode over a plain bf16 latent cache instead of the
 * packed fp8_ds_mla one.
 *
 * [P-FlashMLA] "Related" (the 576-value layout against the 656-byte packed one) and
 * "Risks and impact" (the bf16 sparse path, which the pages' serving stack keeps out of
 * its DCP support; here every call works the same for both layouts).
 *
 * kv_cache  [num_slots, 1152] bytes, 16-byte aligned: record s = 576 little-endian bf16
 *           values at kv_cache + 1152*s, the 512 latent values then the 64 rope values;
 *           key = all 576, value = the 512 latent values.
 * Every other argument, the workspace (sparse_mla_decode_workspace_size), the result and
 * the errors are those of sparse_mla_decode.
 */
int sparse_mla_decode_bf16(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                           int64_t num_slots, const int32_t* slots, int64_t slots_ld, const int32_t* valid_count,
                           int32_t T, int32_t H, int32_t K, float softmax_scale, void* out, int32_t out_dtype,
                           int64_t out_stride_t,
                           int64_t out_stride_h, float* lse, int64_t lse_stride_t, int64_t lse_stride_h,
                           int32_t num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_mla_merge_lse - combine S partial results over disjoint KV shards.
 *
 * [P-FlashMLA] "Implementation breakdown" steps 1 and 3 (the shared DCP merge
 * consumes out and a (T,H) LSE; (0, -inf) is its identity, so an empty shard is
 * dropped and never brings in NaN); [P-SM120] "Summary" and "Why" (partial
 * attention results of DCP ranks are reduced with the returned LSE).
 *
 *   lse[t,h] = ln sum_s exp(lse_s[t,h]),
 *   out[t,h,:] = sum_s exp(lse_s[t,h] - lse[t,h]) * out_s[t,h,:];
 *   an entry whose lse_s are all -inf gives out = 0, lse = -inf.
 *
 * out_parts  [S, T, H, 512] in part_dtype at out_parts + s*p_stride_s + t*p_stride_t +
 *            h*p_stride_h (dims contiguous, 16-byte aligned rows).
 * lse_parts  fp32 at lse_parts + s*lp_stride_s + t*lp_stride_t + h*lp_stride_h (any
 *            layout, (H,T) included).
 * out        [T, H, 512] in out_dtype (16-byte aligned rows); lse fp32, may be NULL.
 * Supported: 1 <= S <= 64, H >= 1.
 */
int sparse_mla_merge_lse(const void* out_parts, int32_t part_dtype, int64_t p_stride_s, int64_t p_stride_t,
                         int64_t p_stride_h, const float* lse_parts, int64_t lp_stride_s, int64_t lp_stride_t,
                         int64_t lp_stride_h, int32_t S, int32_t T, int32_t H, void* out, int32_t out_dtype,
                         int64_t o_stride_t, int64_t o_stride_h, float* lse, int64_t l_stride_t,
                         int64_t l_stride_h, hipStream_t stream);

/*
 * sparse_mla_dense_decode_workspace_size - bytes of workspace sparse_mla_dense_decode
 * needs: the per-row slot lists (B*S rows of the width below, 4 bytes each) plus the
 * workspace of the decode that reads them (automatic split plan on the current device).
 * 0 for invalid sizes.
 */
size_t sparse_mla_dense_decode_workspace_size(int32_t B, int32_t S, int32_t H, int32_t max_seq_len,
                                              int32_t dcp_size, int32_t interleave);

/*
 * sparse_mla_dense_decode - MLA decode over each request's whole paged context, with S
 * query tokens per request (speculative / MTP decode), on one DCP rank.
 *
 * [P-FlashMLA] "Implementation breakdown" step 5 and the flashmla.py forward_mqa snippet:
 * the dense decode returns out and an LSE that the DCP merge consumes as
 * [batch * seq_len, heads]; here the rows are written in that order directly (row
 * t = b*S + s), so no flatten copy exists.
 *
 * Row t = b*S + s is query token s of request b, at position p = seq_lens[b] - S + s; it
 * attends to every position 0..p of request b (p < 0: no position, out = 0, lse = -inf).
 * With dcp_size = D > 1 the rank sees only the positions it owns ((pos / I) % D ==
 * dcp_rank), stored at its local positions 0, 1, ... through block_table (this rank's
 * table, [bt_rows, bt_ld]); the partial results of the D ranks merge with
 * sparse_mla_merge_lse into the unsharded result.  Everything else (q, kv_cache, out, lse,
 * softmax_scale, H, their layouts and alignment) is as in sparse_mla_decode with T = B*S.
 *
 * seq_lens  int32 [B]; every entry must be <= max_seq_len, which sizes the slot lists
 *           (a longer context is cut at max_seq_len).  Requests b >= bt_rows have no
 *           context on this rank.
 * workspace at least sparse_mla_dense_decode_workspace_size(B, S, H, max_seq_len,
 *           dcp_size, interleave) bytes, 256-byte aligned; never NULL when B*S > 0.
 * Supported: the slot-list width (max_seq_len, or the rank-0 share of it under DCP) up to
 * 262144 (64 splits of 4096 entries); H as in sparse_mla_decode; dcp_rank < dcp_size
 * (else SMLA_ERR_UNSUPPORTED).
 */
int sparse_mla_dense_decode(const void* q, int64_t q_stride_t, int64_t q_stride_h, const uint8_t* kv_cache,
                            int64_t num_slots, const int32_t* block_table, int64_t bt_ld, int32_t bt_rows,
                            int32_t bt_width, const int32_t* seq_lens, int32_t B, int32_t S, int32_t H,
                            int32_t block_size, int32_t dcp_size, int32_t dcp_rank, int32_t interleave,
                            int32_t max_seq_len, float softmax_scale, void* out, int32_t out_dtype,
                            int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                            int64_t lse_stride_h, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_mla_cache_write - quantise new tokens into fp8_ds_mla records and store each
 * at the slot this DCP rank owns for it.
 *
 * Placement follows the id-to-slot rule of sparse_mla_convert_index applied to the
 * token's request position ([P-FlashMLA] "Implementation breakdown" step 2; "Review
 * highlights" item 2: a slot mapping of ctx_pos / block_size that ignores DCP
 * disagrees with the DCP-aware mapping the reads use).  For token i < N with
 * p = positions[i] and b = req_id[i]: if p < 0, or dcp_size > 1 and this rank does not
 * own p ((p / I) % D != dcp_rank), or the block is missing (b outside [0, bt_rows),
 * block >= bt_width, table entry < 0), or the slot is >= num_slots, nothing is
 * written and slot_mapping[i] = -1; otherwise the record goes to that slot and
 * slot_mapping[i] is the slot.
 *
 * Record contents (the pages do not give the quantiser): per 128-value latent tile
 * scale = fp32(amax / 448), 1.0 if that is not positive; code = the e4m3fn value
 * nearest to fp32(x / scale), ties to the even code, magnitudes above 448
 * saturating to 448, the sign bit of x kept; rope = nearest-even bf16 of the input.
 * Inputs must be finite.
 *
 * latent    [N, 512] at latent + i*latent_stride (dims contiguous), in_dtype SMLA_BF16 or
 *           SMLA_FP32; 16-byte aligned rows.  rope [N, 64] at rope + i*rope_stride, same
 *           dtype, element-aligned.
 * positions, req_id  int32 [N]; block_table int32 [bt_rows, bt_ld] (this rank's table).
 * kv_cache  [num_slots, 656] bytes, 16-byte aligned; slot_mapping int32 [N] or NULL.
 * Two tokens that map to the same slot race (the caller keeps positions distinct).
 * Requirements as for sparse_mla_convert_index; dcp_size * interleave <= 2^30.
 */
int sparse_mla_cache_write(const void* latent, int64_t latent_stride, const void* rope, int64_t rope_stride,
                           int32_t in_dtype, const int32_t* positions, const int32_t* req_id,
                           const int32_t* block_table, int64_t bt_ld, int32_t bt_rows, int32_t bt_width, int32_t N,
                           int32_t block_size, int32_t dcp_size, int32_t dcp_rank, int32_t interleave,
                           uint8_t* kv_cache, int64_t num_slots, int32_t* slot_mapping, hipStream_t stream);

/*
 * sparse_mla_dcp_local_seq_lens - how many positions below each request's length the
 * rank owns: local_seq_lens[i] = #{ p in [0, seq_lens[i]) : (p / I) % D == dcp_rank }
 * = (L / (I*D)) * I + clamp(L % (I*D) - dcp_rank*I, 0, I), 0 for L <= 0.
 * [P-Stab] "Root causes and fixes", "DCP decode rank scalar" (get_dcp_local_seq_lens;
 * the rank travels as a kernel argument, so no per-call device scalar is built).
 * seq_lens, local_seq_lens: int32 [R], 4-byte aligned.  dcp_rank >= dcp_size (or
 * dcp_size * interleave > 2^30) gives SMLA_ERR_UNSUPPORTED.
 */
int sparse_mla_dcp_local_seq_lens(const int32_t* seq_lens, int32_t R, int32_t dcp_size, int32_t dcp_rank,
                                  int32_t interleave, int32_t* local_seq_lens, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H_ */
