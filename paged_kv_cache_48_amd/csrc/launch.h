// Host launchers of the gfx950 kernels.  Called from api.hip after argument
// validation; every launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum DType : int { kF32 = 0, kBF16 = 1, kFP8E4M3 = 2 };

// Tokens per split-context partition of the decode kernel.  A request with
// context L is cut into ceil(L / kPartTokens) partitions; this depends on L
// only, never on the batch, so a request's result does not depend on its
// neighbours.
constexpr int kPartTokens = 256;

// Largest max_blocks_per_seq the prefill kernel takes: an item's block ids
// are staged in LDS (64 KiB of them).
constexpr int kPrefillMaxBlocks = 16384;

// Compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_slot_mapping(const int32_t* block_table, const int32_t* cu_seqlens,
                               const int32_t* context_lens, int32_t* slot_mapping, int num_seqs,
                               int64_t num_tokens, int block_size, int max_blocks, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* k, const void* v, const int32_t* slot_mapping,
                                    void* k_cache, void* v_cache, int64_t num_tokens,
                                    int64_t pool_rows, int row_bytes, hipStream_t stream);

hipError_t launch_reshape_and_cache_fp8(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache,
                                        void* v_cache, const float* k_scale, const float* v_scale,
                                        int64_t num_tokens, int64_t pool_rows, int row_elems, int head_dim,
                                        int src_dtype, hipStream_t stream);

hipError_t launch_check_metadata(const int32_t* block_table, const int32_t* context_lens, const int32_t* cu_seqlens,
                                 const int32_t* slot_mapping, int num_seqs, int64_t num_tokens, int64_t num_blocks,
                                 int block_size, int max_blocks, int32_t* result, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int64_t num_pairs,
                              int64_t num_blocks, int64_t block_bytes, hipStream_t stream);
// Read-only stream over `bytes` (a multiple of 16) at `src`: HBM read ceiling.
hipError_t launch_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int num_workgroups, hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens;  // prefill and mixed only
  const int32_t* block_table;
  const int32_t* context_lens;
  void* out;
  float scale;
  int num_seqs;
  int64_t num_q_tokens;  // prefill and mixed only
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int64_t num_blocks;
  int max_blocks;
  int dtype;     // q and out (and the pools, unless kv_dtype is kFP8E4M3)
  int kv_dtype;  // the pools' element type
  const float* k_scale;  // kFP8E4M3 pools: per-KV-head scales
  const float* v_scale;
  void* workspace;
  // decode with append: each request's new token [num_seqs, H_kv, D] (null
  // otherwise), of type new_dtype (the pools' type; fp8 pools: kF32 or kBF16)
  const void* k_new;
  const void* v_new;
  int new_dtype;
};

size_t decode_workspace_size(int num_seqs, int num_q_heads, int head_dim, int block_size,
                             int max_blocks);
hipError_t launch_decode(const AttnArgs& a, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop);

size_t prefill_workspace_size(int num_seqs, int64_t num_q_tokens, int num_q_heads,
                              int num_kv_heads);
hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream, hipEvent_t ev_start,
                          hipEvent_t ev_stop);

// Mixed batches (one-token chunks as decodes, longer chunks as prefill) in one
// persistent launch, then the merge of the decodes' partitions.  Batches of
// at most mixed_max_seqs() requests whose work lists fit the queue counters
// (mixed_fits); bf16 q and out, bf16 or fp8 pools.
size_t mixed_workspace_size(int num_seqs, int num_q_heads, int head_dim, int block_size, int max_blocks);
int mixed_max_seqs();
bool mixed_fits(int num_seqs, int64_t num_q_tokens, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                int max_blocks);
hipError_t launch_mixed(const AttnArgs& a, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

// Decode and mixed workspaces keep a sticky status word (give-ups of a work
// queue) at this byte offset of their header; prefill leaves it alone.  The
// kernel copies it to result[0] and clears it.
constexpr size_t kStatusWordOffset = 1008;
hipError_t launch_workspace_status(void* workspace, int32_t* result, hipStream_t stream);

}  // namespace pa
