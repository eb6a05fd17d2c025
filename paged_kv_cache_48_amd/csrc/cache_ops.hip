// Slot mapping and the KV scatter into the block pool (gfx950).
//
// weft, "Cache layouts": the paged per-layer view is [N, P, H_kv, D] and a
// write scatters through slot_mapping.  ember, "The core idea": position p of
// a request lives at block block_table[p / P], offset p % P.  With the slot
// encoding slot = block * P + offset, the [H_kv, D] row of one token is
// contiguous both in the packed input and in the pool, so the scatter is a
// row copy: it moves raw bits and does no floating-point work.
#include "common.h"
#include "launch.h"

namespace pa {

// One thread per new token.  The request is found by binary search over
// cu_seqlens (largest b with cu[b] <= t, which skips empty requests).
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ lens, int32_t* __restrict__ slots, int num_seqs,
    int64_t num_tokens, int block_size, int max_blocks) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int64_t T = (int64_t)cu[b + 1] - cu[b];
  const int64_t pos = (int64_t)lens[b] - T + (t - cu[b]);
  int32_t slot = -1;
  if (pos >= 0 && pos < (int64_t)max_blocks * block_size) {
    const int64_t blk = block_table[(int64_t)b * max_blocks + pos / block_size];
    slot = (int32_t)(blk * block_size + pos % block_size);
  }
  slots[t] = slot;
}

// One wave per token (grid-stride over tokens): lane i moves 16-byte pieces
// i, i+64, ... of the token's K row and of its V row.  A wave reads and writes
// 1 KiB contiguous per step, and the slot is one uniform load per token.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const u32x4_t* __restrict__ k, const u32x4_t* __restrict__ v,
    const int32_t* __restrict__ slots, u32x4_t* __restrict__ kc, u32x4_t* __restrict__ vc,
    int64_t num_tokens, int pieces_per_row, int64_t pool_rows) {
  const int lane = lane_id();
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); t < num_tokens;
       t += waves) {
    const int64_t s = slots[t];
    if (s < 0 || s >= pool_rows) continue;
    const u32x4_t* ks = k + t * pieces_per_row;
    const u32x4_t* vs = v + t * pieces_per_row;
    u32x4_t* kd = kc + s * pieces_per_row;
    u32x4_t* vd = vc + s * pieces_per_row;
    for (int c = lane; c < pieces_per_row; c += 64) {
      const u32x4_t kv = __builtin_nontemporal_load(ks + c);
      const u32x4_t vv = __builtin_nontemporal_load(vs + c);
      kd[c] = kv;
      vd[c] = vv;
    }
  }
}

hipError_t launch_slot_mapping(const int32_t* block_table, const int32_t* cu_seqlens,
                               const int32_t* context_lens, int32_t* slot_mapping, int num_seqs,
                               int64_t num_tokens, int block_size, int max_blocks,
                               hipStream_t stream) {
  const int64_t blocks = (num_tokens + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     block_table, cu_seqlens, context_lens, slot_mapping, num_seqs, num_tokens,
                     block_size, max_blocks);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, const int32_t* slot_mapping,
                                    void* k_cache, void* v_cache, int64_t num_tokens,
                                    int64_t pool_rows, int row_bytes, hipStream_t stream) {
  const int pieces = row_bytes / 16;
  int64_t blocks = (num_tokens + 3) / 4;  // 4 waves per block, one token each
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4_t*)k, (const u32x4_t*)v, slot_mapping, (u32x4_t*)k_cache,
                     (u32x4_t*)v_cache, num_tokens, pieces, pool_rows);
  return hipGetLastError();
}

}  // namespace pa
