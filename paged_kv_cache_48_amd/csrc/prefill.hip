// Varlen / chunked prefill attention over the paged cache for gfx950 (bf16 MFMA).
//
// What is computed (tiny-vllm-py, "KV Cache" and "Mistakes I made"; ember,
// "Deliberately out of scope" for chunked prefill; weft, "Shapes and symbols"
// for the T_total packing): request b's chunk of T_b new tokens is already in
// the pool; chunk row i sits at absolute position L_b - T_b + i and attends
// causally to keys 0 .. L_b - T_b + i of KV head h / G:
//     out[row, h] = sum_{j <= pos} softmax_j(scale * q[row, h] . k_j) v_j.
//
// Design (MI355X):
//   * Work item = (request, tile of TQ = 256 / G chunk tokens, KV head).  The
//     G query heads that share a KV head are packed into the item's 256 rows
//     (head-major), so each K/V tile fetched from the pool serves all of them.
//   * A persistent grid of one 8-wave workgroup per CU (two waves per SIMD,
//     so one's softmax overlaps the other's matrix products) pulls items from a
//     queue that a plan kernel sorts by decreasing key count (largest causal
//     extents first).
//   * The item's block ids are copied to LDS first, so no gather address
//     waits on a global load (a wait on one would drain the loads in flight,
//     which complete in order).
//   * Per 64-key tile, four waves gather K rows and four gather V rows through
//     the block table (16-byte loads), and both are stored row-major in LDS
//     (the same work for every wave).  The K operand is a contiguous LDS
//     read; the V^T operand of the P.V product comes from gfx950's
//     transposing LDS read (ds_read_b64_tr_b16).  Two register sets and two
//     LDS buffers keep the loads of the next two tiles in flight while one
//     tile computes; one barrier per tile.  Waves 4-7 stage the next tile
//     before their products and waves 0-3 after them, so the two waves that
//     share a SIMD overlap staging with matrix work.
//   * Each wave owns 32 rows.  S^T = K Q^T and O^T += V^T P^T run as
//     16x16x32 bf16 MFMAs with fp32 accumulation.  Computing the transposed
//     scores leaves each lane holding one query row's scores for a run of keys,
//     which is exactly the B-operand layout the P.V product needs, so P never
//     leaves registers.  Online softmax in base 2, fp32, with a lazily moved
//     reference max; the row sums of P are products with a ones operand;
//     tiles past every row of a wave are skipped.
//   * Keys past the causal limit, tail slots and out-of-range block ids are
//     masked and never multiply a value: masked K/V tile rows are zero-filled.
#include "prefill_dev.h"

namespace pa {

namespace {

using namespace pre;

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(const int32_t* __restrict__ cu,
                                                                    const int32_t* __restrict__ lens, int B,
                                                                    int cap, int TQ, int num_q_tokens,
                                                                    int item_cap, uint32_t* hdr,
                                                                    int2* __restrict__ items) {
  __shared__ int hist[kBuckets];
  __shared__ int wave_tot[kPlanThreads / 64];
  const int tid = threadIdx.x;
  for (int i = tid; i < kBuckets; i += kPlanThreads) hist[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kPlanThreads) {
    const int T = cu[b + 1] - cu[b];
    const int L = clamp_len(lens[b], cap);
    if (!chunk_ok(cu, b, T, L, num_q_tokens)) continue;
    const int bucket = min(chunk_work(T, L, TQ) / 4, kBuckets - 1);
    atomicAdd(&hist[bucket], (T + TQ - 1) / TQ);
  }
  __syncthreads();
  // descending bucket order: thread t owns bucket kBuckets - 1 - t
  static_assert(kBuckets == kPlanThreads, "one bucket per thread");
  const int mine = hist[kBuckets - 1 - tid];
  const int off = block_excl_scan(mine, wave_tot);
  hist[kBuckets - 1 - tid] = off;
  if (tid == kPlanThreads - 1) hdr[kEntryCountWord] = (uint32_t)min(off + mine, item_cap);
  if (tid < kXcds) hdr[tid * kCounterStride] = 0u;
  __syncthreads();
  for (int b = tid; b < B; b += kPlanThreads) {
    const int T = cu[b + 1] - cu[b];
    const int L = clamp_len(lens[b], cap);
    if (!chunk_ok(cu, b, T, L, num_q_tokens)) continue;
    const int nq = (T + TQ - 1) / TQ;
    const int bucket = min(chunk_work(T, L, TQ) / 4, kBuckets - 1);
    const int at = atomicAdd(&hist[bucket], nq);
    for (int j = 0; j < nq; ++j)
      if (at + j < item_cap) items[at + j] = make_int2(b, nq - 1 - j);
  }
}

// ---------------------------------------------------------------------------
// Prefill kernel: one persistent workgroup of 8 waves per CU pulls items.
// An item is (request, tile of TQ chunk tokens, KV head) with 256 rows
// (TQ tokens x G query heads, head-major); wave w owns rows 32w .. 32w+31.
// Key tiles of 64 go through two LDS buffers; the loads of the next two tiles
// are in flight while one tile computes, and the item's block ids sit in LDS
// so no gather address waits on a global load.
// ---------------------------------------------------------------------------
template <int D, bool kWide, bool kF8>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  __shared__ PrefillLds<D> lds;
  __shared__ uint32_t s_item, s_head;
  const int tid = threadIdx.x;
  const uint32_t entries = p.hdr[kEntryCountWord];
  // With H_kv a multiple of 8, KV head h is worked on by the workgroups of
  // XCD h % 8 (blocks are dealt to the XCDs in turn), so the q tiles that
  // share a request's keys meet in one L2; a workgroup whose queue is empty
  // helps the other queues.  Otherwise one queue serves all.
  const bool affine = p.Hkv % kXcds == 0;
  const uint32_t nqueues = affine ? kXcds : 1;
  const uint32_t per_entry = affine ? (uint32_t)(p.Hkv / kXcds) : (uint32_t)p.Hkv;
  const uint32_t home = blockIdx.x % nqueues;
  uint32_t queue = 0;  // queues found empty so far (thread 0)

  for (;;) {
    __syncthreads();  // the previous item's LDS reads are done
    if (tid == 0) {
      uint32_t e = 0xffffffffu, h = 0;
      while (queue < nqueues) {
        const uint32_t x = (home + queue) % nqueues;
        const uint32_t c = atomicAdd(p.counter + x * kCounterStride, 1u);
        if (c / per_entry < entries) {
          e = c / per_entry;
          h = affine ? x + kXcds * (c % per_entry) : c % per_entry;
          break;
        }
        ++queue;
      }
      s_item = e;
      s_head = h;
    }
    __syncthreads();
    const uint32_t e = s_item;
    if (e == 0xffffffffu) break;
    const int2 it = p.items[e];
    prefill_item<D, kWide, kF8>(p, lds, it.x, it.y, (int)s_head);
  }
}

}  // namespace

size_t prefill_workspace_size(int num_seqs, int64_t num_q_tokens, int num_q_heads, int num_kv_heads) {
  const int G = num_q_heads / num_kv_heads;
  return kHeaderBytes + align256(sizeof(int2) * (size_t)max_prefill_items(num_seqs, num_q_tokens, G));
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  char* ws = static_cast<char*>(a.workspace);
  PrefillParams p;
  p.q = static_cast<const bf16_bits*>(a.q);
  p.kc = static_cast<const char*>(a.k_cache);
  p.vc = static_cast<const char*>(a.v_cache);
  p.cu = a.cu_seqlens;
  p.bt = a.block_table;
  p.lens = a.context_lens;
  p.out = static_cast<bf16_bits*>(a.out);
  p.hdr = reinterpret_cast<const uint32_t*>(ws);
  p.counter = reinterpret_cast<uint32_t*>(ws);
  p.items = reinterpret_cast<const int2*>(ws + kHeaderBytes);
  p.scale_log2 = a.scale * kLog2e;
  p.Hq = a.num_q_heads;
  p.Hkv = a.num_kv_heads;
  p.G = a.num_q_heads / a.num_kv_heads;
  p.TQ = tokens_per_tile(p.G);
  p.P = a.block_size;
  {
    uint32_t l = 0;
    while ((1ull << l) < (uint64_t)a.block_size) ++l;
    p.div_l = l;
    p.div_m = (uint32_t)((((uint64_t)1 << (32 + l)) + (uint64_t)a.block_size - 1) / (uint64_t)a.block_size -
                         ((uint64_t)1 << 32));
  }
  const bool f8 = a.kv_dtype == kFP8E4M3;
  p.row_bytes = (uint32_t)(a.num_kv_heads * a.head_dim * (f8 ? 1 : 2));
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.N = (int)a.num_blocks;
  p.M = a.max_blocks;
  p.cap = (int)((int64_t)a.max_blocks * a.block_size);

  const int64_t item_cap = max_prefill_items(a.num_seqs, a.num_q_tokens, p.G);
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.cu_seqlens, a.context_lens,
                     a.num_seqs, p.cap, p.TQ, (int)a.num_q_tokens, (int)item_cap,
                     reinterpret_cast<uint32_t*>(ws), reinterpret_cast<int2*>(ws + kHeaderBytes));
  const int64_t max_items = item_cap * p.Hkv;
  const int64_t cap = (int64_t)device_cu_count();  // one workgroup (8 waves, 136 KiB of LDS) per CU
  const unsigned blocks = (unsigned)(max_items < cap ? max_items : cap);
  // 32-bit pool offsets when one pool is under 4 GiB
  const bool wide = a.num_blocks * a.block_size * (int64_t)p.row_bytes >= ((int64_t)1 << 32);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
#define PA_PREFILL_LAUNCH(DD, W, F) \
  hipLaunchKernelGGL((prefill_kernel<DD, W, F>), dim3(blocks), dim3(kThreads), 0, stream, p)
  if (a.head_dim == 128) {
    if (f8) {
      if (wide) PA_PREFILL_LAUNCH(128, true, true);
      else PA_PREFILL_LAUNCH(128, false, true);
    } else {
      if (wide) PA_PREFILL_LAUNCH(128, true, false);
      else PA_PREFILL_LAUNCH(128, false, false);
    }
  } else {
    if (f8) {
      if (wide) PA_PREFILL_LAUNCH(64, true, true);
      else PA_PREFILL_LAUNCH(64, false, true);
    } else {
      if (wide) PA_PREFILL_LAUNCH(64, true, false);
      else PA_PREFILL_LAUNCH(64, false, false);
    }
  }
#undef PA_PREFILL_LAUNCH
  if (ev1) {
    const hipError_t e = hipEventRecord(ev1, stream);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace pa
