// Paged decode attention for gfx950: one new query token per request attends to
// its request's cached keys/values, gathered through the block table.
//
// What is computed (tiny-vllm-py, "KV Cache"; weft, "Shapes and symbols"):
//   out[b, h] = sum_j softmax_j(scale * q[b, h] . k_j) v_j  over j < L_b,
// with k_j, v_j taken from KV head h / G of the paged pool [N, P, H_kv, D] at
// block block_table[b][j / P], offset j % P (ember, "The core idea").
//
// Design (MI355X):
//   * Split context.  Each request is cut into partitions of kPartTokens tokens
//     (a count that depends on L_b only).  A (request, partition, KV head, group
//     of up to 16 query heads) is one work item; a single wave64 computes it.
//   * Work queue.  The (request, partition) items are listed full partitions
//     first and short tail partitions last: for batches of up to
//     kSelfPlanMax requests every workgroup derives the list itself in LDS
//     from the lengths, otherwise a tiny plan kernel writes it.  A persistent
//     grid of exactly the resident waves takes one item each to start, then
//     pulls items with one atomic each from per-XCD queues, stealing from the
//     other queues at the end.
//   * Coalesced gathers.  Per tile (16 tokens; 32 for fp8 pools) groups of
//     lanes read whole contiguous row slices of one KV head (16-byte loads);
//     the tile goes through a wave-private LDS region, K row-major and V
//     transposed (bf16) or row-major (fp32, and fp8 codes, read back with
//     the byte-transposing LDS read), which turns it into MFMA operands.  The
//     next tile's loads are in flight while the current one computes.
//   * S^T = K Q^T and O^T += V^T P^T run on MFMA (bf16: 16x16x32 and
//     16x16x16; fp8 via fp16: 16x16x32; fp32: 16x16x4) with fp32
//     accumulation.  The group's query
//     heads are the B-operand columns, so each lane holds one head's scores
//     for four tokens, which is exactly the B operand of the P.V product: the
//     probabilities never leave registers and the outputs need no cross-lane
//     reduction.  Online softmax in base 2 (running max and sum).
//   * Items of a request with one partition write the output directly; the
//     others write (max, sum, output) partials that the reduce kernel merges:
//     m = max_i m_i,  out = sum_i 2^(m_i-m) o_i / sum_i 2^(m_i-m) l_i, where o_i
//     is unnormalised (fp32 requests) or stored as l_i * r_i * (o_i / l_i / r_i)
//     with the last factor in fp16 and r_i a power of two that keeps it in
//     range (bf16 requests: half the partial bytes, whose writes interleaved
//     with the KV reads are costly).
//   * Tokens past the partition end never load: tail slots of a block may hold
//     anything (even NaN).  Block ids outside [0, N) are never dereferenced
//     (their rows read as zeros, so the result is unspecified but safe).
#include "decode_dev.h"

namespace pa {

namespace {

using namespace dec;

// ---------------------------------------------------------------------------
// Plan: lists the (request, partition) items in decreasing size -- every full
// partition first, then the tail partitions grouped by their tile count
// (16 .. 1) -- so the last items handed out are the smallest.  Each item
// carries (request, partition, clamped length, partition count).  One block:
// the bucket sizes are counted with LDS atomics, turned into bucket offsets,
// and each request then takes its positions with a second round of LDS
// atomics (the order inside a bucket is arbitrary; results do not depend on
// which wave computes an item).  It also zeroes the queue counters and picks
// one queue when items are long enough for a single counter to keep up.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const int32_t* __restrict__ lens, int B,
                                                                   int cap, uint32_t* hdr,
                                                                   i32x4_t* __restrict__ items) {
  __shared__ int cnt[kTileBuckets + 1];
  __shared__ int cur[kTileBuckets + 1];
  __shared__ unsigned long long tiles;
  const int tid = threadIdx.x;
  if (tid <= kTileBuckets) cnt[tid] = 0;
  if (tid == 0) tiles = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kPlanThreads) {
    const int L = clamp_len(lens[b], cap);
    const int full = L / kPartTokens, rest = L % kPartTokens;
    if (full) atomicAdd(&cnt[0], full);
    if (rest) atomicAdd(&cnt[(rest + 15) / 16], 1);
    if (L) atomicAdd(&tiles, (unsigned long long)((L + 15) / 16));
  }
  __syncthreads();
  if (tid == 0) {
    int run = cnt[0];
    cur[0] = 0;
    for (int k = kTileBuckets; k >= 1; --k) {
      cur[k] = run;
      run += cnt[k];
    }
    hdr[kItemCountWord] = (uint32_t)run;
    hdr[kFullCountWord] = (uint32_t)cnt[0];
    hdr[kQueueCountWord] = tiles >= 4ull * (unsigned long long)run ? 1u : (uint32_t)kQueues;
  }
  if (tid < kQueues) reinterpret_cast<unsigned long long*>(hdr)[tid * kCounterStride] = 0ull;
  __syncthreads();
  for (int b = tid; b < B; b += kPlanThreads) {
    const int L = clamp_len(lens[b], cap);
    const int full = L / kPartTokens, rest = L % kPartTokens;
    const int np = full + (rest ? 1 : 0);
    if (full) {
      const int at = atomicAdd(&cur[0], full);
      for (int j = 0; j < full; ++j) items[at + j] = i32x4_t{b, j, L, np};
    }
    if (rest) items[atomicAdd(&cur[(rest + 15) / 16], 1)] = i32x4_t{b, full, L, np};
  }
}

// ---------------------------------------------------------------------------
// Partition kernel: every wave computes a stream of work items (see
// decode_stream for the schedule and the per-tile steps).
// ---------------------------------------------------------------------------
// Waves per workgroup: as many as fit in 64 KiB of LDS (at most 4).
template <typename T, int D>
constexpr int waves_per_block() {
  return Geo<T, D>::LDS_PER_WAVE * kWavesPerBlock <= 65536 ? kWavesPerBlock : 2;
}

template <typename T, int D, bool kWide, bool kAligned, int NR, int HP, bool kAppend, bool kTwo>
__device__ __forceinline__ void partition_body(const DecodeParams& prm) {
  using Gm = Geo<T, D>;
  constexpr int wpb = waves_per_block<T, D>();
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* lds = smem + (threadIdx.x >> 6) * Gm::LDS_PER_WAVE;
  PlanLds* pl = reinterpret_cast<PlanLds*>(smem + wpb * Gm::LDS_PER_WAVE);
  unsigned long long tag = 0;
  uint32_t n_items, n_full, nq_plan;
  if (prm.self_plan) {
    tag = launch_tag(prm.salt);
    // workgroup 0 resets the queue counters for this launch
    if (blockIdx.x == 0 && threadIdx.x < kQueues)
      atomicExch(prm.counter + threadIdx.x * kCounterStride, tag << kCountBits);
    self_plan<false>(prm, pl, wpb);
    n_items = (uint32_t)uniform(pl->nitems);
    n_full = (uint32_t)uniform(pl->nfull);
    nq_plan = (uint32_t)uniform(pl->nq);
  } else {
    n_items = prm.hdr[kItemCountWord];
    n_full = prm.hdr[kFullCountWord];
    nq_plan = prm.hdr[kQueueCountWord];
  }
  const uint32_t nwaves = gridDim.x * wpb;
  // (threadIdx.x >> 6 is the same in every lane; readfirstlane tells the compiler)
  const uint32_t wave = blockIdx.x * wpb + (uint32_t)uniform((int)(threadIdx.x >> 6));
  // kTwo (bf16 pools, small batches): two tiles in flight per wave (the same
  // items and arithmetic, so the same bits as one)
  if constexpr (kTwo)
    decode_stream2<T, D, kWide, kAligned, NR, HP, kAppend>(prm, lds, pl, tag, n_items, n_full, nq_plan, wave,
                                                           nwaves, (uint32_t)kMaxStaticRounds);
  else
    decode_stream<T, D, kWide, kAligned, NR, false, HP, kAppend>(prm, lds, pl, tag, n_items, n_full, nq_plan, wave,
                                                               nwaves, (uint32_t)kMaxStaticRounds);
}

template <typename T, int D, bool kWide, bool kAligned, int NR, int HP, bool kAppend>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeParams prm) {
  partition_body<T, D, kWide, kAligned, NR, HP, kAppend, false>(prm);
}

// fp8 pools with append: making the new token's codes would take the kernel
// just past 168 VGPRs (three waves per SIMD to two), or for 128-dim heads read
// in pairs just past 256 (two to one); it is held to kWaves waves per SIMD.
// bf16 pools with two tiles in flight are held to two.
template <typename T, int D, bool kWide, bool kAligned, int NR, int HP, bool kAppend, int kWaves, bool kTwo = false>
__global__ __launch_bounds__(256, kWaves) void decode_partition_kernel_wb(DecodeParams prm) {
  partition_body<T, D, kWide, kAligned, NR, HP, kAppend, kTwo>(prm);
}

template <typename T, int D, bool kWide, bool kAligned, int NR, int HP, bool kAppend, bool kTwo>
hipError_t launch_typed(const DecodeParams& prm, int B, int64_t max_items, hipStream_t stream,
                        hipEvent_t ev0, hipEvent_t ev1) {
  // waves are independent workers
  constexpr int wpb = waves_per_block<T, D>();
  // per-wave tile buffers, then the in-kernel plan
  constexpr unsigned lds_bytes = Geo<T, D>::LDS_PER_WAVE * wpb + (unsigned)sizeof(PlanLds);
  // exactly the blocks that can be resident at once: every wave starts on its
  // first item immediately, and none waits for a slot while holding one
  // two tiles in flight (two register sets): held to two waves per SIMD,
  // where the compiler would otherwise go just past 256 registers
  constexpr bool kWb = (kAppend && Geo<T, D>::kFp8) || kTwo;
  constexpr int kWaves = kTwo ? 2 : (D <= 128 ? 3 : 2);
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    hipError_t e;
    if constexpr (kWb)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &nb, decode_partition_kernel_wb<T, D, kWide, kAligned, NR, HP, kAppend, kWaves, kTwo>, 64 * wpb, lds_bytes);
    else
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &nb, decode_partition_kernel<T, D, kWide, kAligned, NR, HP, kAppend>, 64 * wpb, lds_bytes);
    per_cu = e != hipSuccess || nb < 1 ? 1 : nb;
  }
  const int64_t want = (max_items + wpb - 1) / wpb;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  const unsigned blocks = (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
  if constexpr (kWb)
    hipLaunchKernelGGL((decode_partition_kernel_wb<T, D, kWide, kAligned, NR, HP, kAppend, kWaves, kTwo>), dim3(blocks),
                       dim3(64 * wpb), lds_bytes, stream, prm);
  else
    hipLaunchKernelGGL((decode_partition_kernel<T, D, kWide, kAligned, NR, HP, kAppend>), dim3(blocks),
                       dim3(64 * wpb), lds_bytes, stream, prm);
  if (ev1) {
    const hipError_t e = hipEventRecord(ev1, stream);
    if (e != hipSuccess) return e;
  }
  // partial rows are the real heads' (D / HP elements)
  hipLaunchKernelGGL((decode_reduce_kernel<typename QType<T>::type, D / HP, false>), dim3((prm.Hq + 3) / 4, B),
                     dim3(256), 0, stream, prm);
  return hipGetLastError();
}

template <typename T, int D, bool kWide, int HP, bool kAppend, bool kTwo>
hipError_t launch_mode(const DecodeParams& prm, int B, int64_t max_items, hipStream_t stream, hipEvent_t ev0,
                       hipEvent_t ev1) {
  // tiles of 16 tokens never straddle a block when P is a multiple of 16; a
  // partition touches at most 256 / P + 1 blocks: one id register for P >= 5
  if (prm.P % kTile == 0)
    return launch_typed<T, D, kWide, true, 1, HP, kAppend, kTwo>(prm, B, max_items, stream, ev0, ev1);
  if (prm.P >= 5) return launch_typed<T, D, kWide, false, 1, HP, kAppend, kTwo>(prm, B, max_items, stream, ev0, ev1);
  return launch_typed<T, D, kWide, false, 5, HP, kAppend, kTwo>(prm, B, max_items, stream, ev0, ev1);
}

// bf16 pools: batches of at most this many work items (upper bound from the
// shapes: requests x partitions of the longest context x KV heads x head
// groups) run with two tiles in flight per wave.  Their waves have few items
// each, and a wave with one tile in flight waits a memory latency per tile;
// larger batches keep more waves resident with one tile each, which measured
// faster on them.  Both compute the same bits.
constexpr int64_t kTwoTileMaxItems = 8192;

template <typename T, int D, int HP, bool kAppend>
hipError_t launch_sized(const DecodeParams& prm, int B, int64_t max_items, int64_t pool_bytes,
                        hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const bool wide = pool_bytes >= ((int64_t)1 << 32);
  if constexpr (std::is_same<T, bf16_bits>::value) {
    if (max_items <= kTwoTileMaxItems)
      return wide ? launch_mode<T, D, true, HP, kAppend, true>(prm, B, max_items, stream, ev0, ev1)
                  : launch_mode<T, D, false, HP, kAppend, true>(prm, B, max_items, stream, ev0, ev1);
  }
  return wide ? launch_mode<T, D, true, HP, kAppend, false>(prm, B, max_items, stream, ev0, ev1)
              : launch_mode<T, D, false, HP, kAppend, false>(prm, B, max_items, stream, ev0, ev1);
}

// Kernel choice by pool element type, head size and head pairing.
template <bool kAppend>
hipError_t launch_kinds(const AttnArgs& a, const DecodeParams& prm, bool fp8, bool pairs, int64_t max_items,
                        int64_t pool_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int B = a.num_seqs;
  if (fp8) {  // bf16 q and out
    if (a.head_dim == 128 && pairs)
      return launch_sized<fp8_e4m3, 256, 2, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
    if (a.head_dim == 128)
      return launch_sized<fp8_e4m3, 128, 1, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
    if (pairs) return launch_sized<fp8_e4m3, 128, 2, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
    return launch_sized<fp8_e4m3, 64, 1, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
  }
  if (a.dtype == kBF16) {
    if (a.head_dim == 128)
      return launch_sized<bf16_bits, 128, 1, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
    if (pairs) return launch_sized<bf16_bits, 128, 2, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
    return launch_sized<bf16_bits, 64, 1, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
  }
  if (a.head_dim == 128) return launch_sized<float, 128, 1, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
  return launch_sized<float, 64, 1, kAppend>(prm, B, max_items, pool_bytes, stream, ev0, ev1);
}

}  // namespace

size_t decode_workspace_size(int num_seqs, int num_q_heads, int head_dim, int block_size,
                             int max_blocks) {
  return decode_layout(num_seqs, num_q_heads, head_dim, block_size, max_blocks).total;
}

hipError_t launch_decode(const AttnArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const DecodeLayout Lw = decode_layout(a.num_seqs, a.num_q_heads, a.head_dim, a.block_size, a.max_blocks);
  char* ws = static_cast<char*>(a.workspace);
  DecodeParams prm;
  prm.q = a.q;
  prm.kc = a.k_cache;
  prm.vc = a.v_cache;
  prm.bt = a.block_table;
  prm.lens = a.context_lens;
  prm.out = a.out;
  prm.hdr = reinterpret_cast<const uint32_t*>(ws + Lw.hdr);
  prm.counter = reinterpret_cast<unsigned long long*>(ws + Lw.hdr);
  prm.items = reinterpret_cast<const i32x4_t*>(ws + Lw.items);
  prm.ml = reinterpret_cast<float*>(ws + Lw.ml);
  prm.o = reinterpret_cast<float*>(ws + Lw.o);
  prm.scale_log2 = a.scale * kLog2e;
  prm.Hq = a.num_q_heads;
  const int G = a.num_q_heads / a.num_kv_heads;
  const bool fp8 = a.kv_dtype == kFP8E4M3;
  // bf16 pools with 64-dim heads and fp8 pools: adjacent KV heads are read in
  // pairs, as one head of twice the dimension (256-byte token rows, as the
  // bf16 128-dim kernel reads); each query column keeps its own head's half.
  // A pair's two groups share the 16 columns, so pairs are taken only while
  // the group fits in 8: beyond that, single heads read each slice once.
  const bool pairs = (fp8 || (a.dtype == kBF16 && a.head_dim == 64)) && a.num_kv_heads % 2 == 0 && G <= 8;
  prm.Hkv = pairs ? a.num_kv_heads / 2 : a.num_kv_heads;
  set_query_groups(prm, G, pairs ? 2 : 1);
  prm.P = a.block_size;
  prm.p_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz((unsigned)a.block_size) : -1;
  prm.N = (int)a.num_blocks;
  prm.M = a.max_blocks;
  prm.cap = (int)((int64_t)a.max_blocks * a.block_size);
  prm.max_parts = (int)Lw.max_parts;
  prm.dyn_rounds = kDynamicRounds;
  prm.nq = 0;
  prm.B = a.num_seqs;
  prm.salt = next_salt();
  prm.cu = nullptr;
  prm.num_q_tokens = 0;
  prm.knew = a.k_new;
  prm.vnew = a.v_new;
  prm.new_f32 = a.new_dtype == kF32;
  prm.k_scale = fp8 ? a.k_scale : nullptr;
  prm.v_scale = fp8 ? a.v_scale : nullptr;
  prm.status = reinterpret_cast<uint32_t*>(ws + Lw.hdr) + kStatusWord;
  prm.force_giveup = test_queue_giveup();

  const int64_t max_items = (int64_t)a.num_seqs * Lw.max_parts * prm.Hkv * prm.n_hg;
  // the workgroups plan small batches themselves (their counters then carry
  // a tag and a 24-bit count: items plus one failed claim per wave must fit)
  prm.self_plan = a.num_seqs <= kSelfPlanMax && max_items + kMaxWaves < kMaxQueueItems;
  if (!prm.self_plan)
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.context_lens, a.num_seqs,
                       prm.cap, reinterpret_cast<uint32_t*>(ws + Lw.hdr),
                       reinterpret_cast<i32x4_t*>(ws + Lw.items));
  const int64_t pool_bytes =
      a.num_blocks * a.block_size * a.num_kv_heads * a.head_dim * (fp8 ? 1 : (a.dtype == kBF16 ? 2 : 4));
  if (a.k_new) return launch_kinds<true>(a, prm, fp8, pairs, max_items, pool_bytes, stream, ev0, ev1);
  return launch_kinds<false>(a, prm, fp8, pairs, max_items, pool_bytes, stream, ev0, ev1);
}

}  // namespace pa
