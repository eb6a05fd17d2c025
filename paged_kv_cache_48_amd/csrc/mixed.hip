// Mixed batches for gfx950: decode requests and prefill chunks of one step in
// a single persistent launch.
//
// What is computed (tiny-vllm-py, "KV Cache" and its note that a step may mix
// prefill and decode work, best served by a ragged representation; ember,
// "Deliberately out of scope" for the prefill/decode mix per step): the same
// as the varlen prefill call on the same ragged batch.  Row i of request b's
// chunk of T_b = cu[b+1] - cu[b] tokens sits at absolute position
// L_b - T_b + i and attends causally to keys 0 .. L_b - T_b + i of its KV
// head; a request with T_b = 1 is a decode step over all L_b keys.
//
// Design (MI355X):
//   * One persistent workgroup of 8 waves per CU.  Every workgroup first
//     derives two work lists in LDS from cu_seqlens and the lengths (no plan
//     kernel): the prefill items of the multi-token chunks, largest first,
//     and the split-context partition items of the one-token chunks.
//   * Phase 1: the workgroup pulls prefill items (request, q tile, KV head)
//     from per-XCD queues and computes each with all 8 waves, exactly as the
//     prefill kernel does.
//   * Phase 2: once the prefill queues are empty, its 8 waves turn into
//     independent decode workers and pull partition items, exactly as the
//     decode kernel's waves do.  The short decode items fill the tail that
//     the long prefill items leave, and the decode reads overlap the prefill
//     products still running on other CUs.
//   * Each workgroup's LDS holds the prefill tile buffers, which the decode
//     waves reuse as their private tile regions in phase 2, and both plans.
//   * Queue counters carry a per-launch tag (as in the decode kernel), so the
//     workspace needs no clearing and the call is safe to replay.
//   * Partitions of decode requests with more than one are merged by the
//     decode reduce kernel, restricted to the one-token chunks.  Merging in
//     the same launch would need every partial to be written back from its
//     XCD's L2 before another XCD reads it.
#include "decode_dev.h"
#include "prefill_dev.h"

namespace pa {

namespace {

constexpr int kMixThreads = pre::kThreads;  // 8 waves
constexpr int kMixWaves = kMixThreads / 64;
constexpr int kMixMaxSeqs = dec::kSelfPlanMax;  // requests one launch plans in LDS
constexpr int kClasses = 16;                   // size classes of the prefill list
constexpr int kMixHeaderBytes = 1024;          // prefill queue counters, ahead of the decode workspace

// ---------------------------------------------------------------------------
// Prefill list, derived by every workgroup in LDS.  Chunks of two or more
// tokens are ordered by a size class of their total key tiles (classes a
// factor of about sqrt(2) apart, largest first; requests in increasing order
// within a class), and each request's q tiles run from the last (largest
// causal extent) to the first.  The list depends on the metadata alone, so
// all workgroups agree on it.  Entry e is q tile nq_b - 1 - (e - start[k]) of
// request req[k], for start[k] <= e < start[k + 1].
// ---------------------------------------------------------------------------
struct PrePlanLds {
  int start[kMixMaxSeqs + 1];
  uint16_t req[kMixMaxSeqs];
  uint16_t key[kMixMaxSeqs];  // size class | rank among the chunk's requests of that class << 5
  int pre[dec::kPlanChunks][kClasses + 1];
  int bstart[kClasses + 1];
  int n;                      // requests in the list
};

// Size class (1 .. 16) of a chunk with `work` key tiles; 0: no prefill items.
__device__ __forceinline__ int size_class(int work) {
  const int e = 31 - __clz(work);
  const int half = e >= 1 ? (work >> (e - 1)) & 1 : 0;
  const int c = 2 * e + half - 8;
  return 1 + (c < 0 ? 0 : (c > kClasses - 1 ? kClasses - 1 : c));
}

__device__ __forceinline__ bool is_prefill_chunk(const pre::PrefillParams& p, int b, int num_q_tokens, int& T,
                                                 int& L) {
  T = p.cu[b + 1] - p.cu[b];
  L = pre::clamp_len(p.lens[b], p.cap);
  return T >= 2 && pre::chunk_ok(p.cu, b, T, L, num_q_tokens);
}

// Every thread of the workgroup takes part (four barriers).
__device__ void prefill_self_plan(const pre::PrefillParams& p, int B, int num_q_tokens, PrePlanLds* pl) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nc = (B + 63) >> 6;
  // 1: per chunk of 64 requests: size classes, each request's rank among the
  // chunk's requests of its class (8-bit fields of four words, one prefix sum
  // per word), and the chunk's count of each class
  for (int c = wave; c < nc; c += kMixWaves) {
    const int b = 64 * c + lane;
    int bk = 0;
    if (b < B) {
      int T, L;
      if (is_prefill_chunk(p, b, num_q_tokens, T, L)) bk = size_class(pre::chunk_work(T, L, p.TQ));
    }
    const int kb = bk - 1;
    int sc[4], tw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc[w] = dec::wave_incl_scan(bk != 0 && (kb >> 2) == w ? 1 << (8 * (kb & 3)) : 0);
      tw[w] = __builtin_amdgcn_readlane(sc[w], 63);
    }
    const int mine = kb < 4 ? sc[0] : kb < 8 ? sc[1] : kb < 12 ? sc[2] : sc[3];
    const int rank = bk ? ((mine >> (8 * (kb & 3))) & 255) - 1 : 0;
    const int lk = lane - 1;  // lane k (1 .. 16) takes the count of class k
    const int word = lk < 4 ? tw[0] : lk < 8 ? tw[1] : lk < 12 ? tw[2] : tw[3];
    const int cnt = lane == 0 ? 0 : (word >> (8 * (lk & 3))) & 255;
    if (b < B) pl->key[b] = (uint16_t)(bk | rank << 5);
    if (lane <= kClasses) pl->pre[c][lane] = cnt;
  }
  __syncthreads();
  // 2: exclusive prefixes over the chunks and the first list position of
  // each class (class 16 first)
  if (wave == 0) {
    int tot[kClasses + 1];
#pragma unroll
    for (int k = 1; k <= kClasses; ++k) {
      const int v = lane < nc ? pl->pre[lane][k] : 0;
      const int incl = dec::row16_incl_scan(v);
      if (lane < nc) pl->pre[lane][k] = incl - v;
      tot[k] = __builtin_amdgcn_readlane(incl, dec::kPlanChunks - 1);
    }
    if (lane == 0) {
      int run = 0;
#pragma unroll
      for (int k = kClasses; k >= 1; --k) {
        pl->bstart[k] = run;
        run += tot[k];
      }
      pl->n = run;
    }
  }
  __syncthreads();
  // 3: list positions; start[] holds each listed request's q-tile count
  for (int c = wave; c < nc; c += kMixWaves) {
    const int b = 64 * c + lane;
    if (b < B) {
      const int key = pl->key[b];
      const int bk = key & 31;
      if (bk) {
        const int pos = pl->bstart[bk] + pl->pre[c][bk] + (key >> 5);
        pl->req[pos] = (uint16_t)b;
        pl->start[pos] = (p.cu[b + 1] - p.cu[b] + p.TQ - 1) / p.TQ;
      }
    }
  }
  __syncthreads();
  // 4: exclusive prefix sum of the q-tile counts (one wave, 64 at a time)
  if (wave == 0) {
    const int n = pl->n;
    int carry = 0;
    for (int k0 = 0; k0 < n; k0 += 64) {
      const int k = k0 + lane;
      const int v = k < n ? pl->start[k] : 0;
      const int incl = dec::wave_incl_scan(v);
      if (k < n) pl->start[k] = carry + incl - v;
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) pl->start[n] = carry;
  }
  __syncthreads();
}

// (request, q tile) of prefill list entry e.
__device__ __forceinline__ int2 prefill_entry(const PrePlanLds* pl, int e) {
  int lo = 0, hi = pl->n;  // start[lo] <= e < start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pl->start[mid] <= e) lo = mid;
    else hi = mid;
  }
  const int nq = pl->start[lo + 1] - pl->start[lo];
  return make_int2(pl->req[lo], nq - 1 - (e - pl->start[lo]));
}

struct MixedParams {
  dec::DecodeParams d;
  pre::PrefillParams p;
  unsigned long long* pcounter;  // prefill queue counters (tagged, like the decode ones)
  int B;
  int num_q_tokens;
};

// LDS of a mixed workgroup: the prefill tile buffers, reused as the decode
// waves' tile regions, then the two plans.
template <typename T, int D>
struct MixLds {
  static constexpr size_t kPre = sizeof(pre::PrefillLds<D>);
  static constexpr size_t kDec = (size_t)dec::Geo<T, D>::LDS_PER_WAVE * kMixWaves;
  static constexpr size_t kTiles = ((kPre > kDec ? kPre : kDec) + 15) & ~(size_t)15;
  static constexpr size_t kDecPlan = kTiles;
  static constexpr size_t kPrePlan = kDecPlan + ((sizeof(dec::PlanLds) + 15) & ~(size_t)15);
  static constexpr size_t kBytes = kPrePlan + sizeof(PrePlanLds);
};

template <typename T, int D, bool kWide, bool kAligned, int NR>
__global__ __launch_bounds__(kMixThreads) void mixed_kernel(MixedParams mp) {
  using LY = MixLds<T, D>;
  constexpr bool kF8 = dec::Geo<T, D>::kFp8;
  __shared__ __attribute__((aligned(16))) char smem[LY::kBytes];
  __shared__ uint32_t s_item, s_head;
  pre::PrefillLds<D>& plds = *reinterpret_cast<pre::PrefillLds<D>*>(smem);
  dec::PlanLds* dpl = reinterpret_cast<dec::PlanLds*>(smem + LY::kDecPlan);
  PrePlanLds* ppl = reinterpret_cast<PrePlanLds*>(smem + LY::kPrePlan);
  const int tid = threadIdx.x;
  const unsigned long long tag = dec::launch_tag(mp.d.salt);
  // workgroup 0 resets both sets of queue counters for this launch
  if (blockIdx.x == 0 && tid < 2 * dec::kQueues) {
    unsigned long long* c = tid < dec::kQueues ? mp.d.counter + tid * dec::kCounterStride
                                               : mp.pcounter + (tid - dec::kQueues) * dec::kCounterStride;
    atomicExch(c, tag << dec::kCountBits);
  }
  dec::self_plan<true>(mp.d, dpl, pre::kThreads / 64);
  prefill_self_plan(mp.p, mp.B, mp.num_q_tokens, ppl);

  // ---- phase 1: prefill items, one per workgroup at a time ----
  const uint32_t entries = (uint32_t)ppl->start[ppl->n];
  const int Hkv = mp.p.Hkv;
  const bool affine = Hkv % dec::kQueues == 0;
  const uint32_t nqueues = affine ? dec::kQueues : 1;
  const uint32_t per_entry = affine ? (uint32_t)(Hkv / dec::kQueues) : (uint32_t)Hkv;
  const uint32_t home = blockIdx.x % nqueues;
  uint32_t queue = 0;  // queues found empty so far (thread 0)
  int spins = 0;
  for (;;) {
    if (tid == 0) {
      uint32_t e = 0xffffffffu, h = 0;
      while (queue < nqueues) {
        const uint32_t x = (home + queue) % nqueues;
        const unsigned long long old = atomicAdd(mp.pcounter + x * dec::kCounterStride, 1ull);
        if (mp.d.force_giveup || (old >> dec::kCountBits) != tag) {  // not yet reset for this launch
          if (!mp.d.force_giveup && ++spins < dec::kMaxSpins) {
            __builtin_amdgcn_s_sleep(8);
          } else {
            ++queue;
            atomicOr(mp.d.status, dec::kGaveUpPrefill);
          }
          continue;
        }
        const uint32_t c = (uint32_t)(old & (dec::kMaxQueueItems - 1));
        if (c / per_entry < entries) {
          e = c / per_entry;
          h = affine ? x + dec::kQueues * (c % per_entry) : c % per_entry;
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
    const int2 it = prefill_entry(ppl, (int)e);
    if (it.x < mp.B && it.y >= 0)  // always, for a list built as above; a guard against reading past the batch
      pre::prefill_item<D, kWide, kF8>(mp.p, plds, it.x, it.y, (int)s_head);
    __syncthreads();  // the item's LDS reads are done before the next claim overwrites s_item
  }

  // ---- phase 2: the waves become independent decode workers ----
  const uint32_t n_items = (uint32_t)uniform(dpl->nitems);
  const uint32_t n_full = (uint32_t)uniform(dpl->nfull);
  const uint32_t nq_plan = (uint32_t)uniform(dpl->nq);
  const uint32_t w = (uint32_t)uniform(tid >> 6);
  char* lds = smem + w * dec::Geo<T, D>::LDS_PER_WAVE;
  dec::decode_stream<T, D, kWide, kAligned, NR, true>(mp.d, lds, dpl, tag, n_items, n_full, nq_plan,
                                                      blockIdx.x * kMixWaves + w, gridDim.x * kMixWaves, 0u);
}

template <typename T, int D, bool kWide, bool kAligned, int NR>
hipError_t launch_mixed_typed(const MixedParams& mp, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  static_assert(MixLds<T, D>::kBytes + 16 <= 160 * 1024, "mixed workgroup LDS exceeds a CU's 160 KiB");
  const unsigned blocks = (unsigned)device_cu_count();  // one workgroup (8 waves) per CU
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((mixed_kernel<T, D, kWide, kAligned, NR>), dim3(blocks), dim3(kMixThreads), 0, stream, mp);
  if (ev1) {
    const hipError_t e = hipEventRecord(ev1, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dec::decode_reduce_kernel<bf16_bits, D, true>), dim3((mp.d.Hq + 3) / 4, mp.B), dim3(256), 0,
                     stream, mp.d);
  return hipGetLastError();
}

template <typename T, int D, bool kWide>
hipError_t launch_mixed_mode(const MixedParams& mp, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (mp.d.P % dec::kTile == 0) return launch_mixed_typed<T, D, kWide, true, 1>(mp, stream, ev0, ev1);
  if (mp.d.P >= 5) return launch_mixed_typed<T, D, kWide, false, 1>(mp, stream, ev0, ev1);
  return launch_mixed_typed<T, D, kWide, false, 5>(mp, stream, ev0, ev1);
}

template <typename T, int D>
hipError_t launch_mixed_sized(const MixedParams& mp, bool wide, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (wide) return launch_mixed_mode<T, D, true>(mp, stream, ev0, ev1);
  return launch_mixed_mode<T, D, false>(mp, stream, ev0, ev1);
}

}  // namespace

size_t mixed_workspace_size(int num_seqs, int num_q_heads, int head_dim, int block_size, int max_blocks) {
  return kMixHeaderBytes + dec::decode_layout(num_seqs, num_q_heads, head_dim, block_size, max_blocks).total;
}

int mixed_max_seqs() { return kMixMaxSeqs; }

bool mixed_fits(int num_seqs, int64_t num_q_tokens, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                int max_blocks) {
  if (num_seqs > kMixMaxSeqs) return false;
  const int G = num_q_heads / num_kv_heads;
  const dec::DecodeLayout Lw = dec::decode_layout(num_seqs, num_q_heads, head_dim, block_size, max_blocks);
  // claims per tagged counter (24-bit count): items, plus one failed claim per wave
  dec::DecodeParams groups;
  dec::set_query_groups(groups, G, 1);
  const int64_t dec_items = (int64_t)num_seqs * Lw.max_parts * num_kv_heads * groups.n_hg;
  const int64_t pre_items = pre::max_prefill_items(num_seqs, num_q_tokens, G) * num_kv_heads;
  return dec_items + dec::kMaxWaves < dec::kMaxQueueItems && pre_items + dec::kMaxWaves < dec::kMaxQueueItems;
}

hipError_t launch_mixed(const AttnArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  char* ws = static_cast<char*>(a.workspace);
  const dec::DecodeLayout Lw = dec::decode_layout(a.num_seqs, a.num_q_heads, a.head_dim, a.block_size, a.max_blocks);
  char* dws = ws + kMixHeaderBytes;
  const bool f8 = a.kv_dtype == kFP8E4M3;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int cap = (int)((int64_t)a.max_blocks * a.block_size);
  MixedParams mp;
  mp.B = a.num_seqs;
  mp.num_q_tokens = (int)a.num_q_tokens;
  mp.pcounter = reinterpret_cast<unsigned long long*>(ws);

  dec::DecodeParams& d = mp.d;
  d.q = a.q;
  d.kc = a.k_cache;
  d.vc = a.v_cache;
  d.bt = a.block_table;
  d.lens = a.context_lens;
  d.out = a.out;
  d.hdr = reinterpret_cast<const uint32_t*>(dws + Lw.hdr);
  d.counter = reinterpret_cast<unsigned long long*>(dws + Lw.hdr);
  d.items = nullptr;  // always planned in LDS
  d.ml = reinterpret_cast<float*>(dws + Lw.ml);
  d.o = reinterpret_cast<float*>(dws + Lw.o);
  d.scale_log2 = a.scale * kLog2e;
  d.Hq = a.num_q_heads;
  d.Hkv = a.num_kv_heads;
  dec::set_query_groups(d, G, 1);
  d.P = a.block_size;
  d.p_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz((unsigned)a.block_size) : -1;
  d.N = (int)a.num_blocks;
  d.M = a.max_blocks;
  d.cap = cap;
  d.max_parts = (int)Lw.max_parts;
  d.dyn_rounds = 0;
  d.nq = 0;
  d.B = a.num_seqs;
  d.k_scale = f8 ? a.k_scale : nullptr;
  d.v_scale = f8 ? a.v_scale : nullptr;
  d.self_plan = 1;
  d.salt = dec::next_salt();
  d.cu = a.cu_seqlens;
  d.num_q_tokens = (int)a.num_q_tokens;
  d.knew = nullptr;
  d.vnew = nullptr;
  d.new_f32 = 0;
  // both kinds of give-up go to the status word of the mixed header (at the
  // same offset as in a decode workspace)
  d.status = reinterpret_cast<uint32_t*>(ws) + dec::kStatusWord;
  d.force_giveup = dec::test_queue_giveup();

  pre::PrefillParams& p = mp.p;
  p.q = static_cast<const bf16_bits*>(a.q);
  p.kc = static_cast<const char*>(a.k_cache);
  p.vc = static_cast<const char*>(a.v_cache);
  p.cu = a.cu_seqlens;
  p.bt = a.block_table;
  p.lens = a.context_lens;
  p.out = static_cast<bf16_bits*>(a.out);
  p.hdr = nullptr;
  p.counter = nullptr;
  p.items = nullptr;
  p.scale_log2 = a.scale * kLog2e;
  p.Hq = a.num_q_heads;
  p.Hkv = a.num_kv_heads;
  p.G = G;
  p.TQ = pre::tokens_per_tile(G);
  p.P = a.block_size;
  {
    uint32_t l = 0;
    while ((1ull << l) < (uint64_t)a.block_size) ++l;
    p.div_l = l;
    p.div_m = (uint32_t)((((uint64_t)1 << (32 + l)) + (uint64_t)a.block_size - 1) / (uint64_t)a.block_size -
                         ((uint64_t)1 << 32));
  }
  p.row_bytes = (uint32_t)(a.num_kv_heads * a.head_dim * (f8 ? 1 : 2));
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.N = (int)a.num_blocks;
  p.M = a.max_blocks;
  p.cap = cap;

  const bool wide = a.num_blocks * a.block_size * (int64_t)p.row_bytes >= ((int64_t)1 << 32);
  if (f8) {
    if (a.head_dim == 128) return launch_mixed_sized<dec::fp8_e4m3, 128>(mp, wide, stream, ev0, ev1);
    return launch_mixed_sized<dec::fp8_e4m3, 64>(mp, wide, stream, ev0, ev1);
  }
  if (a.head_dim == 128) return launch_mixed_sized<bf16_bits, 128>(mp, wide, stream, ev0, ev1);
  return launch_mixed_sized<bf16_bits, 64>(mp, wide, stream, ev0, ev1);
}

}  // namespace pa
