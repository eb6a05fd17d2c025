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
//     of up to 4 query heads) is one work item; a single wave64 computes it.
//   * Work queue.  A tiny plan kernel lists the (request, partition) items,
//     full partitions first and short tail partitions last, and zeroes the
//     queue counters; a persistent grid of exactly the resident waves takes
//     one item each to start, then pulls items with one atomic each from
//     per-XCD queues, stealing from the other queues at the end.
//   * Coalesced gathers.  Per 16-token tile each quarter-wave reads whole
//     contiguous row slices of one KV head (16-byte loads); the tile goes
//     through a wave-private LDS region, K row-major and V transposed, which
//     turns it into MFMA operands.  The next tile's loads are in flight while
//     the current one computes.
//   * S^T = K Q^T and O^T += V^T P^T run on MFMA (bf16: 16x16x32 and
//     16x16x16; fp32: 16x16x4) with fp32 accumulation.  The group's query
//     heads are the B-operand columns, so each lane holds one head's scores
//     for four tokens, which is exactly the B operand of the P.V product: the
//     probabilities never leave registers and the outputs need no cross-lane
//     reduction.  Online softmax in base 2 (running max and sum).
//   * Items of a request with one partition write the output directly; the
//     others write (max, sum, unnormalised output) partials that the reduce
//     kernel merges:  m = max_i m_i,  out = sum_i 2^(m_i-m) o_i / sum_i 2^(m_i-m) l_i.
//   * Tokens past the partition end never load: tail slots of a block may hold
//     anything (even NaN).  Block ids outside [0, N) are never dereferenced
//     (their rows read as zeros, so the result is unspecified but safe).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kTile = 16;                        // tokens per MFMA tile
// logical blocks one partition can touch: kPartTokens / P + 1 for P >= 1
constexpr int kMaxPartBlocks = kPartTokens + 64;

constexpr int kWavesPerBlock = 4;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Work-queue header in the workspace: kQueues counters, each on its own
// 128-byte line, and the item count in the last word.
constexpr int kQueues = 8;  // one per XCD of the MI355X
constexpr int kCounterStride = 32;  // uint32 words between counters
constexpr int kHeaderBytes = 1024;
constexpr int kItemCountWord = kHeaderBytes / 4 - 1;

struct DecodeLayout {
  int64_t max_parts;
  size_t hdr, items, ml, o, total;
};

DecodeLayout decode_layout(int B, int Hq, int D, int P, int M) {
  DecodeLayout L;
  L.max_parts = ((int64_t)M * P + kPartTokens - 1) / kPartTokens;
  size_t off = 0;
  L.hdr = off;
  off += kHeaderBytes;
  L.items = off;
  off = align256(off + sizeof(int2) * (size_t)B * L.max_parts);
  L.ml = off;
  off = align256(off + sizeof(float) * 2 * (size_t)B * Hq * L.max_parts);
  L.o = off;
  off = align256(off + sizeof(float) * (size_t)B * Hq * L.max_parts * D);
  L.total = off;
  return L;
}

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// ---------------------------------------------------------------------------
// Plan: list (request, partition) items, full partitions first.
// ---------------------------------------------------------------------------
__device__ int block_excl_scan(int v, int* buf, int* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  *total = buf[1023];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t* __restrict__ lens,
                                                           int B, int cap, uint32_t* hdr,
                                                           int2* __restrict__ items) {
  __shared__ int buf[1024];
  const int tid = threadIdx.x;
  // total number of full partitions = offset of the first tail partition
  int nfull = 0, tot = 0;
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    const int L = b < B ? clamp_len(lens[b], cap) : 0;
    block_excl_scan(L / kPartTokens, buf, &tot);
    nfull += tot;
  }
  int full_off = 0, tail_off = 0;
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    const int L = b < B ? clamp_len(lens[b], cap) : 0;
    const int f = L / kPartTokens;
    const int t = (L % kPartTokens) != 0;
    int ftot, ttot;
    const int fo = block_excl_scan(f, buf, &ftot);
    const int to = block_excl_scan(t, buf, &ttot);
    for (int j = 0; j < f; ++j) items[full_off + fo + j] = make_int2(b, j);
    if (t) items[nfull + tail_off + to] = make_int2(b, f);
    full_off += ftot;
    tail_off += ttot;
  }
  if (tid < kQueues) hdr[tid * kCounterStride] = 0u;
  if (tid == 0) hdr[kItemCountWord] = (uint32_t)(nfull + tail_off);
}

// ---------------------------------------------------------------------------
// Tile geometry.  A tile is 16 consecutive tokens of one KV head.  Lane l
// loads 16-byte piece l % CPR of the head's row slice for tokens
// (l / CPR) * TPL + j, j < TPL, so each quarter-wave reads whole contiguous
// row slices (at most two 128-byte lines per 16 lanes).
// ---------------------------------------------------------------------------
template <typename T, int D>
struct Geo {
  static constexpr int ROWB = D * (int)sizeof(T);  // bytes of one head's row slice
  static constexpr int CPR = ROWB / 16;            // 16-byte pieces per row slice
  static constexpr int TPL = 16 * CPR / 64;        // tokens per lane per tile
  static constexpr int KST = ROWB + 16;            // LDS row stride of K (and of V for fp32)
  static constexpr int VTS = 40;                   // LDS row stride of transposed V (bf16): 16 tokens + pad
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int KBYTES = 16 * KST;
  static constexpr int VBYTES = kBf16 ? D * VTS : 16 * KST;
  static constexpr int IDS_BYTES = 4 * kMaxPartBlocks;  // block ids of one partition
  static constexpr int LDS_PER_WAVE = KBYTES + VBYTES + IDS_BYTES;
  static constexpr int NQ = kBf16 ? D / 32 : D / 4;  // QK MFMA steps over the head dimension
};

// Byte offsets into the pool: 32-bit when the pool is under 4 GiB (one VGPR
// per address, added to a scalar base), 64-bit otherwise.
template <bool kWide>
struct Off {
  typedef typename std::conditional<kWide, uint64_t, uint32_t>::type type;
};

template <typename T, int D>
struct TileRegs {
  u32x4_t k[Geo<T, D>::TPL];
  u32x4_t v[Geo<T, D>::TPL];
  uint32_t ok;  // bit j: token j of this lane is inside the partition with a valid block id
};

struct PoolView {
  const char* k;
  const char* v;
  uint32_t row_bytes;   // H_kv * D * elem: one token's row over all KV heads
  uint32_t head_bytes;  // this item's KV head offset within the row, plus the lane's piece
};

// Issues the K/V loads of one tile.  Block ids come from the wave's LDS copy
// of the partition's block-table slice (a global load here would make the
// wait for it drain the K/V loads already in flight).  Invalid tokens load
// row 0 (always in range, and cached) and are zeroed when staged.
template <typename T, int D, bool kWide, bool kAligned>
__device__ __forceinline__ void load_tile(const PoolView& pv, const int* __restrict__ ids, int blk0, int tile0,
                                          int end, int P, int p_shift, int N, TileRegs<T, D>& r) {
  using Gm = Geo<T, D>;
  using O = typename Off<kWide>::type;
  const int lane = lane_id();
  const int q = lane / Gm::CPR;
  const int first = tile0 + q * Gm::TPL;  // this lane's first token
  r.ok = 0;
  if constexpr (kAligned) {
    // the tile lies inside one block: one (broadcast) id lookup, rows are consecutive
    int lb, off;
    if (p_shift >= 0) {
      lb = tile0 >> p_shift;
      off = tile0 & ((1 << p_shift) - 1);
    } else {
      lb = tile0 / P;
      off = tile0 - lb * P;
    }
    const int blk = ids[lb - blk0];
    const bool bok = blk >= 0 && blk < N;
    const O base = bok ? ((O)blk * (O)P + (O)(off + q * Gm::TPL)) * (O)pv.row_bytes : (O)0;
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j) {
      const bool ok = bok && first + j < end;
      r.ok |= (ok ? 1u : 0u) << j;
      const O e = (ok ? base + (O)j * (O)pv.row_bytes : (O)0) + (O)pv.head_bytes;
      r.k[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pv.k + e));
      r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pv.v + e));
    }
  } else {
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j) {
      const int pos = first + j;
      int lb, off;
      if (p_shift >= 0) {
        lb = pos >> p_shift;
        off = pos & ((1 << p_shift) - 1);
      } else {
        lb = pos / P;
        off = pos - lb * P;
      }
      const bool in = pos < end;
      const int blk = ids[in ? lb - blk0 : 0];
      const bool ok = in && blk >= 0 && blk < N;
      r.ok |= (ok ? 1u : 0u) << j;
      const O e = (ok ? ((O)blk * (O)P + (O)off) * (O)pv.row_bytes : (O)0) + (O)pv.head_bytes;
      r.k[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pv.k + e));
      r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pv.v + e));
    }
  }
}

// Registers -> this wave's LDS region: K row-major; V transposed (bf16, d-major
// so a P.V operand is one 8-byte read) or row-major (fp32).
template <typename T, int D>
__device__ __forceinline__ void stage_tile(char* lds, TileRegs<T, D>& r, bool full) {
  using Gm = Geo<T, D>;
  const int lane = lane_id();
  const int c = lane % Gm::CPR, q = lane / Gm::CPR;
  if (!full) {
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j)
      if (!((r.ok >> j) & 1u)) {
        r.k[j] = u32x4_t{0u, 0u, 0u, 0u};
        r.v[j] = u32x4_t{0u, 0u, 0u, 0u};
      }
  }
#pragma unroll
  for (int j = 0; j < Gm::TPL; ++j)
    *reinterpret_cast<u32x4_t*>(lds + (q * Gm::TPL + j) * Gm::KST + 16 * c) = r.k[j];
  char* vl = lds + Gm::KBYTES;
  if constexpr (Gm::kBf16) {
    // piece c holds head elements 8c..8c+7; this lane owns tokens q*TPL .. q*TPL+TPL-1
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int d = 8 * c + 2 * w;
      if constexpr (Gm::TPL == 4) {
        const u32x2_t lo = {__builtin_amdgcn_perm(r.v[1][w], r.v[0][w], 0x05040100u),
                            __builtin_amdgcn_perm(r.v[3][w], r.v[2][w], 0x05040100u)};
        const u32x2_t hi = {__builtin_amdgcn_perm(r.v[1][w], r.v[0][w], 0x07060302u),
                            __builtin_amdgcn_perm(r.v[3][w], r.v[2][w], 0x07060302u)};
        *reinterpret_cast<u32x2_t*>(vl + d * Gm::VTS + 8 * q) = lo;
        *reinterpret_cast<u32x2_t*>(vl + (d + 1) * Gm::VTS + 8 * q) = hi;
      } else {
        static_assert(Gm::TPL == 2, "bf16 tiles hold 2 or 4 tokens per lane");
        *reinterpret_cast<uint32_t*>(vl + d * Gm::VTS + 4 * q) = __builtin_amdgcn_perm(r.v[1][w], r.v[0][w], 0x05040100u);
        *reinterpret_cast<uint32_t*>(vl + (d + 1) * Gm::VTS + 4 * q) =
            __builtin_amdgcn_perm(r.v[1][w], r.v[0][w], 0x07060302u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j)
      *reinterpret_cast<u32x4_t*>(vl + (q * Gm::TPL + j) * Gm::KST + 16 * c) = r.v[j];
  }
}

// Orders this wave's LDS stores before its later LDS loads (the wave reads
// what other lanes of the same wave wrote).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Partition kernel.
// ---------------------------------------------------------------------------
struct DecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* lens;
  void* out;
  const uint32_t* hdr;
  uint32_t* counter;
  const int2* items;
  float* ml;
  float* o;
  float scale_log2;
  int Hq, Hkv, G, n_hg, P, p_shift, N, M, cap, max_parts;
};

// Softmax reference max is moved only when a score exceeds it by more than
// this (log2 units), so probabilities stay below 2^8 and the rescale of the
// accumulators is rare; the result does not depend on the reference.
constexpr float kRescaleSlack = 8.0f;

// One wave = one work item (request, partition, KV head, group of up to 4
// query heads).  Per 16-token tile:
//   S^T = K Q^T   (A = K rows from LDS, B = Q^T with the group's heads as
//                  columns 0..3), so lane (n, g) gets the scores of head n for
//                  tokens 4g .. 4g+3;
//   online softmax per head (max over the lane's 4 tokens, then across the
//                  four 16-lane rows);
//   O^T += V^T P^T (A = V^T from LDS, B = the lane's own probabilities), so
//                  lane (n, g) accumulates head n's outputs d = 16db + 4g + j.
template <typename T, int D, bool kWide, bool kAligned>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeParams prm) {
  using Gm = Geo<T, D>;
  constexpr int NDB = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* lds = smem + (threadIdx.x >> 6) * Gm::LDS_PER_WAVE;
  int* ids = reinterpret_cast<int*>(lds + Gm::KBYTES + Gm::VBYTES);
  const int lane = lane_id();
  const int n = lane & 15;  // head column (S^T, O^T) / token row (K operand)
  const int g = lane >> 4;
  const uint32_t per_item = (uint32_t)(prm.Hkv * prm.n_hg);
  const uint32_t total = prm.hdr[kItemCountWord] * per_item;
  const T* __restrict__ q = static_cast<const T*>(prm.q);
  PoolView pv;
  pv.k = static_cast<const char*>(prm.kc);
  pv.v = static_cast<const char*>(prm.vc);
  pv.row_bytes = (uint32_t)(prm.Hkv * Gm::ROWB);

  // Item f of the flat list (items x KV heads x head groups).  The first item
  // of each wave is its global wave index.  The rest are split into kQueues
  // interleaved queues, f = nwaves + kQueues * c + x for the c-th claim of
  // queue x; a wave claims from the queue of its XCD (blocks are dealt to the
  // XCDs round robin) and moves on to the next queue when that one is empty.
  // Separate counters keep the claims from serialising on one address.
  const uint32_t nwaves = gridDim.x * (blockDim.x >> 6);
  const uint32_t home = blockIdx.x % kQueues;
  uint32_t queue = 0;  // queues found empty so far
  uint32_t f = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  for (;;) {
    if (f >= total) {
      if (f < nwaves) break;  // fewer items than waves: no queued items either
      bool got = false;
      while (queue < kQueues) {
        const uint32_t x = (home + queue) % kQueues;
        uint32_t c = 0;
        if (lane == 0) c = atomicAdd(prm.counter + x * kCounterStride, 1u);
        c = __builtin_amdgcn_readfirstlane(c);
        const uint32_t fx = nwaves + kQueues * c + x;
        if (fx < total) {
          f = fx;
          got = true;
          break;
        }
        ++queue;
      }
      if (!got) break;
    }
    const int2 it = prm.items[f / per_item];
    const int rem = (int)(f % per_item);
    const int b = it.x, part = it.y;
    const int hkv = rem / prm.n_hg;
    const int hg = rem - hkv * prm.n_hg;
    const int L = clamp_len(prm.lens[b], prm.cap);
    const int nparts = (L + kPartTokens - 1) / kPartTokens;
    const int tok0 = part * kPartTokens;
    const int tok_end = min(L, tok0 + kPartTokens);
    const int ntiles = (tok_end - tok0 + kTile - 1) / kTile;
    const int nh = min(4, prm.G - hg * 4);  // valid heads of this group (columns 0..nh-1)
    const int32_t* __restrict__ bt_row = prm.bt + (int64_t)b * prm.M;
    const bool col_ok = n < nh;
    const int h = hkv * prm.G + hg * 4 + (col_ok ? n : 0);
    pv.head_bytes = (uint32_t)(hkv * Gm::ROWB + 16 * (lane % Gm::CPR));

    // Q^T operand: column n = query head h; k = head dimension
    u32x4_t qv[Gm::kBf16 ? Gm::NQ : Gm::NQ / 4];
    {
      const T* qrow = q + ((int64_t)b * prm.Hq + h) * D;
      if constexpr (Gm::kBf16) {
#pragma unroll
        for (int i = 0; i < Gm::NQ; ++i)
          qv[i] = col_ok ? *reinterpret_cast<const u32x4_t*>(qrow + 32 * i + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int i = 0; i < Gm::NQ / 4; ++i)
          qv[i] = col_ok ? *reinterpret_cast<const u32x4_t*>(qrow + g * (D / 4) + 4 * i) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }

    // this partition's block ids -> the wave's LDS
    int blk0, blk_last;
    if (prm.p_shift >= 0) {
      blk0 = tok0 >> prm.p_shift;
      blk_last = (tok_end - 1) >> prm.p_shift;
    } else {
      blk0 = tok0 / prm.P;
      blk_last = (tok_end - 1) / prm.P;
    }
    wave_lds_sync();  // the previous item is done with the LDS
    for (int i = lane; i <= blk_last - blk0; i += 64) ids[i] = bt_row[blk0 + i];
    wave_lds_sync();

    float m = -INFINITY, l = 0.f;
    f32x4_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // software pipeline: the next tile's K/V loads are in flight while one computes
    TileRegs<T, D> regs;
    load_tile<T, D, kWide, kAligned>(pv, ids, blk0, tok0, tok_end, prm.P, prm.p_shift, prm.N, regs);
    for (int t = 0; t < ntiles; ++t) {
      const int tile0 = tok0 + t * kTile;
      // every token of the tile valid: no zeroing needed (the usual case)
      bool full;
      if constexpr (kAligned)
        full = tile0 + kTile <= tok_end && __builtin_amdgcn_readfirstlane((int)regs.ok) == (1 << Gm::TPL) - 1;
      else
        full = __builtin_amdgcn_readfirstlane((int)(__ballot(regs.ok != (1u << Gm::TPL) - 1u) == 0));
      wave_lds_sync();  // previous tile's LDS reads are done
      stage_tile<T, D>(lds, regs, full);
      wave_lds_sync();
      if (t + 1 < ntiles)
        load_tile<T, D, kWide, kAligned>(pv, ids, blk0, tile0 + kTile, tok_end, prm.P, prm.p_shift, prm.N, regs);

      // ---- S^T = K Q^T ----
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
      if constexpr (Gm::kBf16) {
#pragma unroll
        for (int i = 0; i < Gm::NQ; ++i) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lds + n * Gm::KST + 2 * (32 * i + 8 * g));
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, qv[i]), s, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < Gm::NQ / 4; ++i) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lds + n * Gm::KST + 4 * (g * (D / 4) + 4 * i));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(qv[i][j]), s, 0, 0, 0);
        }
      }
      // ---- online softmax for head n over tokens tile0 + 4g + j ----
      float sc[4];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = (tile0 + 4 * g + j < tok_end) ? s[j] * prm.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (mx > m + kRescaleSlack) {  // also true for the first tile (m = -inf)
        if (m != -INFINITY) {
          const float alpha = fast_exp2(m - mx);
          l *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        }
        m = mx;
      }
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = fast_exp2(sc[j] - m);
        l += p[j];
      }
      // ---- O^T += V^T P^T ----
      const char* vl = lds + Gm::KBYTES;
      if constexpr (Gm::kBf16) {
        const u32x2_t pb = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2_t a = *reinterpret_cast<const u32x2_t*>(vl + (16 * db + n) * Gm::VTS + 8 * g);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                            __builtin_bit_cast(s16x4_t, pb), o[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = *reinterpret_cast<const float*>(vl + (4 * g + j) * Gm::KST + 4 * (16 * db + n));
            o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, p[j], o[db], 0, 0, 0);
          }
      }
    }

    // ---- finish: total of l over the four 16-lane rows; store head n ----
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (col_ok) {
      if (nparts == 1) {
        const float inv = 1.0f / l;
        T* dst = static_cast<T*>(prm.out) + ((int64_t)b * prm.Hq + h) * D + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          if constexpr (Gm::kBf16) {
            *reinterpret_cast<u32x2_t*>(dst + 16 * db) =
                u32x2_t{pack_bf16(o[db][0] * inv, o[db][1] * inv), pack_bf16(o[db][2] * inv, o[db][3] * inv)};
          } else {
            *reinterpret_cast<f32x4_t*>(dst + 16 * db) = o[db] * inv;
          }
        }
      } else {
        const int64_t slot = ((int64_t)b * prm.Hq + h) * prm.max_parts + part;
        float* dst = prm.o + slot * D + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4_t*>(dst + 16 * db) = o[db];
        if (g == 0) {
          prm.ml[slot * 2 + 0] = m;
          prm.ml[slot * 2 + 1] = l;
        }
      }
    }
    f = 0xffffffffu;  // this item is done: claim the next one
  }
}

// ---------------------------------------------------------------------------
// Reduce: merge the partitions of requests that have more than one; write
// zeros for empty requests.  One wave per (query head, request).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams prm) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = clamp_len(prm.lens[b], prm.cap);
  const int np = (L + kPartTokens - 1) / kPartTokens;
  if (np == 1) return;
  T* dst = static_cast<T*>(prm.out) + ((int64_t)b * prm.Hq + h) * D;
  if (np == 0) {
    for (int d = lane; d < D; d += 64) {
      if constexpr (sizeof(T) == 2) dst[d] = 0;
      else dst[d] = 0.f;
    }
    return;
  }
  const int64_t slot0 = ((int64_t)b * prm.Hq + h) * prm.max_parts;
  float mx = -INFINITY;
  for (int i = lane; i < np; i += 64) mx = fmaxf(mx, prm.ml[(slot0 + i) * 2]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  constexpr int PER = D / 64;
  float acc[PER], den = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int i = 0; i < np; ++i) {
    const float w = fast_exp2(prm.ml[(slot0 + i) * 2] - mx);
    den = fmaf(w, prm.ml[(slot0 + i) * 2 + 1], den);
    const float* src = prm.o + (slot0 + i) * D;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = fmaf(w, src[lane + 64 * j], acc[j]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if constexpr (sizeof(T) == 2) dst[lane + 64 * j] = (bf16_bits)f32_to_bf16(acc[j] * inv);
    else dst[lane + 64 * j] = acc[j] * inv;
  }
}

template <typename T, int D, bool kWide, bool kAligned>
hipError_t launch_typed(const DecodeParams& prm, int B, int64_t max_items, hipStream_t stream,
                        hipEvent_t ev0, hipEvent_t ev1) {
  // waves are independent workers; a block holds as many as fit in 64 KiB of LDS (at most 4)
  constexpr int wpb = Geo<T, D>::LDS_PER_WAVE * kWavesPerBlock <= 65536 ? kWavesPerBlock : 2;
  constexpr unsigned lds_bytes = Geo<T, D>::LDS_PER_WAVE * wpb;
  // exactly the blocks that can be resident at once: every wave starts on its
  // first item immediately, and none waits for a slot while holding one
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_partition_kernel<T, D, kWide, kAligned>,
                                                     64 * wpb, lds_bytes) != hipSuccess || nb < 1)
      nb = 1;
    per_cu = nb;
  }
  const int64_t want = (max_items + wpb - 1) / wpb;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  const unsigned blocks = (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_partition_kernel<T, D, kWide, kAligned>), dim3(blocks), dim3(64 * wpb), lds_bytes,
                     stream, prm);
  if (ev1) {
    const hipError_t e = hipEventRecord(ev1, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(prm.Hq, B), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_sized(const DecodeParams& prm, int B, int64_t max_items, int64_t pool_bytes,
                        hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  // tiles of 16 tokens never straddle a block when P is a multiple of 16
  const bool aligned = prm.P % kTile == 0;
  if (pool_bytes < ((int64_t)1 << 32)) {
    if (aligned) return launch_typed<T, D, false, true>(prm, B, max_items, stream, ev0, ev1);
    return launch_typed<T, D, false, false>(prm, B, max_items, stream, ev0, ev1);
  }
  if (aligned) return launch_typed<T, D, true, true>(prm, B, max_items, stream, ev0, ev1);
  return launch_typed<T, D, true, false>(prm, B, max_items, stream, ev0, ev1);
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
  prm.counter = reinterpret_cast<uint32_t*>(ws + Lw.hdr);
  prm.items = reinterpret_cast<const int2*>(ws + Lw.items);
  prm.ml = reinterpret_cast<float*>(ws + Lw.ml);
  prm.o = reinterpret_cast<float*>(ws + Lw.o);
  prm.scale_log2 = a.scale * kLog2e;
  prm.Hq = a.num_q_heads;
  prm.Hkv = a.num_kv_heads;
  prm.G = a.num_q_heads / a.num_kv_heads;
  prm.n_hg = (prm.G + 3) / 4;
  prm.P = a.block_size;
  prm.p_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz((unsigned)a.block_size) : -1;
  prm.N = (int)a.num_blocks;
  prm.M = a.max_blocks;
  prm.cap = (int)((int64_t)a.max_blocks * a.block_size);
  prm.max_parts = (int)Lw.max_parts;

  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, a.context_lens, a.num_seqs,
                     prm.cap, reinterpret_cast<uint32_t*>(ws + Lw.hdr),
                     reinterpret_cast<int2*>(ws + Lw.items));
  const int64_t max_items = (int64_t)a.num_seqs * Lw.max_parts * prm.Hkv * prm.n_hg;
  const int64_t pool_bytes =
      a.num_blocks * a.block_size * a.num_kv_heads * a.head_dim * (a.dtype == kBF16 ? 2 : 4);
  if (a.dtype == kBF16) {
    if (a.head_dim == 128)
      return launch_sized<bf16_bits, 128>(prm, a.num_seqs, max_items, pool_bytes, stream, ev0, ev1);
    return launch_sized<bf16_bits, 64>(prm, a.num_seqs, max_items, pool_bytes, stream, ev0, ev1);
  }
  if (a.head_dim == 128) return launch_sized<float, 128>(prm, a.num_seqs, max_items, pool_bytes, stream, ev0, ev1);
  return launch_sized<float, 64>(prm, a.num_seqs, max_items, pool_bytes, stream, ev0, ev1);
}

}  // namespace pa
