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
//   * Work item = (request, tile of TQ = 128 / G chunk tokens, KV head).  The
//     G query heads that share a KV head are packed into the item's 128 rows
//     (head-major), so each K/V tile fetched from the pool serves all of them.
//   * A persistent grid pulls items from a queue that a plan kernel sorts by
//     decreasing key count (largest causal extents first).
//   * Per 64-key tile the 256 threads gather K and V rows through the block
//     table (16-byte loads), K stored as is in LDS and V stored transposed
//     (d-major) so that both MFMA operands are contiguous LDS reads.  The next
//     tile's loads are in flight while the current tile computes.
//   * Each wave owns 32 rows.  S^T = K Q^T and O^T += V^T P^T run as
//     16x16x32 bf16 MFMAs with fp32 accumulation.  Computing the transposed
//     scores leaves each lane holding one query row's scores for a run of keys,
//     which is exactly the B-operand layout the P.V product needs, so P never
//     leaves registers.  Online softmax in base 2, fp32.
//   * Keys past the causal limit, tail slots and out-of-range block ids are
//     masked and never multiply a value: masked K/V tile rows are zero-filled.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kRows = 128;   // rows (chunk token x query head) per work item
constexpr int kTK = 64;      // keys per tile
constexpr int kThreads = 256;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int tokens_per_tile(int G) { return kRows / G; }

int64_t max_prefill_items(int num_seqs, int64_t num_q_tokens, int G) {
  const int TQ = tokens_per_tile(G);
  return (num_q_tokens + TQ - 1) / TQ + num_seqs;
}

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// ---------------------------------------------------------------------------
// Plan: list (request, q tile) items sorted by decreasing number of key tiles
// (counting sort; ties in any order -- each item is computed independently,
// so the order never changes a result).
// ---------------------------------------------------------------------------
constexpr int kBuckets = 1024;

__device__ __forceinline__ bool chunk_ok(const int32_t* __restrict__ cu, int b, int T, int L,
                                         int num_q_tokens) {
  return T > 0 && T <= L && cu[b] >= 0 && cu[b + 1] <= num_q_tokens;
}

__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t* __restrict__ cu,
                                                            const int32_t* __restrict__ lens, int B,
                                                            int cap, int TQ, int num_q_tokens,
                                                            int item_cap, uint32_t* hdr,
                                                            int2* __restrict__ items) {
  __shared__ int hist[kBuckets];
  __shared__ int total;
  const int tid = threadIdx.x;
  for (int i = tid; i < kBuckets; i += 1024) hist[i] = 0;
  if (tid == 0) total = 0;
  __syncthreads();
  for (int b = tid; b < B; b += 1024) {
    const int T = cu[b + 1] - cu[b];
    const int L = clamp_len(lens[b], cap);
    if (!chunk_ok(cu, b, T, L, num_q_tokens)) continue;
    const int nq = (T + TQ - 1) / TQ;
    for (int j = 0; j < nq; ++j) {
      const int kmax = L - T + min(T, (j + 1) * TQ);
      const int bucket = min((kmax + kTK - 1) / kTK, kBuckets - 1);
      atomicAdd(&hist[bucket], 1);
    }
    atomicAdd(&total, nq);
  }
  __syncthreads();
  // descending exclusive scan over buckets (serial, 1024 entries)
  if (tid == 0) {
    int run = 0;
    for (int i = kBuckets - 1; i >= 0; --i) {
      const int c = hist[i];
      hist[i] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int b = tid; b < B; b += 1024) {
    const int T = cu[b + 1] - cu[b];
    const int L = clamp_len(lens[b], cap);
    if (!chunk_ok(cu, b, T, L, num_q_tokens)) continue;
    const int nq = (T + TQ - 1) / TQ;
    for (int j = 0; j < nq; ++j) {
      const int kmax = L - T + min(T, (j + 1) * TQ);
      const int bucket = min((kmax + kTK - 1) / kTK, kBuckets - 1);
      const int at = atomicAdd(&hist[bucket], 1);
      if (at < item_cap) items[at] = make_int2(b, j);
    }
  }
  if (tid == 0) {
    hdr[0] = 0u;
    hdr[1] = (uint32_t)min(total, item_cap);
  }
}

struct PrefillParams {
  const bf16_bits* q;
  const bf16_bits* kc;
  const bf16_bits* vc;
  const int32_t* cu;
  const int32_t* bt;
  const int32_t* lens;
  bf16_bits* out;
  const uint32_t* hdr;
  uint32_t* counter;
  const int2* items;
  float scale_log2;
  int Hq, Hkv, G, TQ, P, p_shift, N, M, cap;
};

template <int D>
struct __attribute__((aligned(16))) PrefillLds {
  static constexpr int KST = D + 8;     // K row stride (elements)
  static constexpr int VST = kTK + 4;   // V^T row stride (elements)
  bf16_bits k[kTK * KST];
  bf16_bits vt[D * VST];
};

// Gathers of one 64-key tile, held in registers between the global loads
// and the LDS stores.
template <int D>
struct TileRegs {
  static constexpr int KV = D / 4 * 2 / 16;  // 16-byte pieces of K per thread
  u32x4_t k[KV];
  u32x4_t v[4];
};

__device__ __forceinline__ int64_t key_row(const int32_t* __restrict__ bt_row, int pos, int kmax, int P,
                                           int p_shift, int N) {
  if (pos >= kmax) return -1;
  int j, off;
  if (p_shift >= 0) {
    j = pos >> p_shift;
    off = pos & ((1 << p_shift) - 1);
  } else {
    j = pos / P;
    off = pos - j * P;
  }
  const int blk = bt_row[j];
  if (blk < 0 || blk >= N) return -1;
  return (int64_t)blk * P + off;
}

template <int D>
__device__ __forceinline__ void load_tile(const PrefillParams& p, const int32_t* __restrict__ bt_row,
                                          int hkv, int k0, int kmax, TileRegs<D>& r) {
  const int tid = threadIdx.x;
  const int64_t row_elems = (int64_t)p.Hkv * D;
  // K: thread -> key tid/4, quarter tid%4 of the head
  {
    const int kk = tid >> 2, c = tid & 3;
    const int64_t row = key_row(bt_row, k0 + kk, kmax, p.P, p.p_shift, p.N);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p.kc + row * row_elems + (int64_t)hkv * D + c * (D / 4));
#pragma unroll
    for (int i = 0; i < TileRegs<D>::KV; ++i) r.k[i] = row >= 0 ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
  }
  // V: thread -> keys 4*kq .. 4*kq+3, head elements 8*dc .. 8*dc+7
  {
    constexpr int DC = D / 8;
    const int kq = tid / DC, dc = tid % DC;
    if (kq < 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = key_row(bt_row, k0 + 4 * kq + j, kmax, p.P, p.p_shift, p.N);
        const u32x4_t* src =
            reinterpret_cast<const u32x4_t*>(p.vc + row * row_elems + (int64_t)hkv * D + dc * 8);
        r.v[j] = row >= 0 ? *src : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(PrefillLds<D>& s, const TileRegs<D>& r) {
  const int tid = threadIdx.x;
  {
    const int kk = tid >> 2, c = tid & 3;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&s.k[kk * PrefillLds<D>::KST + c * (D / 4)]);
#pragma unroll
    for (int i = 0; i < TileRegs<D>::KV; ++i) dst[i] = r.k[i];
  }
  {
    constexpr int DC = D / 8;
    const int kq = tid / DC, dc = tid % DC;
    if (kq < 16) {
      // transpose the 4 keys x 8 elements block into 8 rows of 4 keys
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w0 = r.v[0][i], w1 = r.v[1][i], w2 = r.v[2][i], w3 = r.v[3][i];
        const u32x2_t lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
        const u32x2_t hi = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
        const int d = dc * 8 + 2 * i;
        *reinterpret_cast<u32x2_t*>(&s.vt[d * PrefillLds<D>::VST + 4 * kq]) = lo;
        *reinterpret_cast<u32x2_t*>(&s.vt[(d + 1) * PrefillLds<D>::VST + 4 * kq]) = hi;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int NI = D / 32;  // MFMA k-steps over the head dimension
  constexpr int NDB = D / 16; // 16-row blocks of O^T
  __shared__ PrefillLds<D> lds;
  __shared__ uint32_t s_item;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const uint32_t total = p.hdr[1] * (uint32_t)p.Hkv;

  for (;;) {
    __syncthreads();
    if (tid == 0) s_item = atomicAdd(p.counter, 1u);
    __syncthreads();
    const uint32_t f = s_item;
    if (f >= total) break;
    const int2 it = p.items[f / p.Hkv];
    const int hkv = (int)(f % p.Hkv);
    const int b = it.x, qt = it.y;
    const int cu0 = p.cu[b];
    const int T = p.cu[b + 1] - cu0;
    const int L = clamp_len(p.lens[b], p.cap);
    const int start = L - T;  // position of chunk row 0
    const int t0 = qt * p.TQ;
    const int nt = min(p.TQ, T - t0);
    const int kmax = start + t0 + nt;  // keys 0 .. kmax-1 are visible to some row
    const int nkt = (kmax + kTK - 1) / kTK;
    const int32_t* __restrict__ bt_row = p.bt + (int64_t)b * p.M;

    // rows of this wave: r = 32w + 16rb + n -> (head r / TQ, chunk token r % TQ)
    int pos[2];
    u32x4_t qop[2][NI];
    int wave_max = -1;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = 32 * w + 16 * rb + n;
      const int hl = r / p.TQ, tl = r - hl * p.TQ;
      const bool ok = hl < p.G && tl < nt;
      pos[rb] = ok ? start + t0 + tl : -1;
      const int64_t qrow = ((int64_t)(cu0 + t0 + tl) * p.Hq + hkv * p.G + hl) * D;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        qop[rb][i] = ok ? *reinterpret_cast<const u32x4_t*>(p.q + qrow + 32 * i + 8 * g)
                        : u32x4_t{0u, 0u, 0u, 0u};
      wave_max = max(wave_max, pos[rb]);
    }
    // largest position of any row in the wave (uniform)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wave_max = max(wave_max, __shfl_xor(wave_max, off));

    float m[2], l[2];
    f32x4_t o[NDB][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      m[rb] = -INFINITY;
      l[rb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    TileRegs<D> regs;
    load_tile<D>(p, bt_row, hkv, 0, kmax, regs);
    for (int kt = 0; kt < nkt; ++kt) {
      const int k0 = kt * kTK;
      __syncthreads();
      store_tile<D>(lds, regs);
      __syncthreads();
      if (kt + 1 < nkt) load_tile<D>(p, bt_row, hkv, k0 + kTK, kmax, regs);
      if (k0 > wave_max) continue;  // every row of this wave is causally done

      // ---- S^T = K Q^T : 4 key blocks x 2 row blocks ----
      f32x4_t s[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        s[kb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
              &lds.k[(kb * 16 + n) * PrefillLds<D>::KST + 32 * i + 8 * g]);
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
          s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, qop[0][i]),
                                                             s[kb][0], 0, 0, 0);
          s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, qop[1][i]),
                                                             s[kb][1], 0, 0, 0);
        }
      }
      // ---- mask, online softmax (per row = per lane column n) ----
      u32x4_t pop[2][2];  // [rb][k-step]: P^T operand, 8 bf16
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kp = k0 + kb * 16 + 4 * g + j;
            const float v = kp <= pos[rb] ? s[kb][rb][j] * p.scale_log2 : -INFINITY;
            s[kb][rb][j] = v;
            tmax = fmaxf(tmax, v);
          }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(m[rb], tmax);
        const float muse = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = fast_exp2(m[rb] - muse);
        m[rb] = mnew;
        l[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][rb] *= alpha;
        float pv[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pv[kb][j] = fast_exp2(s[kb][rb][j] - muse);
            l[rb] += pv[kb][j];
          }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          pop[rb][st] = u32x4_t{pack_bf16(pv[2 * st][0], pv[2 * st][1]), pack_bf16(pv[2 * st][2], pv[2 * st][3]),
                                pack_bf16(pv[2 * st + 1][0], pv[2 * st + 1][1]),
                                pack_bf16(pv[2 * st + 1][2], pv[2 * st + 1][3])};
        }
      }
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16_bits* vrow = &lds.vt[(db * 16 + n) * PrefillLds<D>::VST + 32 * st + 4 * g];
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 16);
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
          o[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, pop[0][st]),
                                                             o[db][0], 0, 0, 0);
          o[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, pop[1][st]),
                                                             o[db][1], 0, 0, 0);
        }
      }
    }

    // ---- normalise and store: lane holds O^T[d = 16db + 4g + j][row n] ----
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float lt = l[rb];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      if (pos[rb] < 0) continue;
      const int r = 32 * w + 16 * rb + n;
      const int hl = r / p.TQ, tl = r - hl * p.TQ;
      const float inv = 1.0f / lt;
      bf16_bits* dst = p.out + ((int64_t)(cu0 + t0 + tl) * p.Hq + hkv * p.G + hl) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x2_t v = {pack_bf16(o[db][rb][0] * inv, o[db][rb][1] * inv),
                           pack_bf16(o[db][rb][2] * inv, o[db][rb][3] * inv)};
        *reinterpret_cast<u32x2_t*>(dst + 16 * db) = v;
      }
    }
  }
}

}  // namespace

size_t prefill_workspace_size(int num_seqs, int64_t num_q_tokens, int num_q_heads, int num_kv_heads) {
  const int G = num_q_heads / num_kv_heads;
  return 256 + align256(sizeof(int2) * (size_t)max_prefill_items(num_seqs, num_q_tokens, G));
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  char* ws = static_cast<char*>(a.workspace);
  PrefillParams p;
  p.q = static_cast<const bf16_bits*>(a.q);
  p.kc = static_cast<const bf16_bits*>(a.k_cache);
  p.vc = static_cast<const bf16_bits*>(a.v_cache);
  p.cu = a.cu_seqlens;
  p.bt = a.block_table;
  p.lens = a.context_lens;
  p.out = static_cast<bf16_bits*>(a.out);
  p.hdr = reinterpret_cast<const uint32_t*>(ws);
  p.counter = reinterpret_cast<uint32_t*>(ws);
  p.items = reinterpret_cast<const int2*>(ws + 256);
  p.scale_log2 = a.scale * kLog2e;
  p.Hq = a.num_q_heads;
  p.Hkv = a.num_kv_heads;
  p.G = a.num_q_heads / a.num_kv_heads;
  p.TQ = tokens_per_tile(p.G);
  p.P = a.block_size;
  p.p_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz((unsigned)a.block_size) : -1;
  p.N = (int)a.num_blocks;
  p.M = a.max_blocks;
  p.cap = (int)((int64_t)a.max_blocks * a.block_size);

  const int64_t item_cap = max_prefill_items(a.num_seqs, a.num_q_tokens, p.G);
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, a.context_lens,
                     a.num_seqs, p.cap, p.TQ, (int)a.num_q_tokens, (int)item_cap,
                     reinterpret_cast<uint32_t*>(ws), reinterpret_cast<int2*>(ws + 256));
  const int64_t max_items = item_cap * p.Hkv;
  const int64_t cap = (int64_t)device_cu_count() * 2;
  const unsigned blocks = (unsigned)(max_items < cap ? max_items : cap);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
  if (a.head_dim == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream, p);
  if (ev1) {
    const hipError_t e = hipEventRecord(ev1, stream);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace pa
