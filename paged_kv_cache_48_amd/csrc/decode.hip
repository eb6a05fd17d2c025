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
//     full partitions first and short tail partitions last, and zeroes a queue
//     counter; a persistent grid of waves pulls items with one atomic each.
//   * Per 16-token tile the wave loads K and V straight from HBM, 16-byte
//     vector loads, lane (n, g) holding token n's quarter g of the head
//     (4 lanes read one 256-byte row).  QK^T is one MFMA chain
//     (16x16x32 bf16 or 16x16x4 f32): the up-to-4 query heads are replicated
//     over the 16 A rows, so every lane receives the scores of all heads for
//     its own token without any cross-lane move.
//   * Online softmax in base 2 (running max and sum); the max over the tile's
//     16 tokens is a 4-step DPP reduction inside each 16-lane row.  P.V runs on
//     the VALU (fp32 FMA): each lane accumulates its token's contribution to its
//     quarter of the head; the 16 token lanes are merged once per item by a
//     DPP reduce-scatter, which leaves each lane with D/16 outputs to store.
//   * Items of a request with one partition write the output directly; the
//     others write (max, sum, unnormalised output) partials that the reduce
//     kernel merges:  m = max_i m_i,  out = sum_i 2^(m_i-m) o_i / sum_i 2^(m_i-m) l_i.
//   * Masked tokens never load: tail slots of a block may hold anything
//     (even NaN), and block ids outside [0, N) mask their token instead of
//     being dereferenced.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kTile = 16;                        // tokens per MFMA tile
constexpr int kWavesPerBlock = 4;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct DecodeLayout {
  int64_t max_parts;
  size_t hdr, items, ml, o, total;
};

DecodeLayout decode_layout(int B, int Hq, int D, int P, int M) {
  DecodeLayout L;
  L.max_parts = ((int64_t)M * P + kPartTokens - 1) / kPartTokens;
  size_t off = 0;
  L.hdr = off;
  off += 256;
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
  if (tid == 0) {
    hdr[0] = 0u;
    hdr[1] = (uint32_t)(nfull + tail_off);
  }
}

// ---------------------------------------------------------------------------
// Element-type traits: K/V slices, MFMA QK step, widening V to fp32.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct Traits {
  static constexpr int E = D / 4;                        // elements per lane per row
  static constexpr int NV = E * (int)sizeof(T) / 16;     // 16-byte vectors per lane
};

// QK^T for one tile: acc[m][n] = sum_k A[m][k] B[k][n], A = query rows, B = K^T.
template <int D>
__device__ __forceinline__ f32x4_t qk_mfma(const u32x4_t (&qv)[Traits<bf16_bits, D>::NV],
                                           const u32x4_t (&kv)[Traits<bf16_bits, D>::NV]) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < Traits<bf16_bits, D>::NV; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qv[i]),
                                                  __builtin_bit_cast(bf16x8_t, kv[i]), acc, 0, 0, 0);
  return acc;
}

template <int D>
__device__ __forceinline__ f32x4_t qk_mfma_f32(const u32x4_t (&qv)[Traits<float, D>::NV],
                                               const u32x4_t (&kv)[Traits<float, D>::NV]) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < Traits<float, D>::NV; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qv[i][j]), __uint_as_float(kv[i][j]),
                                                 acc, 0, 0, 0);
  return acc;
}

template <typename T, int D>
__device__ __forceinline__ void widen_slice(const u32x4_t (&v)[Traits<T, D>::NV],
                                            float (&f)[Traits<T, D>::E]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < Traits<T, D>::NV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[8 * i + 2 * j] = bf16_lo(v[i][j]);
        f[8 * i + 2 * j + 1] = bf16_hi(v[i][j]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < Traits<T, D>::NV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * i + j] = __uint_as_float(v[i][j]);
  }
}

template <typename T, int D>
__device__ __forceinline__ void load_slice(const T* base, bool valid, u32x4_t (&v)[Traits<T, D>::NV]) {
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base);
#pragma unroll
  for (int i = 0; i < Traits<T, D>::NV; ++i) {
    if (valid) v[i] = __builtin_nontemporal_load(p + i);
    else v[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Physical row (blk * P + pos % P) of logical position pos, or -1 if the
// position is past the partition end or its block id is out of range.
__device__ __forceinline__ int64_t token_row(const int32_t* __restrict__ bt_row, int pos, int end,
                                             int P, int p_shift, int N) {
  if (pos >= end) return -1;
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

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeParams prm) {
  using Tr = Traits<T, D>;
  constexpr int E = Tr::E;
  constexpr int NV = Tr::NV;
  const int lane = lane_id();
  const int n = lane & 15;  // token column / A row
  const int g = lane >> 4;  // quarter of the head this lane holds
  const bool b3 = n & 8, b2 = n & 4, b1 = n & 2, b0 = n & 1;
  const uint32_t per_item = (uint32_t)(prm.Hkv * prm.n_hg);
  const uint32_t total = prm.hdr[1] * per_item;
  const T* __restrict__ q = static_cast<const T*>(prm.q);
  const T* __restrict__ kc = static_cast<const T*>(prm.kc);
  const T* __restrict__ vc = static_cast<const T*>(prm.vc);
  const int64_t row_elems = (int64_t)prm.Hkv * D;

  for (;;) {
    uint32_t f = 0;
    if (lane == 0) f = atomicAdd(prm.counter, 1u);
    f = __builtin_amdgcn_readfirstlane(f);
    if (f >= total) break;
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
    const int nh = min(4, prm.G - hg * 4);  // valid heads of this group
    const int32_t* __restrict__ bt_row = prm.bt + (int64_t)b * prm.M;

    // Query operand: A row n carries local head n & 3 (replicated 4 times).
    u32x4_t qv[NV];
    {
      const int r = n & 3;
      const bool qok = r < nh;
      const int h = hkv * prm.G + hg * 4 + (qok ? r : 0);
      load_slice<T, D>(q + ((int64_t)b * prm.Hq + h) * D + g * E, qok, qv);
    }
    const int64_t head_off = (int64_t)hkv * D + g * E;

    float m[4], l[4], o[4][E];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[r] = -INFINITY;
      l[r] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) o[r][e] = 0.f;
    }

    // software pipeline: K/V of tile t+1 are in flight while tile t computes
    u32x4_t kcur[NV], vcur[NV];
    int64_t row = token_row(bt_row, tok0 + n, tok_end, prm.P, prm.p_shift, prm.N);
    load_slice<T, D>(kc + row * row_elems + head_off, row >= 0, kcur);
    load_slice<T, D>(vc + row * row_elems + head_off, row >= 0, vcur);
    bool cur_ok = row >= 0;

    for (int t = 0; t < ntiles; ++t) {
      u32x4_t knxt[NV], vnxt[NV];
      const int64_t nrow = token_row(bt_row, tok0 + (t + 1) * kTile + n, tok_end, prm.P, prm.p_shift, prm.N);
      load_slice<T, D>(kc + nrow * row_elems + head_off, nrow >= 0, knxt);
      load_slice<T, D>(vc + nrow * row_elems + head_off, nrow >= 0, vnxt);

      f32x4_t acc;
      if constexpr (sizeof(T) == 2) acc = qk_mfma<D>(qv, kcur);
      else acc = qk_mfma_f32<D>(qv, kcur);

      float s[4], mnew[4];
      bool grow = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] = cur_ok ? acc[r] * prm.scale_log2 : -INFINITY;
        mnew[r] = fmaxf(m[r], row16_max(s[r]));
        grow |= mnew[r] > m[r];
      }
      if (grow) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float alpha = fast_exp2(m[r] - mnew[r]);
          m[r] = mnew[r];
          l[r] *= alpha;
#pragma unroll
          for (int e = 0; e < E; ++e) o[r][e] *= alpha;
        }
      }
      float vf[E];
      widen_slice<T, D>(vcur, vf);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < nh) {
          const float p = fast_exp2(s[r] - m[r]);
          l[r] += p;
#pragma unroll
          for (int e = 0; e < E; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
        }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        kcur[i] = knxt[i];
        vcur[i] = vnxt[i];
      }
      cur_ok = nrow >= 0;
    }

    // ---- merge the 16 token lanes of each row: DPP reduce-scatter ----------
    float a2[2][E];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float keep = b3 ? o[i + 2][e] : o[i][e];
        const float send = b3 ? o[i][e] : o[i + 2][e];
        a2[i][e] = keep + dpp<kDppRowRor8>(send);
      }
    float c1[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float keep = b2 ? a2[1][e] : a2[0][e];
      const float send = b2 ? a2[0][e] : a2[1][e];
      c1[e] = keep + dpp<kDppRowHalfMirror>(send);
    }
    float c2[E / 2];
#pragma unroll
    for (int e = 0; e < E / 2; ++e) {
      const float keep = b1 ? c1[e + E / 2] : c1[e];
      const float send = b1 ? c1[e] : c1[e + E / 2];
      c2[e] = keep + dpp<kDppQuadXor2>(send);
    }
    float res[E / 4];
#pragma unroll
    for (int e = 0; e < E / 4; ++e) {
      const float keep = b0 ? c2[e + E / 4] : c2[e];
      const float send = b0 ? c2[e] : c2[e + E / 4];
      res[e] = keep + dpp<kDppQuadXor1>(send);
    }
    float lsum[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = row16_sum(l[r]);

    const int hl = (b3 ? 2 : 0) + (b2 ? 1 : 0);
    const float my_l = hl == 0 ? lsum[0] : hl == 1 ? lsum[1] : hl == 2 ? lsum[2] : lsum[3];
    const float my_m = hl == 0 ? m[0] : hl == 1 ? m[1] : hl == 2 ? m[2] : m[3];
    if (hl < nh) {
      const int h = hkv * prm.G + hg * 4 + hl;
      const int d0 = g * E + (b1 ? E / 2 : 0) + (b0 ? E / 4 : 0);
      if (nparts == 1) {
        const float inv = 1.0f / my_l;
        T* dst = static_cast<T*>(prm.out) + ((int64_t)b * prm.Hq + h) * D + d0;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < E / 4; e += 2)
            *reinterpret_cast<uint32_t*>(dst + e) = pack_bf16(res[e] * inv, res[e + 1] * inv);
        } else {
#pragma unroll
          for (int e = 0; e < E / 4; ++e) dst[e] = res[e] * inv;
        }
      } else {
        const int64_t slot = ((int64_t)b * prm.Hq + h) * prm.max_parts + part;
        float* dst = prm.o + slot * D + d0;
#pragma unroll
        for (int e = 0; e < E / 4; ++e) dst[e] = res[e];
        if (g == 0 && !b1 && !b0) {
          prm.ml[slot * 2 + 0] = my_m;
          prm.ml[slot * 2 + 1] = my_l;
        }
      }
    }
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

template <typename T, int D>
hipError_t launch_typed(const DecodeParams& prm, int B, int64_t max_items, hipStream_t stream,
                        hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t want = (max_items + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const unsigned blocks = (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_partition_kernel<T, D>), dim3(blocks), dim3(64 * kWavesPerBlock), 0,
                     stream, prm);
  if (ev1) {
    const hipError_t e = hipEventRecord(ev1, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(prm.Hq, B), dim3(64), 0, stream, prm);
  return hipGetLastError();
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
  if (a.dtype == kBF16) {
    if (a.head_dim == 128) return launch_typed<bf16_bits, 128>(prm, a.num_seqs, max_items, stream, ev0, ev1);
    return launch_typed<bf16_bits, 64>(prm, a.num_seqs, max_items, stream, ev0, ev1);
  }
  if (a.head_dim == 128) return launch_typed<float, 128>(prm, a.num_seqs, max_items, stream, ev0, ev1);
  return launch_typed<float, 64>(prm, a.num_seqs, max_items, stream, ev0, ev1);
}

}  // namespace pa
