// Device code of the varlen / chunked prefill attention kernel (prefill.hip),
// shared with the mixed-batch kernel (mixed.hip): tile gathers through the
// block table, the 64-key tile products and the whole computation of one
// (request, q tile, KV head) item.  The design is described in prefill.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {
namespace pre {

constexpr int kRows = 256;     // rows (chunk token x query head) per work item
constexpr int kTK = 64;        // keys per tile
constexpr int kThreads = 512;  // 8 waves, 32 rows each
constexpr int kIdCap = kPrefillMaxBlocks;  // block ids an item keeps in LDS

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int tokens_per_tile(int G) { return kRows / G; }

inline int64_t max_prefill_items(int num_seqs, int64_t num_q_tokens, int G) {
  const int TQ = tokens_per_tile(G);
  return (num_q_tokens + TQ - 1) / TQ + num_seqs;
}

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// ---------------------------------------------------------------------------
// Plan: the (request, q tile) items, requests ordered by their total number of
// key tiles (largest first; counting sort, ties in any order -- each item is
// computed independently, so the order never changes a result), and each
// request's q tiles from the last (largest causal extent) to the first, so
// that the items sharing a request's keys run at the same time.
// ---------------------------------------------------------------------------
constexpr int kBuckets = 1024;
constexpr int kPlanThreads = 1024;
constexpr int kXcds = 8;            // queues: one per XCD of the MI355X
constexpr int kHeaderBytes = 1024;
constexpr int kCounterStride = 32;  // uint32 words between queue counters (128-byte lines)
constexpr int kEntryCountWord = kHeaderBytes / 4 - 1;

__device__ __forceinline__ bool chunk_ok(const int32_t* __restrict__ cu, int b, int T, int L,
                                         int num_q_tokens) {
  return T > 0 && T <= L && cu[b] >= 0 && cu[b + 1] <= num_q_tokens;
}

// Key tiles of all q tiles of a chunk of T tokens over a prefix of L - T.
__device__ __forceinline__ int chunk_work(int T, int L, int TQ) {
  int w = 0;
  for (int t0 = 0; t0 < T; t0 += TQ) w += (L - T + min(T, t0 + TQ) + kTK - 1) / kTK;
  return w;
}

// Exclusive scan of one value per thread over a kPlanThreads block.
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int t = lane < kPlanThreads / 64 ? wave_tot[lane] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(t, d);
      if (lane >= d) t += y;
    }
    if (lane < kPlanThreads / 64) wave_tot[lane] = t;  // inclusive totals
  }
  __syncthreads();
  return x - v + (wv > 0 ? wave_tot[wv - 1] : 0);
}

struct PrefillParams {
  const bf16_bits* q;
  const char* kc;
  const char* vc;
  const int32_t* cu;
  const int32_t* bt;
  const int32_t* lens;
  bf16_bits* out;
  const uint32_t* hdr;
  uint32_t* counter;
  const int2* items;
  float scale_log2;
  int Hq, Hkv, G, TQ, P, N, M, cap;
  uint32_t div_m, div_l;  // pos / P = (mulhi(pos, div_m) + pos) >> div_l for 0 <= pos < 2^31
  uint32_t row_bytes;     // H_kv * D * element bytes: one token's row of the pool
  const float* k_scale;   // fp8 pools: per-KV-head scales
  const float* v_scale;
};

// Exact unsigned division by the block size with a precomputed multiplier
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): l = ceil(log2 P), m = ceil(2^(32+l) / P) - 2^32.
__device__ __forceinline__ int div_block(const PrefillParams& p, int pos) {
  return (int)((__umulhi((uint32_t)pos, p.div_m) + (uint32_t)pos) >> p.div_l);
}

// LDS of one workgroup: two K / V tile buffers (row-major) and the item's
// block ids.  Both row strides are an odd multiple of 32 bytes modulo 256:
// measured on gfx950, the K operand reads (16 rows x 16 bytes per quarter
// wave) then run without bank conflicts (a 16-byte pad leaves them 2-way
// conflicted), and so do the transposing V reads and the row stores.
template <int D>
struct __attribute__((aligned(16))) PrefillLds {
  static constexpr int KST = D + 16;  // K row stride (elements)
  static constexpr int VST = D + 16;  // V row stride (elements)
  bf16_bits k[2][kTK * KST];
  bf16_bits v[2][kTK * VST];
  int32_t ids[kIdCap];
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// gfx950's transposing LDS read: within each 16-lane group, lane l receives
// element l % 4 of the 8-byte chunks addressed by lanes l / 4, 4 + l / 4,
// 8 + l / 4 and 12 + l / 4 of the group.
__device__ __forceinline__ u32x2_t lds_read_tr16(const bf16_bits* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
}

// One tile's gathers in flight, held in registers between the global loads
// and the LDS stores.  Waves 0-3 gather K and waves 4-7 gather V, D/32
// 16-byte pieces per thread: piece e = u + 256 x of thread u is key e / (D/8),
// elements 8 (e % (D/8)) .. + 7.  ok: bit x set when the key of load x is
// visible and its block id valid.
// fp8 pools: the same pieces as 8-byte loads of E4M3 codes, widened to fp16
// (the values the codes encode) when stored.
template <bool kF8>
struct TileSet {
  typedef typename std::conditional<kF8, u32x2_t, u32x4_t>::type LT;
  LT k[4];
  uint32_t ok;
};

// Gathers of one tile.  Every load is issued unconditionally: a key past kmax
// or with an out-of-range block id reads the head's slice of row 0 instead --
// always in bounds -- and is zeroed when the tile is stored.  The block ids of
// the thread's 4 keys are read from LDS first, all together, so the LDS round
// trip is paid once per tile.  The tile is stored row-major, K and V alike.
template <int D, bool kWide, bool kF8>
__device__ __forceinline__ void load_tile(const PrefillParams& p, const PrefillLds<D>& s, int hkv, int k0,
                                          int kmax, TileSet<kF8>& r) {
  typedef typename TileSet<kF8>::LT LT;
  constexpr int EB = kF8 ? 1 : 2;  // pool bytes per element
  typedef typename std::conditional<kWide, uint64_t, uint32_t>::type O;
  constexpr int CPR = D / 8;
  constexpr int NK = D / 32;
  const int tid = threadIdx.x;
  const bool kw = uniform(tid >> 8) == 0;  // waves 0-3: K, waves 4-7: V
  const int u = tid & 255;
  int pos[NK], off[NK], blk[NK];
#pragma unroll
  for (int x = 0; x < NK; ++x) pos[x] = k0 + (u + 256 * x) / CPR;
#pragma unroll
  for (int x = 0; x < NK; ++x) {
    const int jb = div_block(p, pos[x] < kmax ? pos[x] : 0);
    off[x] = pos[x] - jb * p.P;
    blk[x] = s.ids[jb];
  }
  const O head = (O)(hkv * D * EB);
  r.ok = 0;
  const char* base = kw ? p.kc : p.vc;
#pragma unroll
  for (int x = 0; x < NK; ++x) {
    const bool ok = pos[x] < kmax && blk[x] >= 0 && blk[x] < p.N;
    const O o = (ok ? ((O)blk[x] * (O)p.P + (O)off[x]) * (O)p.row_bytes : (O)0) + head +
                (O)(8 * EB * ((u + 256 * x) % CPR));
    r.ok |= (ok ? 1u : 0u) << x;
    r.k[x] = *reinterpret_cast<const LT*>(base + o);
  }
}

template <int D, bool kF8>
__device__ __forceinline__ void store_tile(PrefillLds<D>& s, int buf, TileSet<kF8>& r_in) {
  constexpr int CPR = D / 8;
  constexpr int NK = D / 32;
  const int tid = threadIdx.x;
  const bool kw = uniform(tid >> 8) == 0;
  const int u = tid & 255;
  const uint32_t all = (1u << NK) - 1u;
  if (__builtin_amdgcn_readfirstlane((int)(__ballot(r_in.ok != all) != 0))) {
#pragma unroll
    for (int x = 0; x < NK; ++x)
      if (!((r_in.ok >> x) & 1u)) r_in.k[x] = typename TileSet<kF8>::LT{};
  }
  bf16_bits* dst = kw ? s.k[buf] : s.v[buf];
  const int stride = kw ? PrefillLds<D>::KST : PrefillLds<D>::VST;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    u32x4_t w;
    if constexpr (kF8) w = e4m3x8_to_f16(r_in.k[i]);
    else w = r_in.k[i];
    const int e = u + 256 * i, key = e / CPR, c = e % CPR;
    *reinterpret_cast<u32x4_t*>(&dst[key * stride + 8 * c]) = w;
  }
}

// Softmax reference max moves only when a score exceeds it by more than this
// (log2 units): probabilities stay below 2^8, and rescaling is rare.
constexpr float kRescaleSlack = 8.0f;

// Per-wave state of one item: 32 rows (two blocks of 16), one per lane column.
template <int D>
struct RowState {
  static constexpr int NI = D / 32;
  static constexpr int NDB = D / 16;
  u32x4_t q[2][NI];  // Q^T operand of each row block
  int pos[2];        // absolute position of the lane's row (-1: no row)
  float m[2];
  f32x4_t l[2];  // row sums, accumulated by MFMA (every component holds the sum)
  f32x4_t o[NDB][2];  // O^T: lane (n, g) holds d = 16 db + 4 g + j of row n
};

// One 64-key tile for this wave's 32 rows: S^T = K Q^T, online softmax, O^T += V^T P^T.
// 16x16x32 products on bf16 operands, or on fp16 ones for fp8 pools.
template <bool kF8>
__device__ __forceinline__ f32x4_t mma32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  if constexpr (kF8)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

template <bool kF8>
__device__ __forceinline__ uint32_t pack_p(float lo, float hi) {
  if constexpr (kF8) return pack_f16(lo, hi);
  else return pack_bf16(lo, hi);
}

// Operand reads of one staged tile pair, for lane (n, g) of the wave:
//   k(kb, i):   K rows kb*16 + n, elements 32 i + 8 g .. + 7 (the A operand
//               of S^T = K Q^T, k-step i);
//   v(db, ks):  the V^T A operand of O^T += V^T P^T for output dims 16 db ..
//               + 15 and keys 32 ks + 4 g + (0..3), 32 ks + 16 + 4 g + (0..3),
//               from two transposing reads (lane n of the group addresses row
//               n / 4 of a 4-row slice, elements 4 (n % 4) .. + 3).
// PaddedTiles: row-major tiles with padded rows (register-staged path).
template <int D>
struct PaddedTiles {
  const bf16_bits* kt;
  const bf16_bits* vt;
  __device__ __forceinline__ PaddedTiles(const PrefillLds<D>& s, int buf) : kt(s.k[buf]), vt(s.v[buf]) {}
  __device__ __forceinline__ u32x4_t k(int kb, int i) const {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    return *reinterpret_cast<const u32x4_t*>(&kt[(kb * 16 + n) * PrefillLds<D>::KST + 32 * i + 8 * g]);
  }
  __device__ __forceinline__ u32x4_t v(int db, int ks) const {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const bf16_bits* a = &vt[(32 * ks + 4 * g + (n >> 2)) * PrefillLds<D>::VST + 16 * db + 4 * (n & 3)];
    const u32x2_t lo = lds_read_tr16(a), hi = lds_read_tr16(a + 16 * PrefillLds<D>::VST);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }
};

template <int D, bool kF8, class Tiles>
__device__ __forceinline__ void attend_tile(const Tiles& tl, int k0, float scale_log2, RowState<D>& st) {
  constexpr int NI = RowState<D>::NI, NDB = RowState<D>::NDB;
  const int lane = lane_id();
  const int g = lane >> 4;
  f32x4_t sc[4][2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    sc[kb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sc[kb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u32x4_t av = tl.k(kb, i);
      sc[kb][0] = mma32<kF8>(av, st.q[0][i], sc[kb][0]);
      sc[kb][1] = mma32<kF8>(av, st.q[1][i], sc[kb][1]);
    }
  }

  u32x4_t pop[2][2];  // [rb][k-step]: P^T operand, 8 bf16
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    // causal mask, only where this row block's last key position is inside
    // the tile (keys past a row's position get -inf)
    // (the lane's keys are kb*16 + 4g + j, kb, j < 4: all visible when lim >= 51)
    const int lim = st.pos[rb] - k0 - 4 * g;  // key kb*16 + 4g + j is visible when kb*16 + j <= lim
    if (__builtin_amdgcn_readfirstlane((int)(__ballot(lim < 3 * 16 + 3) != 0))) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[kb][rb][j] = kb * 16 + j <= lim ? sc[kb][rb][j] : -INFINITY;
    }
    // max of the raw scores (scale_log2 > 0), in log2 units after scaling
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, sc[kb][rb][j]);
    tmax = max_over_rows(tmax);
    tmax *= scale_log2;
    const bool move = tmax > st.m[rb] + kRescaleSlack;
    if (__builtin_amdgcn_readfirstlane((int)(__ballot(move) != 0))) {
      const float alpha = (move && st.m[rb] != -INFINITY) ? fast_exp2(st.m[rb] - tmax) : 1.0f;
      if (move) st.m[rb] = tmax;
      st.l[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) st.o[db][rb] *= alpha;
    }
    const float nm = st.m[rb] == -INFINITY ? 0.f : -st.m[rb];
    float pv[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pv[kb][j] = fast_exp2(fmaf(sc[kb][rb][j], scale_log2, nm));
      }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pop[rb][ks] = u32x4_t{pack_p<kF8>(pv[2 * ks][0], pv[2 * ks][1]), pack_p<kF8>(pv[2 * ks][2], pv[2 * ks][3]),
                            pack_p<kF8>(pv[2 * ks + 1][0], pv[2 * ks + 1][1]),
                            pack_p<kF8>(pv[2 * ks + 1][2], pv[2 * ks + 1][3])};
    // row sums of the probabilities as products with a ones operand
    const uint32_t one2 = kF8 ? 0x3C003C00u : 0x3F803F80u;
    const u32x4_t ones = {one2, one2, one2, one2};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) st.l[rb] = mma32<kF8>(ones, pop[rb][ks], st.l[rb]);
  }
  // k-slots 0..3 of step ks are keys 32 ks + 4 g + j, slots 4..7 keys 32 ks + 16 + 4 g + j
  u32x4_t va[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) va[db][ks] = tl.v(db, ks);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      st.o[db][0] = mma32<kF8>(va[db][ks], pop[0][ks], st.o[db][0]);
      st.o[db][1] = mma32<kF8>(va[db][ks], pop[1][ks], st.o[db][1]);
    }
  }
}

template <int D, bool kF8>
__device__ __forceinline__ void attend(const PrefillLds<D>& s, int buf, int k0, float scale_log2, int wave_max,
                                       RowState<D>& st) {
  if (k0 > wave_max) return;  // every row of this wave is causally done
  attend_tile<D, kF8>(PaddedTiles<D>(s, buf), k0, scale_log2, st);
}

// The part of an item both tile pipelines share: its geometry, its block
// ids copied to LDS, the wave's rows and their queries loaded, and (at the
// end) the normalised outputs stored.
struct ItemGeo {
  int cu0;       // packed row of chunk token 0
  int start;     // position of chunk row 0
  int t0;        // first chunk token of the q tile
  int kmax;      // keys 0 .. kmax-1 are visible to some row
  int nkt;       // key tiles
  int wave_max;  // largest position of this wave's rows (-1: none)
};

template <int D, bool kF8>
__device__ __forceinline__ ItemGeo begin_item(const PrefillParams& p, int32_t* ids, int b, int qt, int hkv,
                                              RowState<D>& st) {
  constexpr int NI = RowState<D>::NI, NDB = RowState<D>::NDB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  ItemGeo ig;
  ig.cu0 = p.cu[b];
  const int T = p.cu[b + 1] - ig.cu0;
  const int L = clamp_len(p.lens[b], p.cap);
  ig.start = L - T;
  ig.t0 = qt * p.TQ;
  const int nt = min(p.TQ, T - ig.t0);
  ig.kmax = ig.start + ig.t0 + nt;
  ig.nkt = (ig.kmax + kTK - 1) / kTK;
  const int32_t* __restrict__ bt_row = p.bt + (int64_t)b * p.M;
  const int nblk = div_block(p, ig.kmax - 1) + 1;  // kmax <= cap = M * P, so nblk <= M
  for (int i = tid; i < nblk; i += kThreads) ids[i] = bt_row[i];

  int wave_max = -1;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 32 * w + 16 * rb + n;
    const int hl = r / p.TQ, tl = r - hl * p.TQ;
    const bool ok = hl < p.G && tl < nt;
    st.pos[rb] = ok ? ig.start + ig.t0 + tl : -1;
    const int64_t qrow = ((int64_t)(ig.cu0 + ig.t0 + tl) * p.Hq + hkv * p.G + hl) * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      st.q[rb][i] = ok ? *reinterpret_cast<const u32x4_t*>(p.q + qrow + 32 * i + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
      if constexpr (kF8) {  // bf16 query -> fp16 operand (exact inside the fp16 range)
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) st.q[rb][i][w2] = pack_f16(bf16_lo(st.q[rb][i][w2]), bf16_hi(st.q[rb][i][w2]));
      }
    }
    if (ok) wave_max = max(wave_max, st.pos[rb]);
    st.m[rb] = -INFINITY;
    st.l[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.o[db][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wave_max = max(wave_max, __shfl_xor(wave_max, off));
  ig.wave_max = uniform(wave_max);
  return ig;
}

// Normalise and store: lane holds O^T[d = 16db + 4g + j][row n].
template <int D>
__device__ __forceinline__ void finish_item(const PrefillParams& p, const ItemGeo& ig, int hkv, float vmul,
                                            const RowState<D>& st) {
  constexpr int NDB = RowState<D>::NDB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = st.l[rb][0];
    if (st.pos[rb] < 0) continue;
    const int r = 32 * w + 16 * rb + n;
    const int hl = r / p.TQ, tl = r - hl * p.TQ;
    const float inv = vmul / lt;
    bf16_bits* dst = p.out + ((int64_t)(ig.cu0 + ig.t0 + tl) * p.Hq + hkv * p.G + hl) * D + 4 * g;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2_t v = {pack_bf16(st.o[db][rb][0] * inv, st.o[db][rb][1] * inv),
                         pack_bf16(st.o[db][rb][2] * inv, st.o[db][rb][3] * inv)};
      *reinterpret_cast<u32x2_t*>(dst + 16 * db) = v;
    }
  }
}

// One item: rows of q tile qt of request b's chunk for KV head hkv, every
// key tile of its causal extent, normalised outputs stored.  All threads of
// the workgroup take part (barriers inside); on entry no thread may still be
// reading the LDS buffers of a previous item.
template <int D, bool kWide, bool kF8>
__device__ __forceinline__ void prefill_item(const PrefillParams& p, PrefillLds<D>& lds, int b, int qt, int hkv) {
  const int w = uniform(threadIdx.x >> 6);
  RowState<D> st;
  const ItemGeo ig = begin_item<D, kF8>(p, lds.ids, b, qt, hkv, st);
  const int kmax = ig.kmax, nkt = ig.nkt, wave_max = ig.wave_max;
  __syncthreads();  // block ids visible

  // fp8 pools: value(code) * scale, staged as value(code)
  const float sl2 = kF8 ? p.scale_log2 * p.k_scale[hkv] : p.scale_log2;
  const float vmul = kF8 ? p.v_scale[hkv] : 1.0f;

  // pipeline: tile j travels in register set j & 1 and LDS buffer j & 1
  TileSet<kF8> ra, rb;
  load_tile<D, kWide, kF8>(p, lds, hkv, 0, kmax, ra);
  if (nkt > 1) load_tile<D, kWide, kF8>(p, lds, hkv, kTK, kmax, rb);
  store_tile<D, kF8>(lds, 0, ra);
  if (nkt > 2) load_tile<D, kWide, kF8>(p, lds, hkv, 2 * kTK, kmax, ra);
  __syncthreads();
  // waves 4-7 stage the next tile before their products, waves 0-3 after, so
  // the two waves of a SIMD are out of phase
  const bool early = w >= 4;
  for (int kt = 0; kt < nkt; kt += 2) {
    if (early && kt + 1 < nkt) {
      store_tile<D, kF8>(lds, 1, rb);
      if (kt + 3 < nkt) load_tile<D, kWide, kF8>(p, lds, hkv, (kt + 3) * kTK, kmax, rb);
    }
    attend<D, kF8>(lds, 0, kt * kTK, sl2, wave_max, st);
    if (!early && kt + 1 < nkt) {
      store_tile<D, kF8>(lds, 1, rb);
      if (kt + 3 < nkt) load_tile<D, kWide, kF8>(p, lds, hkv, (kt + 3) * kTK, kmax, rb);
    }
    __syncthreads();
    if (kt + 1 >= nkt) break;
    if (early && kt + 2 < nkt) {
      store_tile<D, kF8>(lds, 0, ra);
      if (kt + 4 < nkt) load_tile<D, kWide, kF8>(p, lds, hkv, (kt + 4) * kTK, kmax, ra);
    }
    attend<D, kF8>(lds, 1, (kt + 1) * kTK, sl2, wave_max, st);
    if (!early && kt + 2 < nkt) {
      store_tile<D, kF8>(lds, 0, ra);
      if (kt + 4 < nkt) load_tile<D, kWide, kF8>(p, lds, hkv, (kt + 4) * kTK, kmax, ra);
    }
    __syncthreads();
  }
  finish_item<D>(p, ig, hkv, vmul, st);
}

}  // namespace pre
}  // namespace pa
