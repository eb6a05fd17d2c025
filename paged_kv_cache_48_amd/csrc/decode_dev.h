// Device code of the paged decode attention kernels (decode.hip), shared with
// the mixed-batch kernel (mixed.hip): the work list and its in-kernel plan,
// the queue claims, tile gathers, the stream of partition items a wave
// computes, and the split-context merge.  The design is described in
// decode.hip.
#pragma once

#include <math.h>
#include <stdlib.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {
namespace dec {

constexpr int kTile = 16;  // tokens per tile (bf16, fp32); the plan counts tails in these units

constexpr int kWavesPerBlock = 4;
constexpr int kMaxStaticRounds = 64;  // static items per wave: one descriptor per lane
constexpr int kDynamicRounds = 0;     // whole rounds of full partitions handed out by the queues

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Work-queue header in the workspace: kQueues 64-bit counters, each on its
// own 128-byte line, and the plan kernel's counts in the last words.  A
// counter holds a tag in bits 24..63 and the count in bits 0..23: the tag
// names the launch that reset it (zero when the plan kernel did), so a claim
// that lands on a counter left by an earlier call, or on whatever else the
// workspace held, is recognised as such and retried.
constexpr int kQueues = 8;  // one per XCD of the MI355X
constexpr int kCounterStride = 16;  // uint64 words between counters
constexpr int kHeaderBytes = 1024;
constexpr int kItemCountWord = kHeaderBytes / 4 - 1;
constexpr int kFullCountWord = kHeaderBytes / 4 - 2;  // items that are full partitions
constexpr int kQueueCountWord = kHeaderBytes / 4 - 3;  // queues in use
// Sticky status bits: a wave that gives up waiting on a queue (see claim)
// ORs in kGaveUpDecode, a mixed workgroup that gives up on a prefill queue
// kGaveUpPrefill.  Only pa_workspace_status reads and clears the word.
constexpr int kStatusWord = kHeaderBytes / 4 - 4;
static_assert(kStatusWord * 4 == (int)kStatusWordOffset, "status word offset");
constexpr uint32_t kGaveUpDecode = 1u;
constexpr uint32_t kGaveUpPrefill = 2u;
constexpr int kCountBits = 24;
constexpr int64_t kMaxQueueItems = (int64_t)1 << kCountBits;  // claims per counter
constexpr int64_t kMaxWaves = 256 * 32;  // resident waves of a launch, at most

struct DecodeLayout {
  int64_t max_parts;
  size_t hdr, items, ml, o, total;
};

inline DecodeLayout decode_layout(int B, int Hq, int D, int P, int M) {
  DecodeLayout L;
  L.max_parts = ((int64_t)M * P + kPartTokens - 1) / kPartTokens;
  size_t off = 0;
  L.hdr = off;
  off += kHeaderBytes;
  L.items = off;
  off = align256(off + sizeof(i32x4_t) * (size_t)B * L.max_parts);
  L.ml = off;
  off = align256(off + sizeof(float) * 4 * (size_t)B * Hq * L.max_parts);  // (max, sum, scale, -)
  L.o = off;
  off = align256(off + sizeof(float) * (size_t)B * Hq * L.max_parts * D);
  L.total = off;
  return L;
}

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

constexpr int kTileBuckets = kPartTokens / 16;  // bucket k >= 1: tails of k tiles; bucket 0: full
constexpr int kPlanThreads = 1024;

// ---------------------------------------------------------------------------
// fp8 pools: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits), one fp32 scale per KV head for K and for V.
struct fp8_e4m3 {
  uint8_t bits;
};

// Element type of q and out: the pool's, except bf16 for fp8 pools.
template <typename T>
struct QType {
  typedef T type;
};
template <>
struct QType<fp8_e4m3> {
  typedef bf16_bits type;
};

// ---------------------------------------------------------------------------
// Tile geometry.  A tile is TT consecutive tokens of one KV head (16; 32 for
// fp8 pools).  Lane l loads 16-byte piece l % CPR of the head's row slice for
// tokens (l / CPR) * TPL + j, j < TPL, so groups of CPR lanes read whole
// contiguous row slices.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct Geo {
  // fp8 pools: tiles of 32 tokens (the bytes of a 16-token bf16 tile), staged
  // as the codes themselves and widened to the fp16 values they encode when an MFMA
  // operand is read
  static constexpr bool kFp8 = std::is_same<T, fp8_e4m3>::value;
  static constexpr bool kBf16 = std::is_same<T, bf16_bits>::value;
  static constexpr bool kHalf = kBf16 || kFp8;     // 16-bit q and out (fp16 MFMAs for fp8)
  static constexpr int TT = kFp8 ? 32 : 16;        // tokens per tile
  static constexpr int ROWB = D * (int)sizeof(T);  // bytes of one head's row slice (pool and LDS)
  static constexpr int GROWB = ROWB;
  static constexpr int CPR = ROWB / 16;            // 16-byte pieces per row slice
  static constexpr int LOADB = 16;                 // pool bytes a lane loads per token
  static constexpr int TPL = TT * CPR / 64;        // tokens per lane per tile
  static constexpr int KST = ROWB + 16;            // LDS row stride of K (and of V unless bf16)
  static constexpr int VTS = 40;                   // LDS row stride of transposed bf16 V: 16 tokens + pad
  static constexpr int KBYTES = TT * KST;
  static constexpr int VBYTES = kBf16 ? D * VTS : TT * KST;
  static constexpr int LDS_PER_WAVE = KBYTES + VBYTES;
  static constexpr int NQ = kHalf ? D / 32 : D / 4;  // QK MFMA steps over the head dimension
  static constexpr int NQV = kHalf ? NQ : NQ / 4;    // 16-byte Q pieces per lane
};

// Byte offsets into the pool: 32-bit when the pool is under 4 GiB (one VGPR
// per address, added to a scalar base), 64-bit otherwise.
template <bool kWide>
struct Off {
  typedef typename std::conditional<kWide, uint64_t, uint32_t>::type type;
};

template <typename T, int D>
struct TileRegs {
  typedef u32x4_t LT;  // one lane's load per token
  LT k[Geo<T, D>::TPL];
  LT v[Geo<T, D>::TPL];
  uint32_t ok;  // bit j: token j of this lane is inside the partition with a valid block id
};

struct PoolView {
  const char* k;
  const char* v;
  uint32_t row_bytes;   // H_kv * D * elem: one token's row over all KV heads
};

struct DecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* lens;
  void* out;
  const uint32_t* hdr;
  unsigned long long* counter;
  const i32x4_t* items;
  float* ml;
  float* o;
  float scale_log2;
  int Hq, Hkv, G, n_hg, P, p_shift, N, M, cap, max_parts;
  int gw, gs;       // query heads per group (4, 8 or 16) and its log2
  int dyn_rounds;  // full rounds of full partitions left to the queues
  int nq;          // queues in use (at most kQueues); 0: as the plan chose
  int B;
  const float* k_scale;  // fp8 pools: per-KV-head scales (null otherwise)
  const float* v_scale;
  int self_plan;   // 1: the workgroups plan (B <= kSelfPlanMax); 0: the plan kernel did
  unsigned long long salt;  // per call; mixed into the counters' tag
  // mixed batches (kRowMap): request b is a decode when its chunk
  // cu[b] .. cu[b+1] is one token, whose row of q and out is cu[b]; other
  // requests have no decode items.  Null for plain decode (row b).
  const int32_t* cu;
  int num_q_tokens;
  // decode with append: request b's new token, at position L_b - 1, is row b
  // of knew / vnew [B, H_kv, D] (the pool's element type; fp8 pools: bf16
  // values, or fp32 when new_f32, quantised with the head's scale as the
  // scatter does).  The last partition's items take it from there instead of
  // the pool, and those of query-head group 0 write it to its slot.
  const void* knew;
  const void* vnew;
  int new_f32;
  uint32_t* status;  // the header's kStatusWord
  int force_giveup;  // test knob: every claim sees a stale counter and gives up at once
};

// Query heads per item: the G query heads that share a KV head take
// columns of one 16-column MFMA operand, so a group of up to 16 (8 per head
// of a pair) reads each KV slice once; larger G splits into groups of 16.
// The width is a power of two (4, 8 or 16) so a column's head is a shift
// and a mask of its index.
inline void set_query_groups(DecodeParams& prm, int G, int HP) {
  const int cols = 16 / HP;
  prm.gw = G <= 4 ? 4 : (G <= 8 || cols == 8) ? 8 : 16;
  prm.gs = prm.gw == 4 ? 2 : prm.gw == 8 ? 3 : 4;
  prm.G = G;
  prm.n_hg = (G + prm.gw - 1) / prm.gw;
}

// One work item, wave-uniform (scalar registers).
struct Item {
  int b, part, L, nparts;  // request, partition, visible tokens, partitions of the request
  int row;                 // row of q and out
  int hkv, hg, nh;         // KV head, group of query heads, valid heads in the group
  int tok0, tok_end, ntiles, blk0, nblk;
  float sl2, vmul;         // score factor (log2 units) and output factor (fp8 scales folded in)
};

template <bool kRowMap, int TT, int HP>
__device__ __forceinline__ Item make_item(const DecodeParams& prm, i32x4_t d, uint32_t f, uint32_t per_item) {
  Item it;
  it.b = uniform(d[0]);
  it.row = kRowMap ? uniform(prm.cu[it.b]) : it.b;
  it.part = uniform(d[1]);
  it.L = uniform(d[2]);
  it.nparts = uniform(d[3]);
  const int rem = (int)(f % per_item);
  it.hkv = rem / prm.n_hg;
  it.hg = rem - it.hkv * prm.n_hg;
  it.nh = min(prm.gw, prm.G - it.hg * prm.gw);
  it.tok0 = it.part * kPartTokens;
  it.tok_end = min(it.L, it.tok0 + kPartTokens);
  it.ntiles = (it.tok_end - it.tok0 + TT - 1) / TT;
  int last;
  if (prm.p_shift >= 0) {
    it.blk0 = it.tok0 >> prm.p_shift;
    last = (it.tok_end - 1) >> prm.p_shift;
  } else {
    it.blk0 = it.tok0 / prm.P;
    last = (it.tok_end - 1) / prm.P;
  }
  it.nblk = last - it.blk0 + 1;
  // fp8 pools hold value(code) * scale; the operands are value(code) in fp16
  it.sl2 = prm.k_scale ? prm.scale_log2 * prm.k_scale[it.hkv] : prm.scale_log2;
  it.vmul = prm.v_scale ? prm.v_scale[it.hkv] : 1.0f;
  if constexpr (HP == 2) {
    // head pairs: the factors are per column (column n of the lane belongs
    // to KV head 2 hkv + (n / gw) % 2)
    const int hs = 2 * it.hkv + (((lane_id() & 15) >> prm.gs) & 1);
    if (prm.k_scale) it.sl2 = prm.scale_log2 * prm.k_scale[hs];
    if (prm.v_scale) it.vmul = prm.v_scale[hs];
  }
  return it;
}

// The item's block ids, lane i of register r holding entry blk0 + 64r + i.
// The index is clamped so every lane loads (no divergent load to wait on).
template <int NR>
__device__ __forceinline__ void load_ids(const DecodeParams& prm, const Item& it, int (&ids)[NR]) {
  const int lane = lane_id();
  const int32_t* row = prm.bt + (int64_t)it.b * prm.M + it.blk0;
#pragma unroll
  for (int r = 0; r < NR; ++r) ids[r] = row[min(64 * r + lane, it.nblk - 1)];
}

// Q^T operand: column n = query head of the group (heads past the group's
// last read head 0's row; their columns are never stored).
// HP = 2 (adjacent KV heads taken in pairs, read as one head of dimension D:
// 64-dim bf16 or fp8 heads as D = 128, 128-dim fp8 heads as D = 256): columns
// 0 .. gw-1 are the group's query heads of the first KV head of the pair,
// columns gw .. 2gw-1 those of the second.  Each column's query is its own head's D / 2
// dimensions, in both halves of the operand: the score products over the
// first and the second half go to separate accumulators, and each column
// keeps the one of its own head.
template <typename T, int D, int HP>
__device__ __forceinline__ void load_q(const DecodeParams& prm, const Item& it, u32x4_t (&qv)[Geo<T, D>::NQV]) {
  using Gm = Geo<T, D>;
  typedef typename QType<T>::type QT;
  const int lane = lane_id();
  const int n = lane & 15, g = lane >> 4;
  if constexpr (HP == 2) {
    static_assert(Gm::kHalf && (D == 128 || (Gm::kFp8 && D == 256)), "head pairs");
    const int hi = (n >> prm.gs) & 1, c = n & (prm.gw - 1);
    const bool col = n < 2 * prm.gw && c < it.nh;
    const int h = (2 * it.hkv + hi) * prm.G + it.hg * prm.gw + (col ? c : 0);
    const QT* qrow = static_cast<const QT*>(prm.q) + ((int64_t)it.row * prm.Hq + h) * (D / 2);
#pragma unroll
    for (int i = 0; i < Gm::NQV / 2; ++i) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + 32 * i + 8 * g);
      if constexpr (Gm::kFp8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) qv[i][w] = pack_f16(bf16_lo(x[w]), bf16_hi(x[w]));
      } else {
        qv[i] = x;
      }
      qv[i + Gm::NQV / 2] = qv[i];
    }
    return;
  }
  const int h = it.hkv * prm.G + it.hg * prm.gw + (n < it.nh ? n : 0);
  const QT* qrow = static_cast<const QT*>(prm.q) + ((int64_t)it.row * prm.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < Gm::NQV; ++i) {
    if constexpr (Gm::kFp8) {
      // bf16 query -> fp16 operand (exact inside the fp16 range)
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + 32 * i + 8 * g);
#pragma unroll
      for (int w = 0; w < 4; ++w) qv[i][w] = pack_f16(bf16_lo(x[w]), bf16_hi(x[w]));
    } else if constexpr (Gm::kBf16) qv[i] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * i + 8 * g);
    else qv[i] = *reinterpret_cast<const u32x4_t*>(qrow + g * (D / 4) + 4 * i);
  }
}

// Descriptor held in lane `r` of a per-lane descriptor register (wave-uniform result).
__device__ __forceinline__ i32x4_t lane_desc(const i32x4_t& d, int r) {
  return i32x4_t{__builtin_amdgcn_readlane(d[0], r), __builtin_amdgcn_readlane(d[1], r),
                 __builtin_amdgcn_readlane(d[2], r), __builtin_amdgcn_readlane(d[3], r)};
}

// Block id of logical block `idx` (relative to the item's first block) for
// a per-lane index: lane crossbar read from the id registers.
template <int NR>
__device__ __forceinline__ int lane_id_lookup(const int (&ids)[NR], int idx) {
  int blk = __builtin_amdgcn_ds_bpermute((idx & 63) << 2, ids[0]);
#pragma unroll
  for (int r = 1; r < NR; ++r) {
    const int v = __builtin_amdgcn_ds_bpermute((idx & 63) << 2, ids[r]);
    if ((idx >> 6) == r) blk = v;
  }
  return blk;
}

// Issues the K/V loads of one tile.  Block ids come from registers, so no
// global load is waited on here (a wait on one would drain the K/V loads
// already in flight, since loads complete in order).  Invalid tokens load the
// head's slice of row 0 (always in range, and cached) and are zeroed when
// staged.  kAligned: the tile lies inside one block (P a multiple of 16).
// kNew (decode with append, bf16): the lanes that load token npos (the new
// token, L - 1) load it from the new rows (knew / vnew: this lane's piece of
// the item's slice of row b) instead of the pool; every lane issues the same
// loads either way.
template <typename T, int D, bool kWide, bool kAligned, int NR, bool kNew = false>
__device__ __forceinline__ void load_tile(const PoolView& pv, const DecodeParams& prm, const Item& it,
                                          const int (&ids)[NR], int tile0, TileRegs<T, D>& r, int npos = -1,
                                          const char* knew = nullptr, const char* vnew = nullptr) {
  using Gm = Geo<T, D>;
  using O = typename Off<kWide>::type;
  const int lane = lane_id();
  const int q = lane / Gm::CPR;
  const int first = tile0 + q * Gm::TPL;  // this lane's first token
  const O lane_off = (O)(it.hkv * Gm::GROWB + Gm::LOADB * (lane % Gm::CPR));
  typedef typename TileRegs<T, D>::LT LT;
  r.ok = 0;
  if constexpr (kAligned) {
    int lb, off;
    if (prm.p_shift >= 0) {
      lb = tile0 >> prm.p_shift;
      off = tile0 & ((1 << prm.p_shift) - 1);
    } else {
      lb = tile0 / prm.P;
      off = tile0 - lb * prm.P;
    }
    int blk = __builtin_amdgcn_readlane(ids[0], lb - it.blk0);
    int loff = off + q * Gm::TPL;  // block offset of this lane's first token
    if constexpr (Gm::TT > 16) {
      // P is a multiple of 16 and a tile spans 32 tokens: the lane's tokens lie
      // in block lb or lb + 1 (at most 256 / P + 1 <= 17 ids of the item)
      const int blk1 = __builtin_amdgcn_readlane(ids[0], min(lb + 1 - it.blk0, 63));
      if (loff >= prm.P) {
        blk = blk1;
        loff -= prm.P;
      }
    }
    const bool bok = blk >= 0 && blk < prm.N;
    const O base = bok ? ((O)blk * (O)prm.P + (O)loff) * (O)pv.row_bytes : (O)0;
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j) {
      const bool ok = bok && first + j < it.tok_end;
      r.ok |= (ok ? 1u : 0u) << j;
      const O e = (ok ? base + (O)j * (O)pv.row_bytes : (O)0) + lane_off;
      if constexpr (kNew) {
        const bool nw = first + j == npos;
        r.k[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(nw ? knew : pv.k + e));
        r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(nw ? vnew : pv.v + e));
      } else {
        r.k[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(pv.k + e));
        r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(pv.v + e));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j) {
      const int pos = first + j;
      int lb, off;
      if (prm.p_shift >= 0) {
        lb = pos >> prm.p_shift;
        off = pos & ((1 << prm.p_shift) - 1);
      } else {
        lb = pos / prm.P;
        off = pos - lb * prm.P;
      }
      const bool in = pos < it.tok_end;
      const int blk = lane_id_lookup<NR>(ids, in ? lb - it.blk0 : 0);
      const bool ok = in && blk >= 0 && blk < prm.N;
      r.ok |= (ok ? 1u : 0u) << j;
      const O e = (ok ? ((O)blk * (O)prm.P + (O)off) * (O)pv.row_bytes : (O)0) + lane_off;
      if constexpr (kNew) {
        const bool nw = pos == npos;
        r.k[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(nw ? knew : pv.k + e));
        r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(nw ? vnew : pv.v + e));
      } else {
        r.k[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(pv.k + e));
        r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const LT*>(pv.v + e));
      }
    }
  }
}

// Registers -> this wave's LDS region: K row-major; V transposed (bf16, d-major
// so a P.V operand is one 8-byte read) or row-major (fp32, and fp8 codes,
// whose P.V operand comes from the byte-transposing LDS read).
template <typename T, int D>
__device__ __forceinline__ void stage_tile(char* lds, TileRegs<T, D>& r_in, bool full) {
  using Gm = Geo<T, D>;
  typedef typename TileRegs<T, D>::LT LT;
  const int lane = lane_id();
  const int c = lane % Gm::CPR, q = lane / Gm::CPR;
  if (!full) {
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j)
      if (!((r_in.ok >> j) & 1u)) {
        r_in.k[j] = LT{};
        r_in.v[j] = LT{};
      }
  }
  TileRegs<T, D>& r = r_in;
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

// stage_tile for the two-tile stream (bf16 pools): the same LDS contents, but
// the registers are only read (a masked token's values are replaced by zeros
// as they are written to LDS).  Only the loads write a register set there, so
// the wait before staging a set covers that set's loads alone and leaves the
// other set's in flight.
template <typename T, int D, bool kMasked>
__device__ __forceinline__ void stage_tile_ro(char* lds, const TileRegs<T, D>& r) {
  using Gm = Geo<T, D>;
  static_assert(Gm::kBf16, "bf16 pools");
  const int lane = lane_id();
  const int c = lane % Gm::CPR, q = lane / Gm::CPR;
  auto okj = [&](int j) { return !kMasked || ((r.ok >> j) & 1u) != 0; };
#pragma unroll
  for (int j = 0; j < Gm::TPL; ++j)
    *reinterpret_cast<u32x4_t*>(lds + (q * Gm::TPL + j) * Gm::KST + 16 * c) =
        okj(j) ? r.k[j] : u32x4_t{0u, 0u, 0u, 0u};
  char* vl = lds + Gm::KBYTES;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int d = 8 * c + 2 * w;
    uint32_t v[Gm::TPL];
#pragma unroll
    for (int j = 0; j < Gm::TPL; ++j) v[j] = okj(j) ? r.v[j][w] : 0u;
    if constexpr (Gm::TPL == 4) {
      const u32x2_t lo = {__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u)};
      const u32x2_t hi = {__builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
      *reinterpret_cast<u32x2_t*>(vl + d * Gm::VTS + 8 * q) = lo;
      *reinterpret_cast<u32x2_t*>(vl + (d + 1) * Gm::VTS + 8 * q) = hi;
    } else {
      static_assert(Gm::TPL == 2, "bf16 tiles hold 2 or 4 tokens per lane");
      *reinterpret_cast<uint32_t*>(vl + d * Gm::VTS + 4 * q) = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
      *reinterpret_cast<uint32_t*>(vl + (d + 1) * Gm::VTS + 4 * q) = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
    }
  }
}

// Orders this wave's LDS stores before its later LDS loads (the wave reads
// what other lanes of the same wave wrote).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Softmax reference max is moved only when a score exceeds it by more than
// this (log2 units), so probabilities stay below 2^8 and the rescale of the
// accumulators is rare; the result does not depend on the reference.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ unsigned long long uniform64(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// The launch's dispatch id: the packet's index on its hardware queue (every
// launch, graph replays included, gets a new one).
extern "C" __device__ unsigned long long llvm_amdgcn_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// Tag of this launch's queue counters: dispatch id, queue address and the
// host's per-call salt, mixed with the splitmix64 finaliser and cut to the
// tag's 40 bits; never zero (zero marks counters the plan kernel reset).
__device__ __forceinline__ unsigned long long launch_tag(unsigned long long salt) {
  unsigned long long x = llvm_amdgcn_dispatch_id() * 0x9E3779B97F4A7C15ull;
  x ^= (unsigned long long)(uintptr_t)__builtin_amdgcn_queue_ptr() ^ salt;
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  x &= (1ull << (64 - kCountBits)) - 1ull;
  return x ? x : 1ull;
}

// Sleeps a claim may wait for workgroup 0 to reset the counters (a few
// atomics of a resident workgroup, so a handful in practice; the bound only
// guarantees that every wave exits).  A wave that reaches it leaves the
// queue's remaining items uncomputed and records that in the status word.
constexpr int kMaxSpins = 1 << 20;

// Takes the next dynamically scheduled item: with nq queues, queue x holds
// flat items f = first_dyn + nq * c + x; a wave starts at its home queue (its
// XCD's, when there are eight) and moves to the next one when that is empty.
// A self-planned launch checks the counter's tag: a counter not yet reset
// for this launch is tried again after a short sleep.  Returns 0xffffffff
// when all queues are empty.
__device__ __forceinline__ uint32_t claim(const DecodeParams& prm, unsigned long long tag, uint32_t nq, uint32_t home,
                                          uint32_t& queue, uint32_t first_dyn, uint32_t total) {
  if (first_dyn >= total) return 0xffffffffu;  // every item is dealt statically
  const int lane = lane_id();
  int spins = 0;
  while (queue < nq) {
    const uint32_t x = (home + queue) % nq;
    unsigned long long old = 0;
    if (lane == 0) old = atomicAdd(prm.counter + x * kCounterStride, 1ull);
    old = uniform64(old);
    if (prm.force_giveup || (prm.self_plan && (old >> kCountBits) != tag)) {
      if (!prm.force_giveup && ++spins < kMaxSpins) {
        __builtin_amdgcn_s_sleep(8);
      } else {
        ++queue;
        if (lane == 0) atomicOr(prm.status, kGaveUpDecode);
      }
      continue;
    }
    const unsigned long long c = prm.self_plan ? old & (kMaxQueueItems - 1) : old;
    const unsigned long long f = first_dyn + nq * c + x;
    if (f < total) return (uint32_t)f;
    ++queue;
  }
  return 0xffffffffu;
}

// claim() in two halves, so that a stream with two tiles in flight can read
// the atomic's result later: loads complete in order, so reading it at once
// would also wait for the tile loads issued before it.  claim_start issues
// the first attempt (lane 0's atomic on the wave's current queue);
// claim_finish reads it and continues exactly as claim() does.
__device__ __forceinline__ bool claim_start(const DecodeParams& prm, uint32_t nq, uint32_t home, uint32_t queue,
                                            uint32_t first_dyn, uint32_t total, unsigned long long& pending) {
  if (queue >= nq || first_dyn >= total) return false;
  const uint32_t x = (home + queue) % nq;
  if (lane_id() == 0) pending = atomicAdd(prm.counter + x * kCounterStride, 1ull);
  return true;
}

__device__ __forceinline__ uint32_t claim_finish(const DecodeParams& prm, unsigned long long tag, uint32_t nq,
                                                 uint32_t home, uint32_t& queue, uint32_t first_dyn, uint32_t total,
                                                 bool started, unsigned long long pending) {
  if (!started) return 0xffffffffu;
  const int lane = lane_id();
  int spins = 0;
  bool first = true;
  while (queue < nq) {
    const uint32_t x = (home + queue) % nq;
    unsigned long long old = 0;
    if (first) {
      old = uniform64(pending);
      first = false;
    } else {
      if (lane == 0) old = atomicAdd(prm.counter + x * kCounterStride, 1ull);
      old = uniform64(old);
    }
    if (prm.force_giveup || (prm.self_plan && (old >> kCountBits) != tag)) {
      if (!prm.force_giveup && ++spins < kMaxSpins) {
        __builtin_amdgcn_s_sleep(8);
      } else {
        ++queue;
        if (lane == 0) atomicOr(prm.status, kGaveUpDecode);
      }
      continue;
    }
    const unsigned long long c = prm.self_plan ? old & (kMaxQueueItems - 1) : old;
    const unsigned long long f = first_dyn + nq * c + x;
    if (f < total) return (uint32_t)f;
    ++queue;
  }
  return 0xffffffffu;
}

// ---------------------------------------------------------------------------
// In-kernel plan (batches of at most kSelfPlanMax requests).  Each workgroup
// derives the item list from the lengths, in LDS: full partitions first,
// request by request, then the tail partitions by tile count (16 .. 1),
// requests in increasing order within a count.  The list is a function of
// the lengths alone, so all workgroups agree on it without communicating.
// List entry i < F (the full-partition count) is full partition i - pf[b]
// of the request b with pf[b] <= i < pf[b + 1]; entry F + j is the tail of
// request tail_b[j].
// ---------------------------------------------------------------------------
constexpr int kSelfPlanMax = 1024;
constexpr int kPlanChunks = kSelfPlanMax / 64;

struct PlanLds {
  int pf[kSelfPlanMax + 1];                // first list entry of request b's full partitions; pf[B] = F
  int len[kSelfPlanMax];                   // clamped lengths
  uint16_t tail_b[kSelfPlanMax];           // requests with a tail partition, in list order
  uint16_t rk[kSelfPlanMax];               // tile count of the tail | rank among equal counts of its chunk << 5
  int pre[kPlanChunks][kTileBuckets + 1];  // per 64-request chunk: counts, then exclusive prefixes
  int bstart[kTileBuckets + 1];            // first tail position of each tile count
  int nfull, nitems, nq;
};

// Inclusive prefix sums with DPP row shifts (lanes shifted in from outside
// the 16-lane row read zero): inside each row, then across the wave.
template <int CTRL>
__device__ __forceinline__ int dpp_zero(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ int row16_incl_scan(int v) {
  v += dpp_zero<0x111>(v);  // row_shr:1
  v += dpp_zero<0x112>(v);  // row_shr:2
  v += dpp_zero<0x114>(v);  // row_shr:4
  v += dpp_zero<0x118>(v);  // row_shr:8
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v = row16_incl_scan(v);
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane_id() >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Tokens request b contributes to the decode items: its clamped length, or,
// in a mixed batch, zero unless its chunk is exactly one valid token.
template <bool kRowMap>
__device__ __forceinline__ int decode_len(const DecodeParams& prm, int b) {
  if (kRowMap) {
    const int c0 = prm.cu[b], c1 = prm.cu[b + 1];
    const int L = clamp_len(prm.lens[b], prm.cap);
    return c1 - c0 == 1 && c0 >= 0 && c1 <= prm.num_q_tokens ? L : 0;
  }
  return clamp_len(prm.lens[b], prm.cap);
}

// Every thread of the workgroup (nw waves) takes part (three barriers).
template <bool kRowMap>
__device__ void self_plan(const DecodeParams& prm, PlanLds* pl, int nw) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int B = prm.B;
  const int nc = (B + 63) >> 6;
  // 1: per chunk of 64 requests: lengths, the full-partition prefix inside
  // the chunk, each tail's rank among the chunk's tails of equal tile count,
  // and the chunk's counts
  for (int c = wave; c < nc; c += nw) {
    const int b = 64 * c + lane;
    const int L = b < B ? decode_len<kRowMap>(prm, b) : 0;
    const int full = L / kPartTokens, rest = L - full * kPartTokens;
    const int bk = rest ? (rest + kTile - 1) / kTile : 0;
    const int incl = wave_incl_scan(full);
    // tails of k tiles counted in 8-bit field (k - 1) % 4 of word (k - 1) / 4
    // (at most 64 per field): one prefix sum per word gives every lane the
    // number of lower lanes with its tile count, and lane 63 the totals
    const int kb = bk - 1;
    int sc[4], tw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc[w] = wave_incl_scan(bk != 0 && (kb >> 2) == w ? 1 << (8 * (kb & 3)) : 0);
      tw[w] = __builtin_amdgcn_readlane(sc[w], 63);
    }
    const int mine = kb < 4 ? sc[0] : kb < 8 ? sc[1] : kb < 12 ? sc[2] : sc[3];
    const int rank = bk ? ((mine >> (8 * (kb & 3))) & 255) - 1 : 0;
    // lane k (1..16) takes the chunk's count of tails of k tiles, lane 0 its full partitions
    const int lk = lane - 1;
    const int word = lk < 4 ? tw[0] : lk < 8 ? tw[1] : lk < 12 ? tw[2] : tw[3];
    int cnt = (word >> (8 * (lk & 3))) & 255;
    if (lane == 0) cnt = __builtin_amdgcn_readlane(incl, 63);
    if (b < B) {
      pl->len[b] = L;
      pl->pf[b] = incl - full;
      pl->rk[b] = (uint16_t)(bk | rank << 5);
    }
    if (lane <= kTileBuckets) pl->pre[c][lane] = cnt;
  }
  __syncthreads();
  // 2: exclusive prefixes over the chunks (lane c < 16: chunk c), totals,
  // the first tail position of each tile count, and the queue count (one
  // queue when items average at least 4 tiles: 16 per full partition, k
  // per tail of k tiles)
  if (wave == 0) {
    int tot[kTileBuckets + 1], v[kTileBuckets + 1];
#pragma unroll
    for (int k = 0; k <= kTileBuckets; ++k) v[k] = lane < nc ? pl->pre[lane][k] : 0;
#pragma unroll
    for (int k = 0; k <= kTileBuckets; ++k) {
      const int incl = row16_incl_scan(v[k]);
      if (lane < nc) pl->pre[lane][k] = incl - v[k];
      tot[k] = __builtin_amdgcn_readlane(incl, kPlanChunks - 1);
    }
    if (lane == 0) {
      int run = 0;
      long long tiles = (long long)kTileBuckets * tot[0];
#pragma unroll
      for (int k = kTileBuckets; k >= 1; --k) {
        pl->bstart[k] = run;
        run += tot[k];
        tiles += (long long)k * tot[k];
      }
      pl->nfull = tot[0];
      pl->nitems = tot[0] + run;
      pl->nq = tiles >= 4ll * (tot[0] + run) ? 1 : kQueues;
      pl->pf[B] = tot[0];
    }
  }
  __syncthreads();
  // 3: global full-partition offsets and the tail order
  for (int c = wave; c < nc; c += nw) {
    const int b = 64 * c + lane;
    if (b < B) {
      const int rk = pl->rk[b];
      const int bk = rk & 31;
      pl->pf[b] += pl->pre[c][0];
      if (bk) pl->tail_b[pl->bstart[bk] + pl->pre[c][bk] + (rk >> 5)] = (uint16_t)b;
    }
  }
  __syncthreads();
}

// Descriptor {request, partition, length, partitions} of list entry i.
__device__ __forceinline__ i32x4_t plan_desc(const PlanLds* pl, int B, int nfull, int i) {
  int b, part;
  if (i < nfull) {
    int lo = 0, hi = B;  // pf[lo] <= i < pf[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pl->pf[mid] <= i) lo = mid;
      else hi = mid;
    }
    b = lo;
    part = i - pl->pf[lo];
  } else {
    b = pl->tail_b[i - nfull];
    part = pl->len[b] / kPartTokens;
  }
  const int L = pl->len[b];
  return i32x4_t{b, part, L, (L + kPartTokens - 1) / kPartTokens};
}

__device__ __forceinline__ i32x4_t item_desc(const DecodeParams& prm, const PlanLds* pl, uint32_t nfull, uint32_t i) {
  if (prm.self_plan) return plan_desc(pl, prm.B, (int)nfull, (int)i);
  return prm.items[i];
}

// ---------------------------------------------------------------------------
// Partition kernel.  One wave = one work item (request, partition, KV head,
// group of up to 16 query heads) at a time.
//
// Schedule: the flat item list (items x KV heads x head groups) starts with
// the full partitions, all of the same size.  Whole rounds of those are dealt
// statically (wave w takes w, w + nwaves, ...), which balances exactly; lane
// r of a register holds the wave's round-r descriptor, so the next static
// item costs no memory access.  The rest (the last full round and all tail
// partitions, largest first) is claimed dynamically from per-XCD queues, one
// item ahead.
//
// The loop runs over the wave's stream of tiles, across item boundaries: each
// iteration stages the tile that has landed, issues the loads of the next
// tile of the stream (the next item's first tile after an item's last), and
// computes.  The next item's block ids are fetched at its predecessor's
// first tile and its query after the predecessor's last S^T product, so
// items follow one another without draining the loads in flight.
//
// Per 16 tokens of a tile (two such halves for fp8):
//   S^T = K Q^T   (A = K rows from LDS, B = Q^T with the group's heads as
//                  columns 0..3), so lane (n, g) gets the scores of head n for
//                  tokens 4g .. 4g+3 of the half;
//   online softmax per head (max over the lane's 4 tokens, then across the
//                  four 16-lane rows);
//   O^T += V^T P^T (A = V^T from LDS, B = the lane's own probabilities), so
//                  lane (n, g) accumulates head n's outputs d = 16db + 4g + j.
// ---------------------------------------------------------------------------
// Decode with append (bf16 and fp32 pools): the new token's 16-byte piece of
// the item's head slice that this lane stages (piece lane % CPR).
template <typename T, int D, int HP>
__device__ __forceinline__ void load_new(const DecodeParams& prm, const Item& it, u32x4_t& nk, u32x4_t& nv) {
  using Gm = Geo<T, D>;
  static_assert(!Gm::kFp8, "fp8 pools make the new codes in append_lds");
  // the new rows have the pool rows' layout: the item's slice of row b
  const int64_t off = (int64_t)it.b * (prm.Hkv * Gm::GROWB) + it.hkv * Gm::GROWB + 16 * (lane_id() % Gm::CPR);
  nk = *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(prm.knew) + off);
  nv = *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(prm.vnew) + off);
}

// Decode with append, at the last tile of a request's last partition (tile0
// holds position L - 1).  Items of query-head group 0 write the new token to
// its slot, unless the block id is out of range (as the scatter skips such
// slots); the lanes that stage the token's pieces hold (nk, nv).
// Block id of the item's position L - 1 (the new token's), from its block ids.
template <int NR>
__device__ __forceinline__ int append_block(const DecodeParams& prm, const Item& it, const int (&ids)[NR]) {
  const int lb = (it.L - 1) / prm.P;
  return lane_id_lookup<NR>(ids, lb - it.blk0);
}

template <typename T, int D>
__device__ __forceinline__ void append_store(const DecodeParams& prm, const PoolView& pv, const Item& it, int blk,
                                             bool mine, const u32x4_t& nk, const u32x4_t& nv) {
  using Gm = Geo<T, D>;
  if (it.hg != 0) return;
  const int pos = it.L - 1;
  const int lb = pos / prm.P, off = pos - lb * prm.P;
  if (mine && blk >= 0 && blk < prm.N) {
    const uint64_t e = ((uint64_t)blk * (uint64_t)prm.P + (uint64_t)off) * pv.row_bytes +
                       (uint64_t)(it.hkv * Gm::GROWB + 16 * (lane_id() % Gm::CPR));
    *reinterpret_cast<u32x4_t*>(const_cast<char*>(pv.k) + e) = nk;
    *reinterpret_cast<u32x4_t*>(const_cast<char*>(pv.v) + e) = nv;
  }
}

// bf16 and fp32 pools: before the last tile is staged, the lane that stages
// the new token takes its piece from (nk, nv), loaded with the item's first
// tile.  A length beyond the block table (clamped when read) appends nothing.
template <typename T, int D>
__device__ __forceinline__ void append_regs(const DecodeParams& prm, const PoolView& pv, const Item& it, int blk,
                                            int len, int tile0, const u32x4_t& nk, const u32x4_t& nv,
                                            TileRegs<T, D>& regs) {
  using Gm = Geo<T, D>;
  if (len > prm.cap) return;  // the request's unclamped length: beyond the block table, nothing is appended
  const int tL = it.L - 1 - tile0;  // in [0, TT)
  const int qL = tL / Gm::TPL, jL = tL - qL * Gm::TPL;
  const bool mine = lane_id() / Gm::CPR == qL;
#pragma unroll
  for (int j = 0; j < Gm::TPL; ++j)
    if (mine && j == jL) {
      regs.k[j] = nk;
      regs.v[j] = nv;
    }
  append_store<T, D>(prm, pv, it, blk, mine, nk, nv);
}

// Decode with append, two-tile stream (bf16): the item's last tile was loaded
// with the new token (position L - 1) taken from the new rows.  Items of
// query-head group 0 write it to its slot (unless the block id is out of
// range), from the tile's registers, which are only read.
template <typename T, int D>
__device__ __forceinline__ void append_from_regs(const DecodeParams& prm, const PoolView& pv, const Item& it, int blk,
                                                 int tile0, const TileRegs<T, D>& regs) {
  using Gm = Geo<T, D>;
  const int tL = it.L - 1 - tile0;  // in [0, TT)
  const int qL = tL / Gm::TPL, jL = tL - qL * Gm::TPL;
  const bool mine = lane_id() / Gm::CPR == qL;
  u32x4_t nk = {0u, 0u, 0u, 0u}, nv = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < Gm::TPL; ++j)
    if (j == jL) {
      nk = regs.k[j];
      nv = regs.v[j];
    }
  append_store<T, D>(prm, pv, it, blk, mine, nk, nv);
}

// A request whose length is beyond its block table appends nothing (its
// clamped last position is an old token), so the staged row of that position
// is put back from the pool: the K row and the V^T column, after staging,
// read synchronously (a caller error, never on a valid batch).
template <typename T, int D>
__device__ __forceinline__ void unappend_lds(const DecodeParams& prm, const PoolView& pv, const Item& it, int blk,
                                             int tile0, char* lds) {
  using Gm = Geo<T, D>;
  static_assert(Gm::kBf16, "bf16 pools");
  if (blk < 0 || blk >= prm.N) return;  // the token is masked (zero) anyway
  const int lane = lane_id();
  const int tL = it.L - 1 - tile0;
  const int pos = it.L - 1;
  const int lb = pos / prm.P, off = pos - lb * prm.P;
  const int c = lane % Gm::CPR;
  const uint64_t e = ((uint64_t)blk * (uint64_t)prm.P + (uint64_t)off) * pv.row_bytes +
                     (uint64_t)(it.hkv * Gm::GROWB + 16 * c);
  const u32x4_t pk = *reinterpret_cast<const u32x4_t*>(pv.k + e);
  const u32x4_t pvv = *reinterpret_cast<const u32x4_t*>(pv.v + e);
  if (lane < Gm::CPR) {
    *reinterpret_cast<u32x4_t*>(lds + tL * Gm::KST + 16 * c) = pk;
    char* vl = lds + Gm::KBYTES;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int d = 8 * c + 2 * w;
      *reinterpret_cast<uint16_t*>(vl + d * Gm::VTS + 2 * tL) = (uint16_t)(pvv[w] & 0xffffu);
      *reinterpret_cast<uint16_t*>(vl + (d + 1) * Gm::VTS + 2 * tL) = (uint16_t)(pvv[w] >> 16);
    }
  }
}

// fp8 pools: after the last tile is staged, the new token's codes are made
// here, four per lane and word (lanes 0-31 K, 32-63 V), and written over its staged K
// and V rows (unless the token was zeroed: invalid block id) and, by items of
// query-head group 0, to its slot.  Each code is x / scale[h], correctly
// rounded, then encoded, as the fp8 scatter makes it.
template <typename T, int D, int NR, int HP>
__device__ __forceinline__ void append_lds(const DecodeParams& prm, const PoolView& pv, const Item& it,
                                           const int (&ids)[NR], int tile0, uint32_t ok, char* lds) {
  using Gm = Geo<T, D>;
  static_assert(Gm::kFp8, "fp8 pools");
  if (prm.lens[it.b] > prm.cap) return;
  constexpr int W = Gm::ROWB / 4;  // 4-code words of the item's row slice
  const int lane = lane_id();
  const int tL = it.L - 1 - tile0;  // in [0, TT)
  const int qL = tL / Gm::TPL, jL = tL - qL * Gm::TPL;
  const bool tok_ok = ((__builtin_amdgcn_readlane((int)ok, qL * Gm::CPR) >> jL) & 1) != 0;
  const bool isv = lane >= 32;
  static_assert(W <= 64, "at most two words per lane");
#pragma unroll
  for (int w2 = 0; w2 < (W + 31) / 32; ++w2) {  // (two for 256-code slices)
  const int w = (lane & 31) + 32 * w2;
  const bool act = w < W;
  const int e = 4 * (act ? w : 0);  // code index within the slice
  const int h = HP == 2 ? 2 * it.hkv + (e >= D / 2 ? 1 : 0) : it.hkv;
  const float sc = isv ? prm.v_scale[h] : prm.k_scale[h];
  const int64_t e0 = ((int64_t)it.b * prm.Hkv + it.hkv) * D + e;
  const void* src = isv ? prm.vnew : prm.knew;
  float x[4];
  if (prm.new_f32) {
    const f32x4_t f = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(src) + e0);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = f[j];
  } else {
    const u32x2_t u = *reinterpret_cast<const u32x2_t*>(static_cast<const bf16_bits*>(src) + e0);
    x[0] = bf16_lo(u[0]);
    x[1] = bf16_hi(u[0]);
    x[2] = bf16_lo(u[1]);
    x[3] = bf16_hi(u[1]);
  }
  uint32_t code = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) code |= e4m3_from_f32(x[j] / sc) << (8 * j);
  if (act && tok_ok) *reinterpret_cast<uint32_t*>(lds + (isv ? Gm::KBYTES : 0) + tL * Gm::KST + e) = code;
  if (it.hg == 0) {
    const int pos = it.L - 1;
    const int lb = pos / prm.P, off = pos - lb * prm.P;
    const int blk = lane_id_lookup<NR>(ids, lb - it.blk0);
    if (act && blk >= 0 && blk < prm.N) {
      const uint64_t a = ((uint64_t)blk * (uint64_t)prm.P + (uint64_t)off) * pv.row_bytes +
                         (uint64_t)(it.hkv * Gm::GROWB + e);
      *reinterpret_cast<uint32_t*>(const_cast<char*>(isv ? pv.v : pv.k) + a) = code;
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Per-tile arithmetic of a decode item, shared by the decode streams (so that
// every stream computes an item the same way, bit for bit).
// ---------------------------------------------------------------------------
// S^T = K Q^T for the staged tile, per 16-token half: lane (n, g) gets the
// scores of column n for tokens 16h + 4g + j (HP = 2: the products over the
// first D / 2 dimensions in s, over the others in s2).
template <typename T, int D, int HP>
__device__ __forceinline__ void tile_scores(const char* lds, const u32x4_t (&qv)[Geo<T, D>::NQV],
                                            f32x4_t (&s)[Geo<T, D>::TT / 16], f32x4_t (&s2)[Geo<T, D>::TT / 16]) {
  using Gm = Geo<T, D>;
  constexpr int NH = Gm::TT / 16;
  constexpr int NQ1 = Gm::NQ / HP;
  const int lane = lane_id();
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int h = 0; h < NH; ++h) s[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (HP == 2) {
#pragma unroll
    for (int h = 0; h < NH; ++h) s2[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (Gm::kFp8) {
    // K operand: 8 codes of token 16 h + n, widened to fp16 as they are read
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int i = 0; i < NQ1; ++i) {
        const u32x2_t c = *reinterpret_cast<const u32x2_t*>(lds + (16 * h + n) * Gm::KST + 32 * i + 8 * g);
        s[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, e4m3x8_to_f16(c)),
                                                      __builtin_bit_cast(f16x8_t, qv[i]), s[h], 0, 0, 0);
      }
      if constexpr (HP == 2) {
#pragma unroll
        for (int i = NQ1; i < Gm::NQ; ++i) {
          const u32x2_t c = *reinterpret_cast<const u32x2_t*>(lds + (16 * h + n) * Gm::KST + 32 * i + 8 * g);
          s2[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, e4m3x8_to_f16(c)),
                                                         __builtin_bit_cast(f16x8_t, qv[i]), s2[h], 0, 0, 0);
        }
      }
    }
  } else if constexpr (Gm::kBf16) {
#pragma unroll
    for (int i = 0; i < NQ1; ++i) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lds + n * Gm::KST + 2 * (32 * i + 8 * g));
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                     __builtin_bit_cast(bf16x8_t, qv[i]), s[0], 0, 0, 0);
    }
    if constexpr (HP == 2) {
#pragma unroll
      for (int i = NQ1; i < Gm::NQ; ++i) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lds + n * Gm::KST + 2 * (32 * i + 8 * g));
        s2[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, qv[i]), s2[0], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < Gm::NQ / 4; ++i) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lds + n * Gm::KST + 4 * (g * (D / 4) + 4 * i));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(qv[i][j]), s[0], 0, 0,
                                                    0);
    }
  }
}

// HP = 2: each column keeps the scores of its own KV head of the pair.
template <int NH, int HP>
__device__ __forceinline__ void own_half(f32x4_t (&s)[NH], const f32x4_t (&s2)[NH], int gs) {
  const int n = lane_id() & 15;
  if constexpr (HP == 2) {
    const bool hi = ((n >> gs) & 1) != 0;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const f32x4_t lo = s[h], up = s2[h];
      s[h] = f32x4_t{hi ? up[0] : lo[0], hi ? up[1] : lo[1], hi ? up[2] : lo[2], hi ? up[3] : lo[3]};
    }
  }
}

// Online softmax of the tile's scores for column n (tokens tile0 + 16h + 4g +
// j; tokens at or past it.tok_end are masked), then O^T += V^T P^T.
template <typename T, int D>
__device__ __forceinline__ void tile_softmax_pv(const char* lds, const Item& it, int tile0,
                                                const f32x4_t (&s)[Geo<T, D>::TT / 16], float& m, float& l,
                                                f32x4_t (&o)[D / 16]) {
  using Gm = Geo<T, D>;
  constexpr int NH = Gm::TT / 16;
  constexpr int NDB = D / 16;
  const int lane = lane_id();
  const int n = lane & 15, g = lane >> 4;
  float sc[NH][4];
  float mx = -INFINITY;
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[h][j] = (tile0 + 16 * h + 4 * g + j < it.tok_end) ? s[h][j] * it.sl2 : -INFINITY;
      mx = fmaxf(mx, sc[h][j]);
    }
  mx = max_over_rows(mx);
  // move the reference max only when a score exceeds it by the slack
  // (always on the first tile, m = -inf); uniform branch, rarely taken
  const bool move = mx > m + kRescaleSlack;
  if (__builtin_amdgcn_readfirstlane((int)(__ballot(move) != 0))) {
    const float alpha = (move && m != -INFINITY) ? fast_exp2(m - mx) : 1.0f;
    if (move) m = mx;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
  }
  float pp[NH][4];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pp[h][j] = fast_exp2(sc[h][j] - m);
      l += pp[h][j];
    }
  const float* p = pp[0];
  // ---- O^T += V^T P^T ----
  const char* vl = lds + Gm::KBYTES;
  if constexpr (Gm::kFp8) {
    // B operand: the lane's probabilities, k-slots 0-3 = tokens 4g + j and
    // 4-7 = tokens 16 + 4g + j.  A operand (V^T) in the same token order
    // from the byte-transposing read: lane n of each 16-lane group addresses
    // V row 4g + n/2 (n < 8) or 12 + 4g + n/2 (n >= 8), bytes 16db + 8 (n % 2)
    const u32x4_t pb = {pack_f16(pp[0][0], pp[0][1]), pack_f16(pp[0][2], pp[0][3]), pack_f16(pp[1][0], pp[1][1]),
                        pack_f16(pp[1][2], pp[1][3])};
    const char* vrow = vl + ((n < 8 ? 4 * g : 12 + 4 * g) + (n >> 1)) * Gm::KST + 8 * (n & 1);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2_t c = lds_read_tr8(vrow + 16 * db);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, e4m3x8_to_f16(c)),
                                                     __builtin_bit_cast(f16x8_t, pb), o[db], 0, 0, 0);
    }
  } else if constexpr (Gm::kBf16) {
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

// Item done: total of l over the four 16-lane rows, then column n's output
// row (one partition) or its partial row and (max, sum, scale) entry.
template <typename T, int D, int HP>
__device__ __forceinline__ void store_item(const DecodeParams& prm, const Item& it, float m, float l,
                                           const f32x4_t (&o)[D / 16]) {
  using Gm = Geo<T, D>;
  typedef typename QType<T>::type QT;
  constexpr int NDB = D / 16;
  const int lane = lane_id();
  const int n = lane & 15, g = lane >> 4;
  // (HP = 2: column n's head is the pair's first or second, and its outputs
  // are the first or the second half of the rows of O^T)
  constexpr int DH = D / HP, NDBH = NDB / HP;
  l = sum_over_rows(l);
  f32x4_t ov[NDBH];
  bool col;
  int h;
  if constexpr (HP == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) ov[db] = o[db];
    col = n < it.nh;
    h = it.hkv * prm.G + it.hg * prm.gw + n;
  } else {
    const bool hi = ((n >> prm.gs) & 1) != 0;
#pragma unroll
    for (int db = 0; db < NDBH; ++db) {
      // a select of values, not of the two array elements' addresses
      // (which would put o in scratch memory to index it)
      const f32x4_t lo = o[db], up = o[NDBH + db];
      ov[db] = f32x4_t{hi ? up[0] : lo[0], hi ? up[1] : lo[1], hi ? up[2] : lo[2], hi ? up[3] : lo[3]};
    }
    col = n < 2 * prm.gw && (n & (prm.gw - 1)) < it.nh;
    h = (2 * it.hkv + (hi ? 1 : 0)) * prm.G + it.hg * prm.gw + (n & (prm.gw - 1));
  }
  if (col) {
    if (it.nparts == 1) {
      const float inv = it.vmul / l;
      QT* dst = static_cast<QT*>(prm.out) + ((int64_t)it.row * prm.Hq + h) * DH + 4 * g;
#pragma unroll
      for (int db = 0; db < NDBH; ++db) {
        if constexpr (Gm::kHalf) {
          *reinterpret_cast<u32x2_t*>(dst + 16 * db) =
              u32x2_t{pack_bf16(ov[db][0] * inv, ov[db][1] * inv), pack_bf16(ov[db][2] * inv, ov[db][3] * inv)};
        } else {
          *reinterpret_cast<f32x4_t*>(dst + 16 * db) = ov[db] * inv;
        }
      }
    } else {
      const int64_t slot = ((int64_t)it.b * prm.Hq + h) * prm.max_parts + it.part;
      float rs = 1.0f;  // the stored row is o / l / rs (bf16) or o (fp32)
      if constexpr (Gm::kHalf) {
        // bf16 requests: the partial output normalised by its sum, as fp16
        // (half the bytes of fp32; its rounding is far below bf16's).  A
        // normalised row is a weighted mean of value rows, so it can exceed
        // the fp16 range only if the values do; then it is scaled down by a
        // power of two, kept beside (max, sum), so it stays below 2^15.
        const float inv = it.vmul / l;
        float amax = 0.f;
#pragma unroll
        for (int db = 0; db < NDBH; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(ov[db][j]));
        amax = max_over_rows(amax * inv);  // the head's whole row (lanes n, n+16, n+32, n+48)
        if (amax >= 32768.0f) {
          int ex;
          frexpf(amax, &ex);  // amax < 2^ex
          rs = ldexpf(1.0f, ex - 15);
        }
        const float sc = inv / rs;
        uint16_t* dst = reinterpret_cast<uint16_t*>(prm.o) + slot * DH + 4 * g;
#pragma unroll
        for (int db = 0; db < NDBH; ++db)
          *reinterpret_cast<u32x2_t*>(dst + 16 * db) =
              u32x2_t{pack_f16(ov[db][0] * sc, ov[db][1] * sc), pack_f16(ov[db][2] * sc, ov[db][3] * sc)};
      } else {
        float* dst = prm.o + slot * DH + 4 * g;
#pragma unroll
        for (int db = 0; db < NDBH; ++db) *reinterpret_cast<f32x4_t*>(dst + 16 * db) = ov[db];
      }
      if (g == 0) *reinterpret_cast<f32x4_t*>(prm.ml + slot * 4) = f32x4_t{m, l, rs, 0.f};
    }
  }
}

template <typename T, int D, bool kWide, bool kAligned, int NR, bool kRowMap, int HP = 1, bool kAppend = false>
__device__ __forceinline__ void decode_stream(const DecodeParams& prm, char* lds, const PlanLds* pl,
                                              unsigned long long tag, uint32_t n_items, uint32_t n_full,
                                              uint32_t nq_plan, uint32_t wave, uint32_t nwaves,
                                              uint32_t max_rounds) {
  using Gm = Geo<T, D>;
  typedef typename QType<T>::type QT;
  constexpr int NDB = D / 16;
  const int lane = lane_id();
  const int n = lane & 15;  // head column (S^T, O^T) / token row (K operand)
  const int g = lane >> 4;
  const uint32_t per_item = (uint32_t)(prm.Hkv * prm.n_hg);
  const uint32_t total = n_items * per_item;
  // static rounds: whole rounds of full partitions, at most one per lane;
  // the queues hand out the rest (the last kDynamicRounds whole rounds, the
  // partial round and the tails), which balances waves that run at
  // different speeds.  Measured on the Llama-3-8B batch, leaving no whole
  // round to the queues is best.
  uint32_t rounds = min((n_full * per_item) / nwaves, max_rounds);
  rounds = rounds > (uint32_t)prm.dyn_rounds ? rounds - (uint32_t)prm.dyn_rounds : min(rounds, 1u);
  // With no whole static round (a batch whose full partitions do not fill
  // one), each wave's first item is still dealt statically: wave w takes
  // list entry w, the largest items first.  Otherwise every wave would start
  // by claiming from the queue at once, and the claims on one counter are
  // served one at a time.  (Decode calls only: in a mixed launch a wave may
  // still be busy with a prefill item, and its item would wait for it.)
  const bool first_static = !kRowMap && rounds == 0;
  const uint32_t first_dyn = first_static ? min(total, nwaves) : rounds * nwaves;
  const uint32_t nq = prm.nq > 0 ? (uint32_t)prm.nq : nq_plan;
  const uint32_t home = blockIdx.x % nq;
  uint32_t queue = 0;
  PoolView pv;
  pv.k = static_cast<const char*>(prm.kc);
  pv.v = static_cast<const char*>(prm.vc);
  pv.row_bytes = (uint32_t)(prm.Hkv * Gm::GROWB);

  // lane r: descriptor of this wave's item of static round r
  i32x4_t sdesc = {0, 0, 0, 0};
  if (rounds > 0) sdesc = item_desc(prm, pl, n_full, (wave + (uint32_t)min(lane, (int)rounds - 1) * nwaves) / per_item);

  // the current item: round r < rounds is static item wave + r * nwaves
  uint32_t r = 0;
  uint32_t f = wave;
  Item it;
  if (rounds > 0) {
    it = make_item<kRowMap, Gm::TT, HP>(prm, lane_desc(sdesc, 0), f, per_item);
  } else {
    r = rounds;
    if (first_static) {
      if (wave >= first_dyn) return;  // more waves than items
    } else {
      f = claim(prm, tag, nq, home, queue, first_dyn, total);
      if (f >= total) return;
    }
    it = make_item<kRowMap, Gm::TT, HP>(prm, item_desc(prm, pl, n_full, f / per_item), f, per_item);
  }
  int ids[NR];
  load_ids<NR>(prm, it, ids);
  u32x4_t qv[Gm::NQV];
  load_q<T, D, HP>(prm, it, qv);
  TileRegs<T, D> regs;
  load_tile<T, D, kWide, kAligned, NR>(pv, prm, it, ids, it.tok0, regs);
  u32x4_t nk, nv;  // decode with append: the new token's piece (last partitions)
  if constexpr (kAppend && !Gm::kFp8) {
    if (it.part == it.nparts - 1) load_new<T, D, HP>(prm, it, nk, nv);
  }

  Item nx = it;        // the item after the current one, once known
  uint32_t fn = 0;     // its flat index
  bool has_next = false;
  int pend = 0;        // 1: next item claimed (fn), 2: its descriptor loaded (dn)
  i32x4_t dn = {0, 0, 0, 0};
  int idn[NR];         // its block ids
#pragma unroll
  for (int i = 0; i < NR; ++i) idn[i] = 0;

  float m = -INFINITY, l = 0.f;
  f32x4_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int t = 0;;) {
    const int tile0 = it.tok0 + t * Gm::TT;
    const bool last = t + 1 == it.ntiles;
    // every token of the tile valid: no zeroing needed (the usual case)
    bool full;
    if constexpr (kAligned && Gm::TT == 16)
      full = tile0 + Gm::TT <= it.tok_end && __builtin_amdgcn_readfirstlane((int)regs.ok) == (1 << Gm::TPL) - 1;
    else
      full = __builtin_amdgcn_readfirstlane((int)(__ballot(regs.ok != (1u << Gm::TPL) - 1u) == 0));
    if constexpr (kAppend && !Gm::kFp8) {
      if (last && it.part == it.nparts - 1)
        append_regs<T, D>(prm, pv, it, append_block<NR>(prm, it, ids), prm.lens[it.b], tile0, nk, nv, regs);
    }
    wave_lds_sync();  // previous tile's LDS reads are done
    stage_tile<T, D>(lds, regs, full);
    if constexpr (kAppend && Gm::kFp8) {
      if (last && it.part == it.nparts - 1) append_lds<T, D, NR, HP>(prm, pv, it, ids, tile0, regs.ok, lds);
    }
    wave_lds_sync();

    // find the next item and fetch its block ids.  A static item is known at
    // once.  A dynamic one is claimed with an atomic right after tile 1's
    // loads are issued (its wait then only delays tile 0's arithmetic, not
    // the memory stream), its descriptor is loaded at tile 1 and its ids at
    // tile 2; items of one or two tiles claim everything up front.
    const bool stat_next = r + 1 < rounds;
    const bool early = it.ntiles >= 3;
    if (t == 0) {
      if (stat_next) {
        fn = f + nwaves;
        nx = make_item<kRowMap, Gm::TT, HP>(prm, lane_desc(sdesc, (int)r + 1), fn, per_item);
        has_next = true;
        load_ids<NR>(prm, nx, idn);
      } else if (!early) {
        fn = claim(prm, tag, nq, home, queue, first_dyn, total);
        if (fn < total) {
          nx = make_item<kRowMap, Gm::TT, HP>(prm, item_desc(prm, pl, n_full, fn / per_item), fn, per_item);
          has_next = true;
          load_ids<NR>(prm, nx, idn);
        }
      }
    }
    if (pend == 1 && t == 1) {
      dn = item_desc(prm, pl, n_full, fn / per_item);
      pend = 2;
    }
    if (pend == 2 && t == 2) {
      nx = make_item<kRowMap, Gm::TT, HP>(prm, dn, fn, per_item);
      has_next = true;
      load_ids<NR>(prm, nx, idn);
      pend = 0;
    }
    // the next tile of the stream: this item's, or the next item's first
    if (last && has_next) {
      // a real branch, not a select: a select would read idn on every tile
      // and so wait for its load right after it is issued
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < NR; ++i) ids[i] = idn[i];
    }
    if (!last || has_next)
      load_tile<T, D, kWide, kAligned, NR>(pv, prm, last ? nx : it, ids, last ? nx.tok0 : tile0 + Gm::TT, regs);
    if constexpr (kAppend && !Gm::kFp8) {
      if (last && has_next && nx.part == nx.nparts - 1) load_new<T, D, HP>(prm, nx, nk, nv);
    }
    if (t == 0 && early && !stat_next) {
      fn = claim(prm, tag, nq, home, queue, first_dyn, total);
      if (fn < total) pend = 1;
    }

    // ---- S^T = K Q^T, online softmax, O^T += V^T P^T ----
    constexpr int NH = Gm::TT / 16;
    f32x4_t s[NH], s2[NH];
    tile_scores<T, D, HP>(lds, qv, s, s2);
    if (last && has_next) load_q<T, D, HP>(prm, nx, qv);  // this item's query is no longer needed
    own_half<NH, HP>(s, s2, prm.gs);
    tile_softmax_pv<T, D>(lds, it, tile0, s, m, l, o);
    if (!last) {
      ++t;
      continue;
    }

    store_item<T, D, HP>(prm, it, m, l, o);
    if (!has_next) break;
    // the next item's ids, first tile and query are already in flight
    it = nx;
    f = fn;
    r = r + 1 < rounds ? r + 1 : rounds;
    has_next = false;
    t = 0;
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// ---------------------------------------------------------------------------
// Decode stream with two tiles in flight per wave (bf16 pools).  It computes
// the same items in the same order as decode_stream, each with the same
// arithmetic (the helpers above), so its results are the same bits.  The
// difference is in the loads: decode_stream issues a tile's loads after it
// has staged the tile before it, so one tile is in flight while a tile is
// computed; here a producer cursor runs two tiles ahead of the tile being
// computed.  After the consumer has staged tile g of the stream from register
// set g % 2, the producer issues tile g + 2 into that set.  A wave whose
// tiles arrive one memory latency apart (few items per wave: small batches)
// then waits half as long per tile, and fewer waves per SIMD keep as many
// bytes in flight.
//
// The producer fetches the next item (claim, descriptor, block ids) relative
// to its own item's tiles, as decode_stream does relative to the computed
// one.  Items whose first tile is issued but which the consumer has not yet
// started wait in a queue of two (the producer is at most two tiles ahead, and
// every item has at least one tile); the consumer rebuilds an item from its
// descriptor and flat index when it gets to it.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct TileSet {
  TileRegs<T, D> regs;
  int alen;        // decode with append: the request's unclamped length (the item's last tile)
  int ablk;        // decode with append: block id of the item's position L - 1
};

template <typename T, int D, bool kWide, bool kAligned, int NR, int HP = 1, bool kAppend = false>
__device__ __forceinline__ void decode_stream2(const DecodeParams& prm, char* lds, const PlanLds* pl,
                                               unsigned long long tag, uint32_t n_items, uint32_t n_full,
                                               uint32_t nq_plan, uint32_t wave, uint32_t nwaves,
                                               uint32_t max_rounds) {
  using Gm = Geo<T, D>;
  static_assert(!Gm::kFp8, "fp8 pools make the new token's codes in LDS; they use decode_stream");
  constexpr int NDB = D / 16;
  constexpr int NH = Gm::TT / 16;
  const int lane = lane_id();
  const uint32_t per_item = (uint32_t)(prm.Hkv * prm.n_hg);
  const uint32_t total = n_items * per_item;
  // the schedule of decode_stream (plain decode: first item static when no
  // whole round is)
  uint32_t rounds = min((n_full * per_item) / nwaves, max_rounds);
  rounds = rounds > (uint32_t)prm.dyn_rounds ? rounds - (uint32_t)prm.dyn_rounds : min(rounds, 1u);
  const bool first_static = rounds == 0;
  const uint32_t first_dyn = first_static ? min(total, nwaves) : rounds * nwaves;
  const uint32_t nq = prm.nq > 0 ? (uint32_t)prm.nq : nq_plan;
  const uint32_t home = blockIdx.x % nq;
  uint32_t queue = 0;
  PoolView pv;
  pv.k = static_cast<const char*>(prm.kc);
  pv.v = static_cast<const char*>(prm.vc);
  pv.row_bytes = (uint32_t)(prm.Hkv * Gm::GROWB);
  i32x4_t sdesc = {0, 0, 0, 0};
  if (rounds > 0) sdesc = item_desc(prm, pl, n_full, (wave + (uint32_t)min(lane, (int)rounds - 1) * nwaves) / per_item);

  // ---- producer: the item whose tiles it issues ----
  uint32_t r = 0;        // its static round (rounds once dynamic)
  uint32_t pf = wave;    // its flat index
  i32x4_t pd;            // the first item's descriptor
  if (rounds > 0) {
    pd = lane_desc(sdesc, 0);
  } else {
    r = rounds;
    if (first_static) {
      if (wave >= first_dyn) return;  // more waves than items
    } else {
      pf = claim(prm, tag, nq, home, queue, first_dyn, total);
      if (pf >= total) return;
    }
    pd = item_desc(prm, pl, n_full, pf / per_item);
  }
  Item pit = make_item<false, Gm::TT, HP>(prm, pd, pf, per_item);
  int pids[NR];
  load_ids<NR>(prm, pit, pids);
  int pt = 0;            // next tile of pit to issue
  bool pdone = false;    // the stream is fully issued
  // its next item, once known (descriptor and flat index; the item itself
  // is rebuilt from them when the producer gets to it)
  uint32_t fn = 0;
  i32x4_t nd = {0, 0, 0, 0};
  bool has_next = false;
  int idn[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) idn[i] = 0;
  // items issued but not yet started by the consumer (descriptor, flat index)
  i32x4_t qd0 = {0, 0, 0, 0}, qd1 = {0, 0, 0, 0};
  uint32_t qf0 = 0, qf1 = 0;
  int nqueued = 0;
  unsigned long long pending = 0;  // a claim's first atomic, issued but not yet read
  bool claimed = false;

  // ---- consumer: the item being computed ----
  Item it = pit;
  u32x4_t qv[Gm::NQV];   // its query
  load_q<T, D, HP>(prm, it, qv);
  int ct = 0;            // its tile being computed
  float m = -INFINITY, l = 0.f;
  f32x4_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  TileSet<T, D> sa, sb;

  // Issues the stream's next tile into S (nothing once the stream is issued).
  auto produce = [&](TileSet<T, D>& S) {
    if (pt == pit.ntiles && !has_next) pdone = true;
    if (pdone) {
      // the stream is fully issued: the same loads as a tile, every token
      // masked (each lane reads its piece of row 0, which stays in cache).
      // The set is never staged again; the loads are there so that every
      // path issues as many loads after a set's as the wait for it assumes
      // (otherwise the wait before staging would drain both sets).
      load_tile<T, D, kWide, kAligned, NR>(pv, prm, pit, pids, pit.tok_end, S.regs);
      return;
    }
    if (pt == pit.ntiles) {
      // a real branch, not a select: a select would read idn at every tile
      // and so wait for its load right after it is issued
      asm volatile("" ::: "memory");
      pit = make_item<false, Gm::TT, HP>(prm, nd, fn, per_item);
      pf = fn;
#pragma unroll
      for (int i = 0; i < NR; ++i) pids[i] = idn[i];
      r = r + 1 < rounds ? r + 1 : rounds;
      has_next = false;
      pt = 0;
      if (nqueued == 0) {
        qd0 = nd;
        qf0 = fn;
      } else {
        qd1 = nd;
        qf1 = fn;
      }
      ++nqueued;
    }
    if constexpr (kAppend) {
      if (pt + 1 == pit.ntiles && pit.part == pit.nparts - 1) {
        // the item's last tile holds the new token (position L - 1): its
        // lanes load it from the new rows, as the scatter would have written it
        const int64_t off = (int64_t)pit.b * (prm.Hkv * Gm::GROWB) + pit.hkv * Gm::GROWB + 16 * (lane % Gm::CPR);
        load_tile<T, D, kWide, kAligned, NR, true>(pv, prm, pit, pids, pit.tok0 + pt * Gm::TT, S.regs, pit.L - 1,
                                                   static_cast<const char*>(prm.knew) + off,
                                                   static_cast<const char*>(prm.vnew) + off);
        S.alen = prm.lens[pit.b];  // behind the tile's loads, read when the tile is staged
        S.ablk = __builtin_amdgcn_readfirstlane(append_block<NR>(prm, pit, pids));
      } else {
        load_tile<T, D, kWide, kAligned, NR>(pv, prm, pit, pids, pit.tok0 + pt * Gm::TT, S.regs);
      }
    } else {
      load_tile<T, D, kWide, kAligned, NR>(pv, prm, pit, pids, pit.tok0 + pt * Gm::TT, S.regs);
    }
    // the next item: a static one is known at once.  A dynamic one is
    // claimed near the end of this item, so that the claims of waves that
    // started together do not all reach the counter at once: the atomic is
    // issued with tile n - 5, and its result read with tile n - 3, when the
    // consumer has staged the tile issued before it (reading it waits for
    // nothing in flight); the ids are loaded then too, two tiles before they
    // are needed.  Items of fewer than five tiles claim everything up front.
    const bool stat_next = r + 1 < rounds;
    const int n = pit.ntiles;
    if (stat_next) {
      if (pt == 0) {
        fn = pf + nwaves;
        nd = lane_desc(sdesc, (int)r + 1);
        has_next = true;
        load_ids<NR>(prm, make_item<false, Gm::TT, HP>(prm, nd, fn, per_item), idn);
      }
    } else if (n < 5) {
      if (pt == 0) {
        fn = claim(prm, tag, nq, home, queue, first_dyn, total);
        if (fn < total) {
          nd = item_desc(prm, pl, n_full, fn / per_item);
          has_next = true;
          load_ids<NR>(prm, make_item<false, Gm::TT, HP>(prm, nd, fn, per_item), idn);
        }
      }
    } else if (pt == n - 5) {
      claimed = claim_start(prm, nq, home, queue, first_dyn, total, pending);
    } else if (pt == n - 3) {
      fn = claim_finish(prm, tag, nq, home, queue, first_dyn, total, claimed, pending);
      if (fn < total) {
        nd = item_desc(prm, pl, n_full, fn / per_item);
        has_next = true;
        load_ids<NR>(prm, make_item<false, Gm::TT, HP>(prm, nd, fn, per_item), idn);
      }
    }
    ++pt;
  };

  // Stages and computes the stream's tile held in S, after refilling S with
  // the tile two ahead.  Returns true once the stream is done.
  auto consume = [&](TileSet<T, D>& S) -> bool {
    const int tile0 = it.tok0 + ct * Gm::TT;
    const bool last = ct + 1 == it.ntiles;
    bool full;
    if constexpr (kAligned && Gm::TT == 16)
      full = tile0 + Gm::TT <= it.tok_end && __builtin_amdgcn_readfirstlane((int)S.regs.ok) == (1 << Gm::TPL) - 1;
    else
      full = __builtin_amdgcn_readfirstlane((int)(__ballot(S.regs.ok != (1u << Gm::TPL) - 1u) == 0));
    const bool app = kAppend && last && it.part == it.nparts - 1;
    if constexpr (kAppend) {
      if (app && S.alen <= prm.cap) append_from_regs<T, D>(prm, pv, it, S.ablk, tile0, S.regs);
    }
    wave_lds_sync();  // previous tile's LDS reads are done
    if (full) stage_tile_ro<T, D, false>(lds, S.regs);
    else stage_tile_ro<T, D, true>(lds, S.regs);
    if constexpr (kAppend) {
      if (app && S.alen > prm.cap) {
        wave_lds_sync();
        unappend_lds<T, D>(prm, pv, it, S.ablk, tile0, lds);
      }
    }
    wave_lds_sync();
    // ---- S^T = K Q^T, online softmax, O^T += V^T P^T ----
    f32x4_t s[NH], s2[NH];
    tile_scores<T, D, HP>(lds, qv, s, s2);
    // the next item's query, once this item's is no longer needed, and before
    // the tile issued next: reading it then waits only for the tile already
    // in flight, which is staged first anyway (the next item's first tile is
    // issued, so it is queued, when this is the last tile)
    if (last && nqueued > 0) load_q<T, D, HP>(prm, make_item<false, Gm::TT, HP>(prm, qd0, qf0, per_item), qv);
    produce(S);
    own_half<NH, HP>(s, s2, prm.gs);
    tile_softmax_pv<T, D>(lds, it, tile0, s, m, l, o);
    if (!last) {
      ++ct;
      return false;
    }
    store_item<T, D, HP>(prm, it, m, l, o);
    if (nqueued == 0) return true;  // the producer is ahead: no queued item, no next item
    it = make_item<false, Gm::TT, HP>(prm, qd0, qf0, per_item);
    qd0 = qd1;
    qf0 = qf1;
    --nqueued;
    ct = 0;
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    return false;
  };

  produce(sa);
  produce(sb);
  for (;;) {
    if (consume(sa)) break;
    if (consume(sb)) break;
  }
}

// ---------------------------------------------------------------------------
// Reduce: merge the partitions of requests that have more than one; write
// zeros for empty requests.  One wave per (request, query head), four heads
// per block.  Lane i first turns partition i's (max, sum) into its weight
// 2^(m_i - m); the weighted sum over partitions then reads each weight with
// a lane broadcast while the partial outputs stream in, sixteen partitions
// per round so that many loads are in flight.  Lane l owns output elements
// D/64 * l .. D/64 * l + D/64 - 1 (one vector load per partition).
// ---------------------------------------------------------------------------
// Partial outputs: fp32, unnormalised, for fp32 requests; fp16 normalised by
// the partition's sum for bf16 requests.  Lane l reads elements PER*l ..
// PER*l + PER-1 of a partition's row with one load.
template <bool kHalf, int PER>
struct RowPiece;
template <>
struct RowPiece<false, 1> {
  typedef float type;
  static __device__ __forceinline__ float get(const type& v, int) { return v; }
};
template <>
struct RowPiece<false, 2> {
  typedef f32x2_t type;
  static __device__ __forceinline__ float get(const type& v, int j) { return v[j]; }
};
template <>
struct RowPiece<true, 1> {
  typedef uint16_t type;
  static __device__ __forceinline__ float get(const type& v, int) { return f16_lo(v); }
};
template <>
struct RowPiece<true, 2> {
  typedef uint32_t type;
  static __device__ __forceinline__ float get(const type& v, int j) { return j ? f16_hi(v) : f16_lo(v); }
};

// kRowMap: a mixed batch; only its decode requests (one-token chunks) are
// merged, into row cu[b], and requests without partials are left alone.
template <typename T, int D, bool kRowMap>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams prm) {
  constexpr int PER = D / 64;
  constexpr int U = 16;  // partitions per round
  constexpr bool kHalf = sizeof(T) == 2;
  typedef RowPiece<kHalf, PER> RP;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6), b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (h >= prm.Hq) return;
  const int64_t slot0 = ((int64_t)b * prm.Hq + h) * prm.max_parts;
  const f32x4_t* ml = reinterpret_cast<const f32x4_t*>(prm.ml) + slot0;
  // the (max, sum, scale) entries are read before the length is known (slots
  // past the request's partition count exist in the workspace and are masked
  // below), so the two loads overlap
  const f32x4_t ml0 = ml[min(lane, prm.max_parts - 1)];
  const int L = decode_len<kRowMap>(prm, b);
  const int np = (L + kPartTokens - 1) / kPartTokens;
  if (np == 1 || (kRowMap && np == 0)) return;
  const int64_t row = kRowMap ? prm.cu[b] : b;
  T* dst = static_cast<T*>(prm.out) + (row * prm.Hq + h) * D + PER * lane;
  if (np == 0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if constexpr (sizeof(T) == 2) dst[j] = 0;
      else dst[j] = 0.f;
    }
    return;
  }
  // global max over all partitions
  float mx = lane < np ? ml0[0] : -INFINITY;
  for (int i = lane + 64; i < np; i += 64) mx = fmaxf(mx, ml[i][0]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float den = 0.f;
  const typename RP::type* rows =
      kHalf ? reinterpret_cast<const typename RP::type*>(reinterpret_cast<const uint16_t*>(prm.o) + slot0 * D)
            : reinterpret_cast<const typename RP::type*>(prm.o + slot0 * D);
  for (int c0 = 0; c0 < np; c0 += 64) {  // chunks of 64 partitions
    const int nc = min(64, np - c0);
    const f32x4_t mine = c0 == 0 ? ml0 : ml[c0 + min(lane, nc - 1)];
    // lanes past the chunk hold whatever the workspace held: select, never
    // multiply, their values away
    const bool in = lane < nc;
    const float w = in ? fast_exp2(mine[0] - mx) : 0.f;
    float lw = in ? w * mine[1] : 0.f;
    // weight of a partial row: 2^(m_i - m) for unnormalised rows, times l_i and
    // the row's scale for normalised ones
    const float wr = kHalf ? (in ? lw * mine[2] : 0.f) : w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lw += __shfl_xor(lw, off);
    den += lw;
    const typename RP::type* src = rows + (size_t)c0 * (D / PER) + lane;
    for (int i = 0; i < nc; i += U) {
      typename RP::type v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = src[(size_t)min(i + u, nc - 1) * (D / PER)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = i + u < nc ? __shfl(wr, i + u) : 0.f;
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] = fmaf(wu, RP::get(v[u], j), acc[j]);
      }
    }
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if constexpr (sizeof(T) == 2) dst[j] = (bf16_bits)f32_to_bf16(acc[j] * inv);
    else dst[j] = acc[j] * inv;
  }
}

// Per-call salt of the counters' tag: a process-wide sequence from a start
// taken from the clock and the process id.
// Test knob, read on every call: PA_TEST_QUEUE_GIVEUP=1 makes every queue
// claim give up at once (the status word then reports it; the items left in
// the queues are not computed).  Lets a test see the give-up path with every
// kernel exiting normally.
inline int test_queue_giveup() {
  const char* e = getenv("PA_TEST_QUEUE_GIVEUP");
  return e && e[0] == '1' ? 1 : 0;
}

inline unsigned long long next_salt() {
  static std::atomic<unsigned long long> seq{
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() ^
      ((unsigned long long)getpid() << 40)};
  return seq.fetch_add(0x9E3779B97F4A7C15ull, std::memory_order_relaxed);
}

}  // namespace dec
}  // namespace pa
