// Training-time forward: every position of one sequence attends its own
// block selection; and the walk of its continuous-gate backward.
//
// SAS selects KV blocks for each query and trains with a Top-K of 31
// historical 64-token blocks on 32,768-token sequences ("Tencent released
// Simple-Attention-Sparsification ...", aigc.news; "Tencent Hunyuan
// open-sources SAS ...": per-query block selection).  Position t attends,
// causally, the blocks selected for it (its own block t/64 last), plain or
// with each historical block scaled by its continuous gate.
//
// One workgroup per (64-query block, KV head, group of kHW query heads).
// The workgroup marks the union of its queries' selections in an LDS bitmap
// and walks it two blocks at a time: for sequences of up to 512 blocks in a
// paired order (each block with a later one that no wave shares, each
// query's selection looked up in a per-query bitmap), else in ascending
// block order (each query's selection walked with a pointer).  Each visited block's K and V rows
// (32 KiB) are copied once into LDS by the gfx950 global-to-LDS loads
// (global_load_lds_dwordx4) and shared by all waves; a ring of four 32 KiB
// stages keeps the next three blocks in flight while one is consumed.  The
// copies are the only vector-memory operations of the walk (the selections of
// the 64 queries are staged in LDS first), so each iteration waits for
// exactly the copies of the block it consumes.
//
// The selections are sparse (31 of up to 511 blocks per query), so a wave's
// 16 MFMA columns hold few queries and all their heads: 16/kHW queries x kHW
// heads (kHW = 4 for groups of 3 or more heads, else the group size), and
// the workgroup has 4 kHW waves (64 queries).  A wave whose queries did not
// select a block skips it; with 4 queries per wave about a fifth of the
// waves work on each block of a 511-block union, against two thirds with 16
// queries per wave, for the same useful columns.
//
// Rows are stored unpadded (the copy writes 1 KiB per instruction) with a
// row-dependent XOR swizzle instead: K's 16-byte slots by row % 16 (the
// A-operand reads of 16 rows at one column hit 16 different slots), V's
// 32-byte pairs by row % 4 (the transposing reads of 4 rows x 32 bytes hit 4
// different pairs).  Per visited block a working wave forms
//   S^T (64 keys x 16 columns) = K . Q^T with v_mfma_f32_16x16x32_bf16, K
//     read from LDS as the A operand;
//   the column of a query that did not select the block is masked to -inf;
//     the query's own block is masked causally (key <= query);
//   online softmax in the log2 domain; O^T += V^T . P^T, V^T read with
//     ds_read_b64_tr_b16.
// 16 QK + 16 PV MFMAs per working wave and block.
#include <limits.h>

#include "prefill_backward.h"
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {
namespace {

constexpr int kRow = kHeadDim * 2;        // 256-byte K / V rows, unpadded
constexpr int kTile = kBlock * kRow;      // 16 KiB
constexpr int kStage = 2 * kTile;         // K tile, then V tile
constexpr int kStages = 4;                // ring: 3 blocks in flight + 1 consumed
constexpr int kMaxSel = 64;               // selections per query staged in LDS (budgets up to 4,096)
constexpr float kMaxSlack = 8.f;          // lag of the softmax's reference max behind the true max (log2 units)

// Wave layout for kHW heads per query column group: the wave's 16 MFMA
// columns are kQW queries x kHW heads (column j: query j / kHW, head j % kHW)
template <int kHW>
struct Layout {
  static constexpr int kWaves = 4 * kHW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQW = 16 / kHW;
  static constexpr int kCopies = kTile / 1024 / kWaves;  // 1 KiB copies per wave per tile (K or V)
};

__device__ __forceinline__ bf16x8 as_bf16(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 2^x by the hardware instruction (results below the normal range flush to
// zero, which a softmax weight can afford)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the four 16-lane rows of a wave for each lane position l%16
// (the lanes that hold one column), by the gfx950 row-swap moves:
// permlane16_swap pairs rows (0,1) and (2,3), permlane32_swap pairs the halves
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, b16x2));
}

// LDS of a walk: the ring first (1 KiB aligned), the union bitmap, the
// queries' selections (block indices) and counts
struct WalkLds {
  uint8_t ring[kStages][kStage];
  uint32_t bm[SAS_MAX_BLOCKS_DEV / 32];
  int16_t sel[kBlock][kMaxSel];
  int cnt[kBlock];
};

// The 64 queries' selections into LDS (gates too when gate_l is given) and
// their union as a bitmap over blocks 0 .. qb; returns the bitmap's words.
template <int kThreads>
__device__ __forceinline__ int stage_union(WalkLds &L, float (*gate_l)[kMaxSel], const int32_t *sel,
                                           const float *gates, const int32_t *cnt, int n_kv_heads, int kvh,
                                           int max_sel, int t0, int nq, int qb) {
  const int tid = threadIdx.x;
  const int nwords = (qb + 32) >> 5;
  for (int i = tid; i < nwords; i += kThreads) L.bm[i] = 0;
  if (tid < kBlock) L.cnt[tid] = tid < nq ? cnt[(int64_t)(t0 + tid) * n_kv_heads + kvh] : 0;
  __syncthreads();
  for (int e = tid; e < nq * max_sel; e += kThreads) {
    const int q = e / max_sel, slot = e - q * max_sel;
    if (slot < L.cnt[q]) {
      const int64_t u = ((int64_t)(t0 + q) * n_kv_heads + kvh) * max_sel + slot;
      int c = sel[u];
      c = (unsigned)c <= (unsigned)qb ? c : qb;  // out-of-range entries are not trusted
      L.sel[q][slot] = (int16_t)c;
      if (gate_l) gate_l[q][slot] = gates[u];
      atomicOr(&L.bm[c >> 5], 1u << (c & 31));
    }
  }
  return nwords;
}

// The ring's block copies: wave w writes 1 KiB pieces w kCopies .. of the K
// tile and of the V tile (4 rows each); lane i of a piece lands at byte 16i
// of it, so it fetches the global 16 bytes that the swizzle puts there.
// kVLikeK: V stored with K's swizzle (read as an A operand, not transposed).
template <int kHW, bool kVLikeK>
struct Ring {
  static constexpr int kC = Layout<kHW>::kCopies;
  const char *kbase, *vbase;
  const __attribute__((address_space(4))) int32_t *btc;  // the block table, read by scalar loads
  int64_t page_bytes, tok_bytes;
  uint32_t dst0;
  int wave;

  __device__ __forceinline__ Ring(const uint16_t *k_pool, const uint16_t *v_pool, const int32_t *block_table,
                                  int64_t page_stride, int64_t tok_stride, int64_t head_stride, int kvh,
                                  const uint8_t *ring0, int wave_) {
    kbase = reinterpret_cast<const char *>(k_pool) + (int64_t)kvh * head_stride * 2;
    vbase = reinterpret_cast<const char *>(v_pool) + (int64_t)kvh * head_stride * 2;
    btc = (const __attribute__((address_space(4))) int32_t *)block_table;
    page_bytes = page_stride * 2;
    tok_bytes = tok_stride * 2;
    wave = wave_;
    dst0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)ring0 + 1024 * kC * wave;
  }
  // the per-lane source offsets are recomputed at each copy (a few integer
  // operations) rather than held in registers across the walk
  __device__ __forceinline__ void copy(int c, int st) const { copy_page(btc[c], st); }
  // the same with the block's page already known (no block-table load)
  __device__ __forceinline__ void copy_page(int page, int st) const {
    const int64_t off = (int64_t)page * page_bytes;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(dst0 + st * kStage);
    const int lane = threadIdx.x & 63, sl = lane & 15;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      const int row = 4 * (kC * wave + k) + (lane >> 4);
      copy16(kbase + off + row * tok_bytes + 16 * (sl ^ (row & 15)), dst + 1024 * k);
    }
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      const int row = 4 * (kC * wave + k) + (lane >> 4);
      const int64_t col = kVLikeK ? 16 * (sl ^ (row & 15)) : 32 * ((sl >> 1) ^ (row & 3)) + 16 * (sl & 1);
      copy16(vbase + off + row * tok_bytes + col, dst + kTile + 1024 * k);
    }
  }
};

// uniform cursor over the union bitmap, ascending
struct Cursor {
  const uint32_t *bm;
  int wi, nwords;
  uint32_t bits;
  __device__ __forceinline__ Cursor(const uint32_t *bm_, int nwords_) : bm(bm_), wi(0), nwords(nwords_) {
    bits = __builtin_amdgcn_readfirstlane(bm[0]);
  }
  __device__ __forceinline__ int next() {
    while (bits == 0) {
      if (++wi >= nwords) return -1;
      bits = __builtin_amdgcn_readfirstlane(bm[wi]);
    }
    const int c = (wi << 5) + __builtin_ctz(bits);
    bits &= bits - 1;
    return c;
  }
};

// The walk: the first three blocks copied ahead (a missing one replaced by a
// copy of the first into its unused stage, to keep the copy count fixed),
// then per block: wait for its copies (at most the two later stages' copies
// outstanding), the workgroup barrier (block i-1's stage is free), the copy
// of block i+3 into that stage, visit(c, stage).  before_visit(c, stage)
// runs after the barrier (it may write the stage and must end with its own
// barrier).
template <int kHW, bool kVLikeK, typename Before, typename Visit>
__device__ __forceinline__ void walk(const Ring<kHW, kVLikeK> &ring, Cursor &cur, Before before_visit, Visit visit) {
  constexpr int kC = Layout<kHW>::kCopies;
  int c0 = cur.next();  // never -1: every query selects its own block
  int c1 = cur.next();
  int c2 = cur.next();
  ring.copy(c0, 0);
  ring.copy(c1 >= 0 ? c1 : c0, 1);
  ring.copy(c2 >= 0 ? c2 : c0, 2);
  for (int i = 0;; ++i) {
    const int st = i & (kStages - 1);
    const int c = c0;
    wait_vm<2 * 2 * kC>();  // this wave's copies of block i landed (blocks i+1, i+2 may be in flight)
    lds_barrier();          // ... and every other wave's; block i-1's stage is free
    before_visit(c, st);
    const int c3 = cur.next();
    ring.copy(c3 >= 0 ? c3 : c, (i + 3) & (kStages - 1));
    visit(c, st);
    if (c1 < 0) break;  // block i was the walk's last
    c0 = c1;
    c1 = c2;
    c2 = c3;
  }
  wait_vm<0>();  // the trailing filler copies land before the workgroup ends
}

// The same walk taking the blocks two at a time: one barrier per pair, the
// next pair's copies (into the stages of the previous pair) in flight while
// the current pair is visited by visit_pair(c0, stage0, c1, stage1) (c1 = -1
// for a last, unpaired block: no query selects it).  The waves that work on only one of the
// two overlap with those on the other, where the one-block walk makes every
// wave wait at the barrier after each block.  A wave whose queries selected
// both blocks sets the pair's pace, so visit_pair may interleave the two
// blocks' work for it (the backward's walk does; the forward's online
// softmax needs more registers for that than its 16-wave layout leaves).
template <int kHW, bool kVLikeK, typename Before, typename Visit, typename VisitPair>
__device__ __forceinline__ void walk_pairs(const Ring<kHW, kVLikeK> &ring, Cursor &cur, Before before_visit,
                                           Visit visit, VisitPair visit_pair) {
  int a0 = cur.next();  // never -1: every query selects its own block
  int a1 = cur.next();
  ring.copy(a0, 0);
  ring.copy(a1 >= 0 ? a1 : a0, 1);
  for (int k = 0;; ++k) {
    const int s0 = (2 * k) & (kStages - 1), s1 = (2 * k + 1) & (kStages - 1);
    wait_vm<0>();   // this wave's copies of the pair landed (nothing else is in flight)
    lds_barrier();  // ... and every other wave's; the previous pair's stages are free
    before_visit(a0, s0);
    if (a1 >= 0) before_visit(a1, s1);
    const int b0 = a1 >= 0 ? cur.next() : -1;
    const int b1 = b0 >= 0 ? cur.next() : -1;
    ring.copy(b0 >= 0 ? b0 : a0, (2 * k + 2) & (kStages - 1));  // a missing block: a filler copy, fixed count
    ring.copy(b1 >= 0 ? b1 : a0, (2 * k + 3) & (kStages - 1));
    visit_pair(a0, s0, a1, s1);  // a1 = -1: no second block (no query selects it)
    if (b0 < 0) break;  // the pair was the walk's last
    a0 = b0;
    a1 = b1;
  }
  wait_vm<0>();  // the trailing filler copies land before the workgroup ends
}
constexpr bool kWalkPairs = true;

// ---- the paired visiting order (sequences of up to kOrdBlocks blocks)
//
// Between two barriers the walk visits two blocks, and a wave whose queries
// selected both sets the pace (its two visits run back to back while the
// other waves wait).  With the blocks in ascending order that is the case
// for most pairs of a long union; paired greedily instead, each block with
// a later one that no wave shares, it is rare.  Each query's selection is
// then looked up per block in a bitmap (qbits) rather than walked in order.
constexpr int kOrdWords = 16;               // union bitmap words of a paired walk
constexpr int kOrdBlocks = 32 * kOrdWords;  // 512 blocks: 32,768 tokens

// qbits[q]: bit c set when query q selected block c; qpre[q][w]: the
// query's selected blocks in words 0 .. w-1, so that block c is its slot
// qpre[q][c/32] + (its selected blocks below c in word c/32)
template <int kThreads>
__device__ __forceinline__ void stage_query_bits(const WalkLds &L, uint32_t (*qbits)[kOrdWords],
                                                 uint8_t (*qpre)[kOrdWords]) {
  const int tid = threadIdx.x;
  for (int e = tid; e < kBlock * kOrdWords; e += kThreads) (&qbits[0][0])[e] = 0u;
  __syncthreads();
  for (int e = tid; e < kBlock * kMaxSel; e += kThreads) {
    const int q = e / kMaxSel, slot = e - q * kMaxSel;
    if (slot < L.cnt[q]) {
      const int c = L.sel[q][slot];
      if ((unsigned)c < (unsigned)kOrdBlocks) atomicOr(&qbits[q][c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  for (int e = tid; e < kBlock * kOrdWords; e += kThreads) {
    const int q = e / kOrdWords, w = e - q * kOrdWords;
    int a = 0;
    for (int v = 0; v < w; ++v) a += __builtin_popcount(qbits[q][v]);
    qpre[q][w] = (uint8_t)a;
  }
}

// The union's blocks in ascending order (ulist), each block's mask of the
// waves with a query that selected it (wmask), then, chunk by chunk of 64
// blocks (a wave per chunk), pairs taken greedily: each block not yet taken
// with the first later untaken block of its chunk that shares no wave with
// it, else the next untaken one.  Pair k is (order[2k], order[2k+1]); only
// the last pair of an odd union has no second block (-1).  The walk reads
// pair k as one 16-byte entry of the pair table (pair_table): each block
// with its wave mask in the upper 16 bits (0xFFFF: no second block), then
// the two blocks' pages (the first's again for a missing second block), so
// that it needs no block-table load and a wave skips a block none of its
// queries selected without reading their bitmaps.  The arrays take the
// place of the staged selections (L.sel), read into qbits before.  Returns
// the number of pairs; the caller synchronises before the walk.
__device__ __forceinline__ u32x4 *pair_table(WalkLds &L) {
  return reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(&L.sel[0][0]) + kOrdBlocks * (2 + 2 + 4));
}
template <int kThreads, int kQW>
__device__ __forceinline__ int stage_order(WalkLds &L, const uint32_t (*qbits)[kOrdWords], int *wpre, int nwords,
                                           const int32_t *block_table) {
  static_assert(sizeof(L.sel) >= kOrdBlocks * (2 + 2 + 4) + kOrdBlocks / 2 * 16,
                "order arrays exceed the selection buffer");
  static_assert(kThreads / 64 <= 16, "wave masks are 16 bits");
  int16_t *ulist = reinterpret_cast<int16_t *>(&L.sel[0][0]);
  int16_t *order = ulist + kOrdBlocks;
  uint32_t *wmask = reinterpret_cast<uint32_t *>(ulist + 2 * kOrdBlocks);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __syncthreads();  // L.sel is read no more
  for (int c = tid; c < kOrdBlocks; c += kThreads) wmask[c] = 0u;
  if (tid <= kOrdWords) {
    int a = 0;
    for (int v = 0; v < tid && v < nwords; ++v) a += __builtin_popcount(L.bm[v]);
    wpre[tid] = a;
  }
  __syncthreads();
  for (int c = tid; c < 32 * nwords; c += kThreads) {
    const uint32_t word = L.bm[c >> 5], bit = 1u << (c & 31);
    if (word & bit) ulist[wpre[c >> 5] + __builtin_popcount(word & (bit - 1u))] = (int16_t)c;
  }
  for (int e = tid; e < kBlock * kOrdWords; e += kThreads) {
    const int q = e / kOrdWords, w = e - q * kOrdWords;
    for (uint32_t bits = qbits[q][w]; bits; bits &= bits - 1u)
      atomicOr(&wmask[32 * w + __builtin_ctz(bits)], 1u << (q / kQW));
  }
  __syncthreads();
  const int n = wpre[nwords];
  constexpr int kWaves = kThreads / 64;
  for (int k = wave; 64 * k < n; k += kWaves) {
    const int cnt = min(64, n - 64 * k);
    const bool valid = lane < cnt;
    const int b = valid ? ulist[64 * k + lane] : 0;
    const uint32_t m = valid ? wmask[b] : 0u;
    uint64_t taken = 0;
    int pi = 0;
    for (int i = 0; i < cnt; ++i) {
      if ((taken >> i) & 1u) continue;
      taken |= 1ull << i;
      const uint32_t mi = (uint32_t)__builtin_amdgcn_readlane((int)m, i);
      const bool open = valid && lane > i && !((taken >> lane) & 1u);
      uint64_t cand = __builtin_amdgcn_ballot_w64(open && (m & mi) == 0u);
      if (cand == 0) cand = __builtin_amdgcn_ballot_w64(open);
      const int j = cand ? (int)__builtin_ctzll(cand) : -1;
      if (j >= 0) taken |= 1ull << j;
      const int bi = __builtin_amdgcn_readlane(b, i);
      const int bj = j >= 0 ? __builtin_amdgcn_readlane(b, j) : -1;
      if (lane == 0) {
        order[64 * k + 2 * pi] = (int16_t)bi;
        order[64 * k + 2 * pi + 1] = (int16_t)bj;
      }
      ++pi;
    }
  }
  __syncthreads();
  const int np = (n + 1) >> 1;
  u32x4 *pairs = pair_table(L);
  for (int i = tid; i < np; i += kThreads) {
    const int b0 = order[2 * i], b1 = order[2 * i + 1];
    const int pg0 = block_table[b0];
    pairs[i] = u32x4{(uint32_t)b0 | wmask[b0] << 16, b1 >= 0 ? (uint32_t)b1 | wmask[b1] << 16 : 0xFFFFu,
                     (uint32_t)pg0, (uint32_t)(b1 >= 0 ? block_table[b1] : pg0)};
  }
  return np;
}

// The walk of walk_pairs over the pair table of stage_order:
// visit_pair(c0, wm0, stage0, c1, wm1, stage1) with each block's wave mask
// (c1 = -1: no second block).  The next pair's entry is read before the
// barrier (the table does not change during the walk), so its copies go out
// right after it.
template <int kHW, bool kVLikeK, typename Before, typename VisitPair>
__device__ __forceinline__ void walk_ordered(const Ring<kHW, kVLikeK> &ring, const u32x4 *pairs, int npairs,
                                             Before before_visit, VisitPair visit_pair) {
  auto uni = [](uint32_t v) { return __builtin_amdgcn_readfirstlane((int)v); };
  const u32x4 e0 = pairs[0];
  int x0 = uni(e0.x), x1 = uni(e0.y);  // x0's block: never missing (every query selects its own block)
  ring.copy_page(uni(e0.z), 0);
  ring.copy_page(uni(e0.w), 1);  // a missing second block: a filler copy of the first, fixed count
  for (int k = 0; k < npairs; ++k) {
    const int s0 = (2 * k) & (kStages - 1), s1 = (2 * k + 1) & (kStages - 1);
    const u32x4 nx = pairs[k + 1 < npairs ? k + 1 : k];  // after the last pair: filler copies
    wait_vm<0>();   // this wave's copies of the pair landed (nothing else is in flight)
    lds_barrier();  // ... and every other wave's; the previous pair's stages are free
    const int a0 = x0 & 0xFFFF, a1 = (x1 & 0xFFFF) == 0xFFFF ? -1 : x1 & 0xFFFF;
    before_visit(a0, s0);
    if (a1 >= 0) before_visit(a1, s1);
    const int y0 = uni(nx.x), y1 = uni(nx.y);
    ring.copy_page(uni(nx.z), (2 * k + 2) & (kStages - 1));
    ring.copy_page(uni(nx.w), (2 * k + 3) & (kStages - 1));
    visit_pair(a0, (uint32_t)x0 >> 16, s0, a1, (uint32_t)x1 >> 16, s1);
    x0 = y0;
    x1 = y1;
  }
  wait_vm<0>();  // the trailing filler copies land before the workgroup ends
}

// blockIdx -> (query block, KV head, head group): heaviest query blocks
// first, consecutive workgroups on different KV heads
struct Tile {
  int hg, kvh, qb, t0, nq;
};
__device__ __forceinline__ Tile tile_of(int head_groups, int n_kv_heads, int n_qblocks, int seq_len) {
  Tile w;
  w.hg = blockIdx.x % head_groups;
  const int rest = blockIdx.x / head_groups;
  w.kvh = rest % n_kv_heads;
  w.qb = n_qblocks - 1 - rest / n_kv_heads;
  w.t0 = w.qb * kBlock;
  w.nq = min(kBlock, seq_len - w.t0);
  return w;
}

}  // namespace

template <bool kGated, int kHW, bool kOrdered>
__global__ __launch_bounds__(Layout<kHW>::kThreads, 1) void prefill_attend_kernel(PrefillParams p) {
  using Lay = Layout<kHW>;
  __shared__ __attribute__((aligned(1024))) WalkLds L;
  __shared__ float gate_l[kGated ? kBlock : 1][kMaxSel];
  __shared__ uint32_t qbits[kOrdered ? kBlock : 1][kOrdWords];
  __shared__ uint8_t qpre[kOrdered ? kBlock : 1][kOrdWords];
  __shared__ int wpre[kOrdWords + 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int G = p.group;
  const Tile w = tile_of(p.head_groups, p.n_kv_heads, p.n_qblocks, p.seq_len);
  const int nh = min(kHW, G - kHW * w.hg);  // heads of this workgroup (>= 1)
  const int qi = Lay::kQW * wave + j / kHW;  // this lane's column: query within the block, and head
  const int hh = j % kHW;
  const bool qvalid = qi < w.nq;
  const bool cvalid = qvalid && hh < nh;
  const int tq = w.t0 + qi;
  const int64_t qrow = (int64_t)(cvalid ? tq : 0) * p.n_q_heads + w.kvh * G + (cvalid ? kHW * w.hg + hh : 0);

  const int nwords = stage_union<Lay::kThreads>(L, kGated ? gate_l : nullptr, p.sel, p.gates, p.cnt, p.n_kv_heads,
                                                w.kvh, p.max_sel, w.t0, w.nq, w.qb);
  int npairs = 0;
  if constexpr (kOrdered) {
    __syncthreads();
    stage_query_bits<Lay::kThreads>(L, qbits, qpre);
    npairs = stage_order<Lay::kThreads, Lay::kQW>(L, qbits, wpre, nwords, p.block_table);
  }

  // B operand of S^T = K Q^T: lane l holds q[its column][32ks + 8(l/16) .. +7]
  bf16x8 qB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qB[ks] = as_bf16(cvalid ? ld16(p.q + qrow * kHeadDim + 8 * g + 32 * ks) : u32x4{0, 0, 0, 0});
  wait_vm<0>();  // every compiler-visible load done before the copies start
  __syncthreads();

  // ---- this lane's walk through its query's ascending selection (LDS;
  // the paired order looks each block up in the query's bitmap instead)
  const int cq = kOrdered ? 0 : L.cnt[qi];
  int ptr = 0;
  int nxt_c = !kOrdered && cq > 0 ? L.sel[qi][0] : INT_MAX;

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), ls = 0.f;

  const Ring<kHW, false> ring(p.k_pool, p.v_pool, p.block_table, p.page_stride, p.tok_stride, p.head_stride, w.kvh,
                              &L.ring[0][0], wave);
  Cursor cur(L.bm, nwords);
  const int T = p.seq_len;
  // transposed V reads: within the 16-lane group g, lane 4e+q4 addresses row
  // 4g+e (+16 for the upper half of a k-step, +32 per k-step), bytes 8q4 of
  // the 32-byte pair dt, stored at pair dt ^ e (row % 4 == e).  The pair's low
  // two bits take the XOR; its high bit, the k-step and the half are
  // constant offsets, so four per-lane offsets serve all 32 reads.
  uint32_t tr_off[4];
  {
    const int tr_e = (lane & 15) >> 2, tr_q = lane & 3;
#pragma unroll
    for (int d3 = 0; d3 < 4; ++d3) tr_off[d3] = (4 * g + tr_e) * kRow + 32 * (d3 ^ tr_e) + 8 * tr_q;
  }
  auto before = [&](int c, int st) {
         if (c * kBlock + kBlock > T) {  // the sequence's last, partial block: zero V rows past the end
           uint8_t *vt = L.ring[st] + kTile;
           for (int b = tid * 16 + (T - c * kBlock) * kRow; b < kTile; b += Lay::kThreads * 16)
             *reinterpret_cast<u32x4 *>(vt + b) = u32x4{0, 0, 0, 0};
           lds_barrier();
         }
       };
  // wm: the waves with a query that selected c (the paired order; all ones
  // for the ascending walk, whose waves test their queries' pointers)
  auto visit = [&](int c, uint32_t wm, int st) {
         if (kOrdered && ((wm >> wave) & 1u) == 0u) return;
         bool s_l;
         float g_l = 0.f;
         if constexpr (kOrdered) {
           // the query's bitmap word of c and its prefix count, read together,
           // so that the gate's slot is known one LDS round trip in and its
           // read goes out with the key tiles'
           const uint32_t wb = qbits[kOrdered ? qi : 0][c >> 5], bit = 1u << (c & 31);
           const int pre = qpre[kOrdered ? qi : 0][c >> 5];
           s_l = (wb & bit) != 0u;
           if constexpr (kGated) {  // read whether or not the query selected c (no branch)
             const float gv = gate_l[kGated ? qi : 0][min(pre + __builtin_popcount(wb & (bit - 1u)), kMaxSel - 1)];
             g_l = s_l ? gv : 0.f;
           }
         } else {
           s_l = nxt_c == c;
           g_l = kGated && s_l ? gate_l[kGated ? qi : 0][ptr] : 0.f;
           if (s_l) {
             ++ptr;
             nxt_c = ptr < cq ? L.sel[qi][ptr] : INT_MAX;
           }
           if (__builtin_amdgcn_ballot_w64(s_l) == 0) return;
         }
         const uint8_t *kt = L.ring[st];
         const uint8_t *vt = L.ring[st] + kTile;
         f32x4 sacc[4];  // [key tile]
#pragma unroll
         for (int t = 0; t < 4; ++t) {
           u32x4 ka[4];
#pragma unroll
           for (int ks = 0; ks < 4; ++ks)
             ka[ks] = *reinterpret_cast<const u32x4 *>(kt + (16 * t + j) * kRow + 16 * ((4 * ks + g) ^ j));
           sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
           for (int ks = 0; ks < 4; ++ks)
             sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(ka[ks]), qB[ks], sacc[t], 0, 0, 0);
         }
         // a block before the query's own is whole and visible: the column's
         // mask is one term added to every exponent (-inf for a query that did
         // not select the block); the own block (uniform branch) masks per key
         const bool causal = c == w.qb;
         float arg[4][4];  // exponents, relative to the new running max
         float mx;
         if (!causal) {
           float mr = -__builtin_inff();
#pragma unroll
           for (int t = 0; t < 4; ++t)
#pragma unroll
             for (int r = 0; r < 4; ++r) mr = fmaxf(mr, sacc[t][r]);
           mx = s_l ? mr * p.scale_log2 : -__builtin_inff();
         } else {
           mx = -__builtin_inff();
#pragma unroll
           for (int t = 0; t < 4; ++t)
#pragma unroll
             for (int r = 0; r < 4; ++r) {
               const bool keep = s_l && 16 * t + 4 * g + r <= qi;
               arg[t][r] = keep ? sacc[t][r] * p.scale_log2 : -__builtin_inff();
               mx = fmaxf(mx, arg[t][r]);
             }
         }
         mx = rows_max(mx);
         // the reference max moves only when a block's max exceeds it by more
         // than kMaxSlack (log2 units), so the output's rescale is rare: the
         // weights then reach at most 2^kMaxSlack, exact in fp32 and in bf16's
         // range, and the normalisation uses the same reference
         const float m_new = mx > m + kMaxSlack ? mx : m;
         const bool live = m_new != -__builtin_inff();
         const float alpha = live ? fast_exp2(m - m_new) : 1.0f;
         if (!causal) {
           const float nb = s_l && live ? -m_new : -__builtin_inff();
#pragma unroll
           for (int t = 0; t < 4; ++t)
#pragma unroll
             for (int r = 0; r < 4; ++r) arg[t][r] = fmaf(sacc[t][r], p.scale_log2, nb);
         } else {
#pragma unroll
           for (int t = 0; t < 4; ++t)
#pragma unroll
             for (int r = 0; r < 4; ++r) arg[t][r] = live ? arg[t][r] - m_new : -__builtin_inff();
         }
         float psum = 0.f;
         u32x4 pB[2];
#pragma unroll
         for (int s2 = 0; s2 < 2; ++s2) {
           float pv[8];
#pragma unroll
           for (int e = 0; e < 8; ++e) {
             const int t = 2 * s2 + (e >> 2), r = e & 3;
             const float pe = fast_exp2(arg[t][r]);
             psum += pe;
             pv[e] = kGated ? pe * g_l : pe;
           }
           pB[s2] = u32x4{pack_rne(pv[0], pv[1]), pack_rne(pv[2], pv[3]), pack_rne(pv[4], pv[5]),
                          pack_rne(pv[6], pv[7])};
         }
         ls = ls * alpha + psum;
         m = m_new;
         // the running max rarely moves once a query has seen a few blocks (and
         // never for a query that did not select this one): rescale only then
         if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
           for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
         }
         // O^T += V^T P^T in 16 steps (k-step s2 = i / 8, output tile dt =
         // i % 8): step i + 1's V^T operand is read while step i's product
         // runs, so that the reads do not wait one by one
         auto vread = [&](int i) {
           const int s2 = i >> 3, dt = i & 7;
           const uint8_t *vrd = vt + tr_off[dt & 3] + 128 * (dt >> 2) + 32 * s2 * kRow;
           const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)vrd);
           const i16x4 a1 =
               __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(vrd + 16 * kRow));
           const u32x2 lo2 = __builtin_bit_cast(u32x2, a0), hi2 = __builtin_bit_cast(u32x2, a1);
           return u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
         };
         u32x4 va = vread(0);
#pragma unroll
         for (int i = 0; i < 16; ++i) {
           const u32x4 vn = i + 1 < 16 ? vread(i + 1) : va;
           o[i & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(va), as_bf16(pB[i >> 3]), o[i & 7], 0, 0, 0);
           va = vn;
         }
       };
  // the two blocks of a pair in turn (c1 = -1: no second block)
  auto visit_pair_m = [&](int c0, uint32_t wm0, int st0, int c1, uint32_t wm1, int st1) {
    visit(c0, wm0, st0);
    if (c1 >= 0) visit(c1, wm1, st1);
  };
  if constexpr (kOrdered) {
    walk_ordered(ring, pair_table(L), npairs, before, visit_pair_m);
  } else {
    auto visit1 = [&](int c, int st) { visit(c, ~0u, st); };
    auto visit_pair = [&](int c0, int st0, int c1, int st1) { visit_pair_m(c0, ~0u, st0, c1, ~0u, st1); };
    if (kWalkPairs) walk_pairs(ring, cur, before, visit1, visit_pair);
    else walk(ring, cur, before, visit1);
  }

  // ---- normalise and store: lane holds dims 16dt + 4(l/16) .. +3 of its column
  const float l = rows_sum(ls);
  if (cvalid) {
    const float inv = 1.0f / l;
    uint16_t *dst = p.out + qrow * kHeadDim + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 v = o[dt] * inv;
      *reinterpret_cast<u32x2 *>(dst + 16 * dt) = u32x2{pack_rne(v[0], v[1]), pack_rne(v[2], v[3])};
    }
    // log-sum-exp of the (ungated) logits, natural log: (m + log2 l) ln 2
    if (p.lse && g == 0) p.lse[qrow] = (m + log2f(l)) * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------- backward: dL/dg of every selected block
// The gradient of the gated output with respect to each selected block's
// continuous gate, for the backward of the training-time forward:
//   dg_i = sum_{h in group} sum_{j in block c_i, j <= t} P_hj <dO_h, v_j>,
// with P_hj = 2^(z_hj - lse2_h) from the forward's log-sum-exp (the plain
// softmax over the query's selected tokens; the gates scale the blocks'
// shares afterwards).  The walk and the wave layout are the forward's; per
// block a working wave forms S^T = K Q^T and D^T = V dO^T on MFMA (V is read
// like K, as the A operand, so it is stored with K's swizzle), then per
// column the sum over the block's keys of P * D, and per query the sum over
// its kHW head columns, written to the query's slot in LDS (each query's
// heads are all in one wave: one write per slot).  A group of G > 4 heads
// spans several workgroups, whose partial sums the chain kernel adds in
// order.
template <int kHW, bool kOrdered>
__global__ __launch_bounds__(Layout<kHW>::kThreads, 1) void prefill_grad_kernel(PrefillBackwardParams p) {
  using Lay = Layout<kHW>;
  __shared__ __attribute__((aligned(1024))) WalkLds L;
  __shared__ float dg_l[kBlock][kMaxSel];
  __shared__ uint32_t qbits[kOrdered ? kBlock : 1][kOrdWords];
  __shared__ uint8_t qpre[kOrdered ? kBlock : 1][kOrdWords];
  __shared__ int wpre[kOrdWords + 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int G = p.group;
  const Tile w = tile_of(p.head_groups, p.n_kv_heads, p.n_qblocks, p.seq_len);
  const int nh = min(kHW, G - kHW * w.hg);
  const int qi = Lay::kQW * wave + j / kHW;
  const int hh = j % kHW;
  const bool qvalid = qi < w.nq;
  const bool cvalid = qvalid && hh < nh;
  const int tq = w.t0 + qi;
  const int64_t qrow = (int64_t)(cvalid ? tq : 0) * p.n_q_heads + w.kvh * G + (cvalid ? kHW * w.hg + hh : 0);

  for (int e = tid; e < kBlock * kMaxSel; e += Lay::kThreads) (&dg_l[0][0])[e] = 0.f;
  const int nwords = stage_union<Lay::kThreads>(L, nullptr, p.sel, nullptr, p.cnt, p.n_kv_heads, w.kvh, p.max_sel,
                                                w.t0, w.nq, w.qb);

  // B operands (q and dO of this lane's column) and the forward's
  // log-sum-exp in log2 units
  bf16x8 qB[4], dB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qB[ks] = as_bf16(cvalid ? ld16(p.q + qrow * kHeadDim + 8 * g + 32 * ks) : u32x4{0, 0, 0, 0});
    dB[ks] = as_bf16(cvalid ? ld16(p.d_out + qrow * kHeadDim + 8 * g + 32 * ks) : u32x4{0, 0, 0, 0});
  }
  const float lse2 = cvalid ? p.lse[qrow] * kLog2e : 0.f;
  wait_vm<0>();  // every compiler-visible load done before the copies start
  __syncthreads();

  int npairs = 0;
  if constexpr (kOrdered) {
    stage_query_bits<Lay::kThreads>(L, qbits, qpre);
    npairs = stage_order<Lay::kThreads, Lay::kQW>(L, qbits, wpre, nwords, p.block_table);
    __syncthreads();
  }
  const int cq = kOrdered ? 0 : L.cnt[qi];
  int ptr = 0;
  int nxt_c = !kOrdered && cq > 0 ? L.sel[qi][0] : INT_MAX;

  const Ring<kHW, true> ring(p.k_pool, p.v_pool, p.block_table, p.page_stride, p.tok_stride, p.head_stride, w.kvh,
                             &L.ring[0][0], wave);
  Cursor cur(L.bm, nwords);
  // whether this lane's query selected block c, and the slot it takes
  auto advance = [&](int c, int &slot) {
    if constexpr (kOrdered) {
      if (c < 0) return false;  // no second block
      const uint32_t wb = qbits[kOrdered ? qi : 0][c >> 5], bit = 1u << (c & 31);
      slot = qpre[kOrdered ? qi : 0][c >> 5] + __builtin_popcount(wb & (bit - 1u));
      return (wb & bit) != 0u;
    } else {
      const bool s_l = nxt_c == c;
      slot = ptr;
      if (s_l) {
        ++ptr;
        nxt_c = ptr < cq ? L.sel[qi][ptr] : INT_MAX;
      }
      return s_l;
    }
  };
  // key tile t of the block in stage st: this lane's sum over its 4 keys of
  // P * D.  Keys the query may not see (later keys of its own block, rows
  // past the sequence end) are dropped by a select on the own block, so
  // that whatever such rows hold never enters the sum.
  auto tile_sum = [&](int st, int t, bool causal, float acc) {
    const uint8_t *kt = L.ring[st];
    const uint8_t *vt = L.ring[st] + kTile;
    u32x4 ka[4], va[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int off = (16 * t + j) * kRow + 16 * ((4 * ks + g) ^ j);
      ka[ks] = *reinterpret_cast<const u32x4 *>(kt + off);
      va[ks] = *reinterpret_cast<const u32x4 *>(vt + off);
    }
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(ka[ks]), qB[ks], sacc, 0, 0, 0);
      dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(va[ks]), dB[ks], dacc, 0, 0, 0);
    }
    if (!causal) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = fmaf(fast_exp2(fmaf(sacc[r], p.scale_log2, -lse2)), dacc[r], acc);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool keep = 16 * t + 4 * g + r <= qi;
        const float pe = fast_exp2(sacc[r] * p.scale_log2 - lse2);
        acc += keep ? pe * dacc[r] : 0.f;
      }
    }
    return acc;
  };
  // the column sums of one block to the query's slot: a query that did not
  // select the block contributes nothing (the select also drops whatever
  // its column computed); the query's kHW head columns are adjacent lanes
  auto finish = [&](float acc, bool s_l, int slot) {
    acc = s_l ? acc : 0.f;
    acc = rows_sum(acc);
    if (kHW >= 2) acc += __shfl_xor(acc, 1, 64);
    if (kHW >= 4) acc += __shfl_xor(acc, 2, 64);
    if (s_l && g == 0 && hh == 0) dg_l[qi][slot] = acc;
  };
  auto block_sum = [&](int c, int st) {
    const bool causal = c == w.qb;
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = tile_sum(st, t, causal, acc);
    return acc;
  };
  auto visit = [&](int c, int st) {
    int slot;
    const bool s_l = advance(c, slot);
    if (__builtin_amdgcn_ballot_w64(s_l) != 0) finish(block_sum(c, st), s_l, slot);
  };
  // two blocks (c0 < c1: only c1 can be a query's own block) with their wave
  // masks (m: the waves with a query that selected the block; all ones for
  // the ascending walk, whose waves test their queries' pointers); a wave
  // with queries in both whole blocks works on the two key tiles side by side
  auto visit_pair_m = [&](int c0, uint32_t wm0, int st0, int c1, uint32_t wm1, int st1) {
    if (kOrdered && ((wm0 >> wave) & 1u) == 0u && (c1 < 0 || ((wm1 >> wave) & 1u) == 0u)) return;
    int slot0, slot1;
    const bool s0 = advance(c0, slot0);
    const bool s1 = advance(c1, slot1);
    const bool any0 = kOrdered ? ((wm0 >> wave) & 1u) != 0u : __builtin_amdgcn_ballot_w64(s0) != 0;
    const bool any1 = kOrdered ? c1 >= 0 && ((wm1 >> wave) & 1u) != 0u : __builtin_amdgcn_ballot_w64(s1) != 0;
    if (!any0 || !any1 || c0 == w.qb || c1 == w.qb) {
      if (any0) finish(block_sum(c0, st0), s0, slot0);
      if (any1) finish(block_sum(c1, st1), s1, slot1);
      return;
    }
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc0 = tile_sum(st0, t, false, acc0);
      acc1 = tile_sum(st1, t, false, acc1);
    }
    finish(acc0, s0, slot0);
    finish(acc1, s1, slot1);
  };
  auto visit_pair = [&](int c0, int st0, int c1, int st1) { visit_pair_m(c0, ~0u, st0, c1, ~0u, st1); };
  if constexpr (kOrdered)
    walk_ordered(ring, pair_table(L), npairs, [&](int, int) {}, visit_pair_m);
  else if (kWalkPairs) walk_pairs(ring, cur, [&](int, int) {}, visit, visit_pair);
  else walk(ring, cur, [&](int, int) {}, visit);
  __syncthreads();
  float *dst = p.ws_dgp + (((int64_t)w.hg * p.seq_len + w.t0) * p.n_kv_heads + w.kvh) * p.max_sel;
  for (int e = tid; e < w.nq * p.max_sel; e += Lay::kThreads) {
    const int q = e / p.max_sel, slot = e - q * p.max_sel;
    dst[(int64_t)q * p.n_kv_heads * p.max_sel + slot] = dg_l[q][slot];
  }
}

namespace {
template <int kHW>
hipError_t launch_attend_hw(PrefillParams p, hipStream_t st) {
  p.head_groups = (p.group + kHW - 1) / kHW;
  const dim3 grid((unsigned)(p.n_qblocks * p.n_kv_heads * p.head_groups));
  // the paired order for sequences of up to kOrdBlocks blocks (its bitmaps' size)
  const bool ordered = p.n_qblocks <= kOrdBlocks;
  if (p.gates && ordered)
    hipLaunchKernelGGL((prefill_attend_kernel<true, kHW, true>), grid, dim3(Layout<kHW>::kThreads), 0, st, p);
  else if (p.gates)
    hipLaunchKernelGGL((prefill_attend_kernel<true, kHW, false>), grid, dim3(Layout<kHW>::kThreads), 0, st, p);
  else if (ordered)
    hipLaunchKernelGGL((prefill_attend_kernel<false, kHW, true>), grid, dim3(Layout<kHW>::kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((prefill_attend_kernel<false, kHW, false>), grid, dim3(Layout<kHW>::kThreads), 0, st, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill_attend(const PrefillParams &p, hipStream_t st) {
  switch (prefill_heads_per_wave(p.group)) {
    case 1: return launch_attend_hw<1>(p, st);
    case 2: return launch_attend_hw<2>(p, st);
    default: return launch_attend_hw<4>(p, st);
  }
}

hipError_t launch_prefill_grad(const PrefillBackwardParams &p, hipStream_t st) {
  const int hw = prefill_heads_per_wave(p.group);
  const dim3 grid((unsigned)(p.n_qblocks * p.n_kv_heads * p.head_groups));
  const bool ordered = p.n_qblocks <= kOrdBlocks;  // the paired order (its bitmaps' size)
  if (hw == 1 && ordered)
    hipLaunchKernelGGL((prefill_grad_kernel<1, true>), grid, dim3(Layout<1>::kThreads), 0, st, p);
  else if (hw == 1)
    hipLaunchKernelGGL((prefill_grad_kernel<1, false>), grid, dim3(Layout<1>::kThreads), 0, st, p);
  else if (hw == 2 && ordered)
    hipLaunchKernelGGL((prefill_grad_kernel<2, true>), grid, dim3(Layout<2>::kThreads), 0, st, p);
  else if (hw == 2)
    hipLaunchKernelGGL((prefill_grad_kernel<2, false>), grid, dim3(Layout<2>::kThreads), 0, st, p);
  else if (ordered)
    hipLaunchKernelGGL((prefill_grad_kernel<4, true>), grid, dim3(Layout<4>::kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((prefill_grad_kernel<4, false>), grid, dim3(Layout<4>::kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
