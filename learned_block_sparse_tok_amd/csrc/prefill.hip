// Training-time forward: every position of one sequence attends its own
// block selection.
//
// SAS selects KV blocks for each query and trains with a Top-K of 31
// historical 64-token blocks on 32,768-token sequences ("Tencent released
// Simple-Attention-Sparsification ...", aigc.news; "Tencent Hunyuan
// open-sources SAS ...": per-query block selection).  Position t attends,
// causally, the blocks selected for it (its own block t/64 last), plain or
// with each historical block scaled by its continuous gate.
//
// One 512-thread workgroup per (64-query block, KV head, group of up to 4
// query heads).  The workgroup marks the union of its queries' selections in
// an LDS bitmap and walks it in ascending block order.  Each visited block's
// K and V rows (32 KiB) are copied once into LDS by the gfx950 global-to-LDS
// loads (global_load_lds_dwordx4) and shared by the 4 waves; a ring of four
// 32 KiB stages keeps the next three blocks in flight while one is consumed.
// Eight waves, two per SIMD, so that one wave's softmax runs while the
// other's matrix products do.
// The copies are the only vector-memory operations of the walk (the
// selections of the 64 queries are staged in LDS first), so each iteration
// waits for exactly the copies of the block it consumes.
// Rows are stored unpadded (the copy writes 1 KiB per instruction) with a
// row-dependent XOR swizzle instead: K's 16-byte slots by row % 16 (the
// A-operand reads of 16 rows at one column hit 16 different slots), V's
// 32-byte pairs by row % 4 (the transposing reads of 4 rows x 32 bytes hit 4
// different pairs).  Wave w owns queries 16(w%4) .. 16(w%4)+15 of the block
// and two of the group's heads, 2(w/4) and 2(w/4)+1:
//   S^T (64 keys x 16 queries) = K . Q^T per head with
//     v_mfma_f32_16x16x32_bf16, K read from LDS as the A operand;
//   the lane of a query that did not select the block masks its column to
//     -inf; the query's own block is masked causally (key <= query);
//   online softmax in the log2 domain; O^T += V^T . P^T, V^T read with
//     ds_read_b64_tr_b16.
// A wave none of whose 16 queries selected the block skips its arithmetic.
// The work is a dense contraction per visited block: 2 heads x (16 QK + 16
// PV) MFMAs x 2 per wave.
#include <limits.h>

#include "prefill_backward.h"
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {
namespace {

constexpr int kThreads = 512;  // 8 waves: 4 query quarters x 2 head pairs, two waves per SIMD
constexpr int kRow = kHeadDim * 2;        // 256-byte K / V rows, unpadded
constexpr int kTile = kBlock * kRow;      // 16 KiB
constexpr int kStage = 2 * kTile;         // K tile, then V tile
constexpr int kStages = 4;                // ring: 3 blocks in flight + 1 consumed
constexpr int kCopies = kStage / 1024 / 8;  // 1 KiB copy instructions per wave per stage: 4
constexpr int kCt = 2;                      // query heads per wave
constexpr int kMaxSel = 64;               // selections per query staged in LDS (budgets up to 4,096)

__device__ __forceinline__ bf16x8 as_bf16(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 2^x by the hardware instruction (results below the normal range flush to
// zero, which a softmax weight can afford)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the four 16-lane rows of a wave for each lane position l%16
// (the lanes that hold one query's column), by the gfx950 row-swap moves:
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

}  // namespace

template <bool kGated>
__global__ __launch_bounds__(kThreads, 1) void prefill_attend_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][kStage];
  __shared__ uint32_t bm[SAS_MAX_BLOCKS_DEV / 32];
  __shared__ int16_t sel_l[kBlock][kMaxSel];
  __shared__ float gate_l[kGated ? kBlock : 1][kMaxSel];
  __shared__ int cnt_l[kBlock];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int G = p.group;
  // blockIdx -> (query block, KV head, head group): heaviest query blocks
  // first, consecutive workgroups on different KV heads
  const int hg = blockIdx.x % p.head_groups;
  const int rest = blockIdx.x / p.head_groups;
  const int kvh = rest % p.n_kv_heads;
  const int qb = p.n_qblocks - 1 - rest / p.n_kv_heads;
  const int nh = min(4, G - 4 * hg);  // heads of this workgroup (>= 1)
  const int T = p.seq_len;
  const int t0 = qb * kBlock;
  const int nq = min(kBlock, T - t0);
  const int qw = wave & 3, hp = wave >> 2;  // query quarter, head pair
  const int qi = 16 * qw + j;              // this lane's query within the block
  const int h_lo = 4 * hg + 2 * hp;        // this wave's first query head within the group
  const bool qvalid = qi < nq;
  const int tq = t0 + qi;

  // ---- the queries' selections into LDS and their union (blocks 0 .. qb)
  const int nwords = (qb + 32) >> 5;
  for (int i = tid; i < nwords; i += kThreads) bm[i] = 0;
  if (tid < kBlock) cnt_l[tid] = tid < nq ? p.cnt[(int64_t)(t0 + tid) * p.n_kv_heads + kvh] : 0;
  __syncthreads();
  for (int e = tid; e < nq * p.max_sel; e += kThreads) {
    const int q = e / p.max_sel, slot = e - q * p.max_sel;
    if (slot < cnt_l[q]) {
      const int64_t u = ((int64_t)(t0 + q) * p.n_kv_heads + kvh) * p.max_sel + slot;
      int c = p.sel[u];
      c = (unsigned)c <= (unsigned)qb ? c : qb;  // out-of-range entries are not trusted
      sel_l[q][slot] = (int16_t)c;
      if (kGated) gate_l[kGated ? q : 0][slot] = p.gates[u];
      atomicOr(&bm[c >> 5], 1u << (c & 31));
    }
  }

  // B operand of S^T = K Q^T: lane l holds q[query qi][head][32ks + 8(l/16) .. +7]
  bf16x8 qB[kCt][4];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    const bool ok = qvalid && 2 * hp + ct < nh;
    const uint16_t *qrow =
        p.q + ((int64_t)(ok ? tq : 0) * p.n_q_heads + kvh * G + (ok ? h_lo + ct : 0)) * kHeadDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qB[ct][ks] = as_bf16(ok ? ld16(qrow + 32 * ks) : u32x4{0, 0, 0, 0});
  }
  wait_vm<0>();  // every compiler-visible load done before the copies start
  __syncthreads();

  // ---- this lane's walk through its query's ascending selection (LDS)
  const int cq = cnt_l[qi];
  int ptr = 0;
  int nxt_c = cq > 0 ? sel_l[qi][0] : INT_MAX;
  float nxt_g = kGated ? gate_l[kGated ? qi : 0][0] : 1.f;

  f32x4 o[kCt][8];
  float m[kCt], ls[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[ct] = -__builtin_inff();
    ls[ct] = 0.f;
  }

  // ---- block copies into the ring: wave w writes 1 KiB pieces 2w, 2w+1 of
  // the K tile and of the V tile (4 rows each); lane i of a piece lands at
  // byte 16i of it, so it fetches the global 16 bytes that the swizzle puts
  // there
  const char *kbase = reinterpret_cast<const char *>(p.k_pool) + (int64_t)kvh * p.head_stride * 2;
  const char *vbase = reinterpret_cast<const char *>(p.v_pool) + (int64_t)kvh * p.head_stride * 2;
  const int64_t tok_bytes = p.tok_stride * 2, page_bytes = p.page_stride * 2;
  int64_t k_src[kCopies / 2], v_src[kCopies / 2];  // per-lane byte offsets inside a block
#pragma unroll
  for (int k = 0; k < kCopies / 2; ++k) {
    const int row = 4 * (2 * wave + k) + (lane >> 4), sl = lane & 15;
    k_src[k] = row * tok_bytes + 16 * (sl ^ (row & 15));
    v_src[k] = row * tok_bytes + 32 * ((sl >> 1) ^ (row & 3)) + 16 * (sl & 1);
  }
  // the block table is read-only here: read it through the constant address
  // space so that a uniform index gives a scalar load
  const __attribute__((address_space(4))) int32_t *btc =
      (const __attribute__((address_space(4))) int32_t *)p.block_table;
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)&ring[0][0];
  auto copy_block = [&](int c, int st) {
    const int64_t off = (int64_t)btc[c] * page_bytes;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring0 + st * kStage + 2048 * wave);
#pragma unroll
    for (int k = 0; k < kCopies / 2; ++k) copy16(kbase + off + k_src[k], dst + 1024 * k);
#pragma unroll
    for (int k = 0; k < kCopies / 2; ++k) copy16(vbase + off + v_src[k], dst + kTile + 1024 * k);
  };
  // uniform cursor over the bitmap
  int wi = 0;
  uint32_t bits = __builtin_amdgcn_readfirstlane(bm[0]);
  auto next_block = [&]() -> int {
    while (bits == 0) {
      if (++wi >= nwords) return -1;
      bits = __builtin_amdgcn_readfirstlane(bm[wi]);
    }
    const int c = (wi << 5) + __builtin_ctz(bits);
    bits &= bits - 1;
    return c;
  };

  // prologue: the first three blocks of the walk (a missing one is replaced
  // by a copy of the first into its unused stage, to keep the copy count fixed)
  int c0 = next_block();  // never -1: every query selects its own block
  int c1 = next_block();
  int c2 = next_block();
  copy_block(c0, 0);
  copy_block(c1 >= 0 ? c1 : c0, 1);
  copy_block(c2 >= 0 ? c2 : c0, 2);

  const int tr_e = (lane & 15) >> 2, tr_q = lane & 3;
  for (int i = 0;; ++i) {
    const int st = i & (kStages - 1);
    const int c = c0;
    wait_vm<2 * kCopies>();  // this wave's copies of block i landed (blocks i+1, i+2 may be in flight)
    lds_barrier();           // ... and every other wave's; block i-1's stage is free
    if (c * kBlock + kBlock > T) {  // the sequence's last, partial block: zero V rows past the end
      uint8_t *vt = ring[st] + kTile;
      for (int b = tid * 16 + (T - c * kBlock) * kRow; b < kTile; b += kThreads * 16)
        *reinterpret_cast<u32x4 *>(vt + b) = u32x4{0, 0, 0, 0};
      lds_barrier();
    }
    // block i+3 into the stage block i-1 used
    const int c3 = next_block();
    copy_block(c3 >= 0 ? c3 : c, (i + 3) & (kStages - 1));

    // ---- attend block c
    const bool s_l = nxt_c == c;
    const float g_l = s_l ? nxt_g : 0.f;
    if (s_l) {
      ++ptr;
      nxt_c = ptr < cq ? sel_l[qi][ptr] : INT_MAX;
      if (kGated) nxt_g = gate_l[kGated ? qi : 0][min(ptr, kMaxSel - 1)];
    }
    if (__builtin_amdgcn_ballot_w64(s_l) != 0) {
      const uint8_t *kt = ring[st];
      const uint8_t *vt = ring[st] + kTile;
      f32x4 sacc[kCt][4];  // [head][key tile]
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 ka[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          ka[ks] = *reinterpret_cast<const u32x4 *>(kt + (16 * t + j) * kRow + 16 * ((4 * ks + g) ^ j));
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
          sacc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            sacc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(ka[ks]), qB[ct][ks], sacc[ct][t], 0, 0, 0);
        }
      }
      const bool causal = c == qb;
      u32x4 pB[kCt][2];
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        float z[4][4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tau = 16 * t + 4 * g + r;
            const bool keep = s_l && (!causal || tau <= qi);
            z[t][r] = keep ? sacc[ct][t][r] * p.scale_log2 : -__builtin_inff();
            mx = fmaxf(mx, z[t][r]);
          }
        mx = rows_max(mx);
        const float m_new = fmaxf(m[ct], mx);
        const bool live = m_new != -__builtin_inff();
        const float alpha = live ? fast_exp2(m[ct] - m_new) : 1.0f;
        float psum = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 2 * s2 + (e >> 2), r = e & 3;
            const float pe = live ? fast_exp2(z[t][r] - m_new) : 0.f;
            psum += pe;
            pv[e] = kGated ? pe * g_l : pe;
          }
          pB[ct][s2] = u32x4{pack_rne(pv[0], pv[1]), pack_rne(pv[2], pv[3]), pack_rne(pv[4], pv[5]),
                             pack_rne(pv[6], pv[7])};
        }
        ls[ct] = ls[ct] * alpha + psum;
        m[ct] = m_new;
        // the running max rarely moves once a query has seen a few blocks (and
        // never for a query that did not select this one): rescale only then
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[ct][dt] *= alpha;
        }
      }
      // tr-read lane roles: within the 16-lane group g, lane 4e+q4 addresses
      // row 4g+e (+16 for the upper half of the k-step, +32 per k-step), bytes
      // 8q4 of the 32-byte pair dt, stored at pair dt ^ e (row % 4 == e)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint8_t *vrd = vt + (32 * s2 + 4 * g + tr_e) * kRow + 32 * (dt ^ tr_e) + 8 * tr_q;
          i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)vrd);
          i16x4 a1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(vrd + 16 * kRow));
          u32x2 lo2 = __builtin_bit_cast(u32x2, a0), hi2 = __builtin_bit_cast(u32x2, a1);
          const bf16x8 a = as_bf16(u32x4{lo2.x, lo2.y, hi2.x, hi2.y});
#pragma unroll
          for (int ct = 0; ct < kCt; ++ct)
            o[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16(pB[ct][s2]), o[ct][dt], 0, 0, 0);
        }
      }
    }
    if (c1 < 0) break;  // block i was the walk's last
    c0 = c1;
    c1 = c2;
    c2 = c3;
  }
  wait_vm<0>();  // the trailing filler copies land before the workgroup ends

  // ---- normalise and store: lane holds dims 16dt + 4(l/16) .. +3 of its query
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    const float l = rows_sum(ls[ct]);
    if (qvalid && 2 * hp + ct < nh) {
      const float inv = 1.0f / l;
      const int64_t row = (int64_t)tq * p.n_q_heads + kvh * G + h_lo + ct;
      uint16_t *dst = p.out + row * kHeadDim + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[ct][dt] * inv;
        *reinterpret_cast<u32x2 *>(dst + 16 * dt) = u32x2{pack_rne(v[0], v[1]), pack_rne(v[2], v[3])};
      }
      // log-sum-exp of the (ungated) logits, natural log: (m + log2 l) ln 2
      if (p.lse && g == 0) p.lse[row] = (m[ct] + log2f(l)) * 0.6931471805599453f;
    }
  }
}

// ---------------------------------------------------------------- backward: dL/dg of every selected block
// The gradient of the gated output with respect to each selected block's
// continuous gate, for the backward of the training-time forward:
//   dg_i = sum_{h in group} sum_{j in block c_i, j <= t} P_hj <dO_h, v_j>,
// with P_hj = 2^(z_hj - lse2_h) from the forward's log-sum-exp (the plain
// softmax over the query's selected tokens; the gates scale the blocks'
// shares afterwards).  The walk is the forward's: one workgroup per
// (64-query block, KV head, group of up to 4 query heads), the union of the
// queries' selections in ascending order, each block's K and V rows copied
// once into the LDS ring.  Per block, wave w (queries 16(w%4) .., heads
// 2(w/4), 2(w/4)+1) forms S^T = K Q^T and D^T = V dO^T on MFMA (V is read
// like K, as the A operand, so it is stored with K's swizzle), then per query
// the sum over the block's keys and its two heads of P * D, added to the
// query's slot in LDS.  Exactly two waves (the two head pairs) add to each
// slot, and a sum of two terms onto zero does not depend on their order, so
// the result is deterministic.  The groups of 4 heads write separate partial
// sums, added in order by the chain kernel.
__global__ __launch_bounds__(kThreads, 1) void prefill_grad_kernel(PrefillBackwardParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][kStage];
  __shared__ uint32_t bm[SAS_MAX_BLOCKS_DEV / 32];
  __shared__ int16_t sel_l[kBlock][kMaxSel];
  __shared__ float dg_l[kBlock][kMaxSel];
  __shared__ int cnt_l[kBlock];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int G = p.group;
  const int hg = blockIdx.x % p.head_groups;
  const int rest = blockIdx.x / p.head_groups;
  const int kvh = rest % p.n_kv_heads;
  const int qb = p.n_qblocks - 1 - rest / p.n_kv_heads;
  const int nh = min(4, G - 4 * hg);
  const int T = p.seq_len;
  const int t0 = qb * kBlock;
  const int nq = min(kBlock, T - t0);
  const int qw = wave & 3, hp = wave >> 2;
  const int qi = 16 * qw + j;
  const int h_lo = 4 * hg + 2 * hp;
  const bool qvalid = qi < nq;
  const int tq = t0 + qi;

  // ---- the queries' selections into LDS and their union; slot sums zeroed
  const int nwords = (qb + 32) >> 5;
  for (int i = tid; i < nwords; i += kThreads) bm[i] = 0;
  for (int e = tid; e < kBlock * kMaxSel; e += kThreads) (&dg_l[0][0])[e] = 0.f;
  if (tid < kBlock) cnt_l[tid] = tid < nq ? p.cnt[(int64_t)(t0 + tid) * p.n_kv_heads + kvh] : 0;
  __syncthreads();
  for (int e = tid; e < nq * p.max_sel; e += kThreads) {
    const int q = e / p.max_sel, slot = e - q * p.max_sel;
    if (slot < cnt_l[q]) {
      int c = p.sel[((int64_t)(t0 + q) * p.n_kv_heads + kvh) * p.max_sel + slot];
      c = (unsigned)c <= (unsigned)qb ? c : qb;  // out-of-range entries are not trusted
      sel_l[q][slot] = (int16_t)c;
      atomicOr(&bm[c >> 5], 1u << (c & 31));
    }
  }

  // B operands (q and dO of this lane's query, the wave's two heads) and the
  // forward's log-sum-exp in log2 units
  bf16x8 qB[kCt][4], dB[kCt][4];
  float lse2[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    const bool ok = qvalid && 2 * hp + ct < nh;
    const int64_t row = (int64_t)(ok ? tq : 0) * p.n_q_heads + kvh * G + (ok ? h_lo + ct : 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qB[ct][ks] = as_bf16(ok ? ld16(p.q + row * kHeadDim + 8 * g + 32 * ks) : u32x4{0, 0, 0, 0});
      dB[ct][ks] = as_bf16(ok ? ld16(p.d_out + row * kHeadDim + 8 * g + 32 * ks) : u32x4{0, 0, 0, 0});
    }
    lse2[ct] = ok ? p.lse[row] * kLog2e : 0.f;
  }
  wait_vm<0>();  // every compiler-visible load done before the copies start
  __syncthreads();

  const int cq = cnt_l[qi];
  int ptr = 0;
  int nxt_c = cq > 0 ? sel_l[qi][0] : INT_MAX;

  // ---- block copies into the ring, K and V both with K's swizzle (16-byte
  // slots by row % 16): wave w writes 1 KiB pieces 2w, 2w+1 of each tile
  const char *kbase = reinterpret_cast<const char *>(p.k_pool) + (int64_t)kvh * p.head_stride * 2;
  const char *vbase = reinterpret_cast<const char *>(p.v_pool) + (int64_t)kvh * p.head_stride * 2;
  const int64_t tok_bytes = p.tok_stride * 2, page_bytes = p.page_stride * 2;
  int64_t src[kCopies / 2];
#pragma unroll
  for (int k = 0; k < kCopies / 2; ++k) {
    const int row = 4 * (2 * wave + k) + (lane >> 4), sl = lane & 15;
    src[k] = row * tok_bytes + 16 * (sl ^ (row & 15));
  }
  const __attribute__((address_space(4))) int32_t *btc =
      (const __attribute__((address_space(4))) int32_t *)p.block_table;
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)&ring[0][0];
  auto copy_block = [&](int c, int st) {
    const int64_t off = (int64_t)btc[c] * page_bytes;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring0 + st * kStage + 2048 * wave);
#pragma unroll
    for (int k = 0; k < kCopies / 2; ++k) copy16(kbase + off + src[k], dst + 1024 * k);
#pragma unroll
    for (int k = 0; k < kCopies / 2; ++k) copy16(vbase + off + src[k], dst + kTile + 1024 * k);
  };
  int wi = 0;
  uint32_t bits = __builtin_amdgcn_readfirstlane(bm[0]);
  auto next_block = [&]() -> int {
    while (bits == 0) {
      if (++wi >= nwords) return -1;
      bits = __builtin_amdgcn_readfirstlane(bm[wi]);
    }
    const int c = (wi << 5) + __builtin_ctz(bits);
    bits &= bits - 1;
    return c;
  };
  int c0 = next_block();  // never -1: every query selects its own block
  int c1 = next_block();
  int c2 = next_block();
  copy_block(c0, 0);
  copy_block(c1 >= 0 ? c1 : c0, 1);
  copy_block(c2 >= 0 ? c2 : c0, 2);

  for (int i = 0;; ++i) {
    const int st = i & (kStages - 1);
    const int c = c0;
    wait_vm<2 * kCopies>();  // this wave's copies of block i landed
    lds_barrier();           // ... and every other wave's; block i-1's stage is free
    const int c3 = next_block();
    copy_block(c3 >= 0 ? c3 : c, (i + 3) & (kStages - 1));

    const bool s_l = nxt_c == c;
    const int slot = ptr;
    if (s_l) {
      ++ptr;
      nxt_c = ptr < cq ? sel_l[qi][ptr] : INT_MAX;
    }
    if (__builtin_amdgcn_ballot_w64(s_l) != 0) {
      const uint8_t *kt = ring[st];
      const uint8_t *vt = ring[st] + kTile;
      f32x4 sacc[kCt][4], dacc[kCt][4];  // [head][key tile]
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 ka[4], va[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int off = (16 * t + j) * kRow + 16 * ((4 * ks + g) ^ j);
          ka[ks] = *reinterpret_cast<const u32x4 *>(kt + off);
          va[ks] = *reinterpret_cast<const u32x4 *>(vt + off);
        }
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
          sacc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          dacc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            sacc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(ka[ks]), qB[ct][ks], sacc[ct][t], 0, 0, 0);
            dacc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(va[ks]), dB[ct][ks], dacc[ct][t], 0, 0, 0);
          }
        }
      }
      // keys the query may not see (another query's block, later keys of its
      // own block, rows past the sequence end) are dropped by the select, so
      // that whatever such rows hold never enters the sum
      const bool causal = c == qb;
      float acc = 0.f;
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tau = 16 * t + 4 * g + r;
            const bool keep = s_l && (!causal || tau <= qi);
            const float pe = fast_exp2(sacc[ct][t][r] * p.scale_log2 - lse2[ct]);
            acc += keep ? pe * dacc[ct][t][r] : 0.f;
          }
      acc = rows_sum(acc);
      if (s_l && g == 0) atomicAdd(&dg_l[qi][slot], acc);
    }
    if (c1 < 0) break;  // block i was the walk's last
    c0 = c1;
    c1 = c2;
    c2 = c3;
  }
  wait_vm<0>();  // the trailing filler copies land before the workgroup ends
  __syncthreads();
  float *dst = p.ws_dgp + (((int64_t)hg * T + t0) * p.n_kv_heads + kvh) * p.max_sel;
  for (int e = tid; e < nq * p.max_sel; e += kThreads) {
    const int q = e / p.max_sel, slot = e - q * p.max_sel;
    dst[(int64_t)q * p.n_kv_heads * p.max_sel + slot] = dg_l[q][slot];
  }
}

hipError_t launch_prefill_attend(const PrefillParams &p, hipStream_t st) {
  const dim3 grid((unsigned)(p.n_qblocks * p.n_kv_heads * p.head_groups));
  if (p.gates)
    hipLaunchKernelGGL((prefill_attend_kernel<true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((prefill_attend_kernel<false>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_prefill_grad(const PrefillBackwardParams &p, hipStream_t st) {
  const dim3 grid((unsigned)(p.n_qblocks * p.n_kv_heads * p.head_groups));
  hipLaunchKernelGGL(prefill_grad_kernel, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
