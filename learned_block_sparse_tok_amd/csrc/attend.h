// Per-block attention of the block-sparse flash-decode (device code shared
// by the decode kernel and the fused decode step).  The layouts and the
// schedule are described where the decode kernel is defined.
#pragma once
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {

constexpr int kWaves = 8;  // waves per workgroup, one workgroup per CU

#ifndef SAS_V_NT
#define SAS_V_NT 1
#endif
#ifndef SAS_K_NT
#define SAS_K_NT 1
#endif

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
template <bool kNT>
__device__ __forceinline__ u32x4 ld16_kv(const char *p) {
  if (kNT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);  // RNE
  return __builtin_bit_cast(uint32_t, b);
}

// V tile in LDS: 64 rows of 256 bytes at a 288-byte pitch.  The 32-byte pad
// moves consecutive rows 8 banks apart, so both the row writes (16 lanes x
// 16 B per row) and the transposing reads (16 rows x 32 B per instruction)
// are conflict-free, and every lane address is one base plus an immediate.
constexpr int kVPitch = 288;
constexpr int kVTileBytes = kBlock * kVPitch;  // 18 KiB

struct BlockRegs {
  u32x4 k[4][4];  // [token tile][k-step]: token 16t + l%16, dims 32ks + 8(l/16) .. +7
  u32x4 v[16];    // row 4r + l/16, dims 8(l%16) .. +7
};

// Byte offsets inside one (page, KV head) block: a per-lane part fixed for
// the kernel plus uniform steps (kept in scalar registers).
struct LaneOffsets {
  uint32_t k;       // token l%16, dims 8(l/16)
  uint32_t v;       // row l/16, dims 8(l%16)
  int64_t k_tile;   // 16 rows (token tile t adds t * k_tile)
  int64_t v_rows;   // 4 rows (V load r adds r * v_rows)
};

struct WaveState {
  f32x4 o[8];   // O^T tiles: lane holds dims 16dt + 4(l/16) + r of head l%16
  float m;      // running max (log2 domain) of head l%16
  float lsum;   // this lane's share of head l%16's softmax denominator
};

struct BlockSrc {
  const char *k, *v;  // this KV head's 64 x 128 K and V rows
  int nvalid;         // rows before the cache end
  float gate;
};

// One selected block, with the next block's loads issued as soon as the
// registers they land in are free: V rows go to the LDS tile, V(next) is
// issued; S^T = K Q^T, K(next) is issued; online softmax; O^T += V^T P^T.
// kMode: 0 plain Top-K attention; 1 each selected block's share of the
// output scaled by its gate; 2 the gate as a factor on exp(logit) before
// normalising (a log-gate bias on the block's logits)
template <int kMode, bool kNext>
__device__ __forceinline__ void attend_block(WaveState &w, BlockRegs &b, const BlockSrc &cur, const BlockSrc &nxt,
                                             const bf16x8 (&qB)[4], const LaneOffsets &lo, uint8_t *vt,
                                             float scale_log2, int g, int j, int tr_e, int tr_q) {
  // V -> LDS (row 4r + l/16, bytes 16(l%16)); rows past the cache end are zeroed
  uint8_t *vw = vt + g * kVPitch + 16 * j;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    *reinterpret_cast<u32x4 *>(vw + 4 * r * kVPitch) = 4 * r + g < cur.nvalid ? b.v[r] : u32x4{0, 0, 0, 0};
  if (kNext) {
#pragma unroll
    for (int r = 0; r < 16; ++r) b.v[r] = ld16_kv<SAS_V_NT>(nxt.v + r * lo.v_rows + lo.v);
  }
  f32x4 sacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(b.k[t][ks]), qB[ks], sacc[t], 0, 0, 0);
  }
  if (kNext) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) b.k[t][ks] = ld16_kv<SAS_K_NT>(nxt.k + t * lo.k_tile + 64 * ks + lo.k);
  }
  float z[4][4];
  float mx = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tau = 16 * t + 4 * g + r;
      z[t][r] = tau < cur.nvalid ? sacc[t][r] * scale_log2 : -__builtin_inff();
      mx = fmaxf(mx, z[t][r]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_new = fmaxf(w.m, mx);
  const bool live = m_new != -__builtin_inff();
  const float alpha = live ? exp2f(w.m - m_new) : 1.0f;
  float psum = 0.f;
  u32x4 pB[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = 2 * s2 + (e >> 2), r = e & 3;
      const float pe = live ? exp2f(z[t][r] - m_new) : 0.f;
      pv[e] = kMode ? pe * cur.gate : pe;
      psum += kMode == 2 ? pv[e] : pe;
    }
    pB[s2] = u32x4{pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]), pack2(pv[6], pv[7])};
  }
  w.lsum = w.lsum * alpha + psum;
  w.m = m_new;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) w.o[dt] *= alpha;

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // tr-read lane roles: within the 16-lane group g, lane 4e+q4 addresses row
  // 4g+e (+16 for the upper half of the k-step, +32 per k-step), columns
  // 16dt + 4q4 .. +3
  const uint8_t *vr = vt + (4 * g + tr_e) * kVPitch + 8 * tr_q;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(vr + 32 * s2 * kVPitch + 32 * dt));
      i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(vr + (32 * s2 + 16) * kVPitch + 32 * dt));
      u32x2 lo2 = __builtin_bit_cast(u32x2, a0), hi2 = __builtin_bit_cast(u32x2, a1);
      u32x4 a = u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
      w.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pB[s2]), w.o[dt], 0, 0, 0);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A selected block as the lookups give it: its page, its logical index and
// its gate (1 in plain mode).
struct BlockRef {
  int32_t page, blk;
  float gate;
};

// This lane's byte offsets inside one (page, KV head) block.
__device__ __forceinline__ LaneOffsets lane_offsets(const DecodeParams &p) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  LaneOffsets lo;
  lo.k = (uint32_t)((j * p.tok_stride + 8 * g) * 2);
  lo.v = (uint32_t)((g * p.tok_stride + 8 * j) * 2);
  lo.k_tile = 16 * p.tok_stride * 2;
  lo.v_rows = 4 * p.tok_stride * 2;
  return lo;
}

// K and V rows of a selected block of KV head kvh.
__device__ __forceinline__ BlockSrc block_rows(const DecodeParams &p, int kvh, const BlockRef &r, int32_t L) {
  const int64_t off = (int64_t)r.page * p.page_stride * 2 + (int64_t)kvh * p.head_stride * 2;
  return BlockSrc{reinterpret_cast<const char *>(p.k_pool) + off, reinterpret_cast<const char *>(p.v_pool) + off,
                  min(kBlock, L - r.blk * kBlock), r.gate};
}

// Issues a block's 32 loads into b, V rows first (the order they are consumed).
__device__ __forceinline__ void issue_block(BlockRegs &b, const BlockSrc &cur, const LaneOffsets &lo) {
#pragma unroll
  for (int r = 0; r < 16; ++r) b.v[r] = ld16_kv<SAS_V_NT>(cur.v + r * lo.v_rows + lo.v);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) b.k[t][ks] = ld16_kv<SAS_K_NT>(cur.k + t * lo.k_tile + 64 * ks + lo.k);
}

// B operand of S^T = K Q^T for (sequence s, KV head kvh): lane l holds
// q[head l%16][32ks + 8(l/16) .. +7] (heads >= G zero).
__device__ __forceinline__ void load_query_operand(const DecodeParams &p, int s, int kvh, bf16x8 (&qB)[4]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const uint16_t *qrow = p.q + ((int64_t)s * p.n_q_heads + kvh * p.group + j) * kHeadDim + 8 * g;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qB[ks] = as_bf16x8(j < p.group ? ld16(qrow + 32 * ks) : u32x4{0, 0, 0, 0});
}

__device__ __forceinline__ void wave_state_init(WaveState &ws) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) ws.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  ws.m = -__builtin_inff();
  ws.lsum = 0.f;
}

// One wave attends the selected blocks item(i0), item(i0 + 1), ...,
// item(i1 - 1) in that order (item(i) gives a BlockRef; it is called for i0
// even when i0 >= i1, so it must stay in bounds), accumulating into ws; vt
// is the wave's V tile.  When first_issued, item(i0)'s loads are already in
// b (issue_block).
template <int kMode, class Item>
__device__ __forceinline__ void attend_blocks(const DecodeParams &p, uint8_t *vt, int kvh, int32_t L, int i0, int i1,
                                              Item item, BlockRegs &b, bool first_issued, const bf16x8 (&qB)[4],
                                              WaveState &ws) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const BlockRef r0 = item(i0);
  const LaneOffsets lo = lane_offsets(p);
  const char *kpool = reinterpret_cast<const char *>(p.k_pool) + (int64_t)kvh * p.head_stride * 2;
  const char *vpool = reinterpret_cast<const char *>(p.v_pool) + (int64_t)kvh * p.head_stride * 2;
  const int64_t page_bytes = p.page_stride * 2;
  const int tr_e = (lane & 15) >> 2, tr_q = lane & 3;
  auto rows = [&](const BlockRef &r) {
    const int64_t off = (int64_t)r.page * page_bytes;
    return BlockSrc{kpool + off, vpool + off, min(kBlock, L - r.blk * kBlock), r.gate};
  };
  if (i0 < i1) {
    // one register set: block i+1's loads are issued into it while block i is
    // consumed; the steady-state loop issues them unconditionally so that the
    // load counters wait for exactly the block being consumed
    BlockSrc cur = rows(r0);
    if (!first_issued) issue_block(b, cur, lo);
    for (int i = i0; i + 1 < i1; ++i) {
      const BlockSrc nxt = rows(item(i + 1));
      attend_block<kMode, true>(ws, b, cur, nxt, qB, lo, vt, p.scale_log2, g, j, tr_e, tr_q);
      cur = nxt;
    }
    attend_block<kMode, false>(ws, b, cur, cur, qB, lo, vt, p.scale_log2, g, j, tr_e, tr_q);
  }
}

// The waves of one workgroup merge their (max, sum, output) in LDS (vlds:
// the waves' V tiles), in wave order, and the workgroup writes the bf16
// output of (sequence s, KV head kvh) = unit (one workgroup per unit) or its
// partial (max, sum, unnormalised output).
__device__ __forceinline__ void merge_waves(const DecodeParams &p, uint8_t (*vlds)[kVTileBytes], int s, int kvh,
                                            int unit, int wg, int wave, const WaveState &ws) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int G = p.group;
  float lsum = ws.lsum;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  {
    float *wo = reinterpret_cast<float *>(vlds[wave]);  // [16][128] o, then m[16], l[16]
    if (j < G) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4 *>(wo + j * kHeadDim + 16 * dt + 4 * g) = ws.o[dt];
      if (g == 0) {
        wo[16 * kHeadDim + j] = ws.m;
        wo[16 * kHeadDim + 16 + j] = lsum;
      }
    }
  }
  __syncthreads();
  const int nwg = p.wg_per_unit;
  const int64_t pbase = ((int64_t)unit * nwg + wg) * G;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kWaves * 64) {
    const int jj = idx >> 7, d = idx & (kHeadDim - 1);
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, reinterpret_cast<const float *>(vlds[w])[16 * kHeadDim + jj]);
    float num = 0.f, den = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float *wo = reinterpret_cast<const float *>(vlds[w]);
        const float f = exp2f(wo[16 * kHeadDim + jj] - M);
        den = fmaf(f, wo[16 * kHeadDim + 16 + jj], den);
        num = fmaf(f, wo[jj * kHeadDim + d], num);
      }
    }
    if (nwg == 1) {
      p.out[((int64_t)s * p.n_q_heads + kvh * G + jj) * kHeadDim + d] = (uint16_t)f32_to_bf16(num / den);
    } else {
      p.part_o[(pbase + jj) * kHeadDim + d] = num;
      if (d == 0) {
        p.part_ml[(pbase + jj) * 2] = M;
        p.part_ml[(pbase + jj) * 2 + 1] = den;
      }
    }
  }
}

// One workgroup's share of a (sequence s, KV head kvh) = unit: wave `wave`
// attends the selected blocks [i0, min(count, i0 + blocks_per_wave)), the
// local block (the last, count - 1) first when the share ends with it; then
// the waves merge (merge_waves).  source(i) gives selected block i; it is
// called for i0 before count is tested, so it must stay in bounds for any i0.
template <int kMode, class Source>
__device__ __forceinline__ void attend_unit(const DecodeParams &p, uint8_t (*vlds)[kVTileBytes], int s, int kvh,
                                            int unit, int wg, int wave, int i0, int count, int32_t L,
                                            Source source, BlockRegs &b, bool first_issued) {
  bf16x8 qB[4];
  load_query_operand(p, s, kvh, qB);
  const int i1 = min(count, i0 + p.blocks_per_wave);
  const bool local_first = i1 == count;
  auto item = [&](int i) { return source(local_first ? (i == i0 ? count - 1 : i - 1) : i); };
  WaveState ws;
  wave_state_init(ws);
  attend_blocks<kMode>(p, vlds[wave], kvh, L, i0, i1, item, b, first_issued, qB, ws);
  merge_waves(p, vlds, s, kvh, unit, wg, wave, ws);
}

}  // namespace sas
