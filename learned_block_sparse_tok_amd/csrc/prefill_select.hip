// Selection of the training-time forward, batched per half of a 64-token block.
//
// Every position t of one sequence selects as a decode step of length t+1
// would: gate query at position t (Qproj, RMSNorm, RoPE, mean over the KV
// head's query heads), scores of the complete blocks before t's own block,
// Top-K, its own block last ("Tencent released Simple-Attention-
// Sparsification ...", aigc.news: Top-K of 31 historical blocks, gate hidden
// size 128, Qproj, Q/K normalization, gate RoPE; "Tencent Hunyuan
// open-sources SAS ...": per-query block selection).  The positions of a
// 64-token block share their candidate set (blocks 0 .. b-1 for block b), so
// one 512-thread workgroup (8 waves of at most 128 VGPRs) per (32 positions
// of one block, KV head) does:
//   1. the RoPE table of its 32 positions (angles reduced in fp64);
//   2. per query head and 16-position tile (one work item per wave),
//      U^T = W_q[h] . Q^T on v_mfma_f32_16x16x32_bf16 (bf16 products are
//      exact, sums fp32), RMSNorm, * w_qnorm and RoPE on the accumulator
//      lanes, added into the mean gate query in LDS in head order
//      (deterministic);
//   3. the scores S^T = GK . ghat^T / sqrt(128) on MFMA with ghat split into
//      bf16 high and low parts (about 16 significant bits: the scores keep
//      fp32-level accuracy), gate keys gathered through the block table;
//   4. one exact Top-K per position (wave_select), eight waves in parallel.
// Its LDS (the score keys of 32 positions, 66 KiB) leaves room for two
// workgroups per CU, so one workgroup's latency-bound phases (projection,
// gathers, radix selects) overlap the other's.
// It replaces per-position gate workgroups, each of which re-read W_q and
// the candidates' gate keys.
#include "sas_device.h"
#include "sas_kernels.h"
#include "select.h"

namespace sas {
namespace {

constexpr int kPos = 32;                 // positions per workgroup (half a 64-token block)
constexpr int kTiles = kPos / 16;        // 16-position MFMA tiles
constexpr int kWavesSel = 8;             // waves per workgroup (128 VGPRs each: two workgroups per CU)
constexpr int kThreadsSel = 64 * kWavesSel;
constexpr int kRowWords = kMaxCandBatched + 4;  // LDS row of score keys: 16-byte aligned, staggered banks
constexpr int kGhatPitch = kGateDim + 4;  // LDS row of the mean gate query (floats)

__device__ __forceinline__ bf16x8 b8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace

__global__ __launch_bounds__(kThreadsSel, 2) void prefill_select_kernel(PrefillSelectParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t big[kPos * kRowWords];  // phases 1-2 tables, then score keys
  __shared__ __attribute__((aligned(16))) uint32_t hist[kWavesSel][256];
  __shared__ int32_t bt_l[kMaxCandBatched];
  __shared__ float wqn_l[kGateDim];
  float *cosv = reinterpret_cast<float *>(big);  // [kPos positions][64 frequencies]
  float *sinv = cosv + kPos * 64;
  float *ghat = sinv + kPos * 64;                 // [kPos positions][kGhatPitch]
  uint32_t *keys = big;                           // [kPos positions][kRowWords]

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63, g = lane >> 4, j = lane & 15;
  const int kvh = blockIdx.x % p.n_kv_heads;
  // heaviest (latest) positions first
  const int qh = 2 * p.n_qblocks - 1 - (int)(blockIdx.x / p.n_kv_heads);  // half block
  const int t0 = qh * kPos;
  const int nq = max(0, min(kPos, p.seq_len - t0));
  const int nc = qh >> 1;  // candidates of every position here: blocks 0 .. b-1 of its block b
  const int G = p.group;

  // ---- 1. RoPE table, block-table row, zeroed mean gate query
  for (int e = t; e < kPos * 64; e += kThreadsSel) {
    float c, s;
    rope_cos_sin((double)(t0 + (e >> 6)), p.inv_freq[e & 63], c, s);
    cosv[e] = c;
    sinv[e] = s;
  }
  for (int e = t; e < kPos * kGhatPitch; e += kThreadsSel) ghat[e] = 0.f;
  for (int c = t; c < nc; c += kThreadsSel) bt_l[c] = p.block_table[c];
  if (t < kGateDim) wqn_l[t] = p.w_qnorm[t];
  __syncthreads();

  // ---- 2. gate queries.  Work item i = (head i / kTiles, position tile
  // i % kTiles), one per wave, in rounds of kWavesSel items (whole heads:
  // kHpr per round)
  const float inv_g = 1.0f / (float)G;
  constexpr int kHpr = kWavesSel / kTiles;  // heads per round
  for (int i0 = 0; i0 < kTiles * G; i0 += kWavesSel) {
    const int h = (i0 + wave) / kTiles, nt = wave % kTiles;
    const bool active = h < G;
    const int head = kvh * G + (active ? h : 0);
    const int pos = 16 * nt + j;
    // B operand: lane l holds q[position 16nt + l%16][head][32ks + 8(l/16) .. +7]
    bf16x8 qB[4];
    {
      const bool ok = active && pos < nq;
      const uint16_t *qrow = p.q + ((int64_t)(t0 + (ok ? pos : 0)) * p.n_q_heads + head) * kHeadDim + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qB[ks] = b8(ok ? ld16(qrow + 32 * ks) : u32x4{0, 0, 0, 0});
    }
    f32x4 acc[8];  // [row tile]: lane holds rows 16mt + 4g + r of position 16nt + l%16
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
      const uint16_t *wrow = p.w_q + (int64_t)head * kGateDim * kHeadDim + 8 * g;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        u32x4 a[4];  // A operand: lane l holds W_q[h][row 16mt + l%16][32ks + 8(l/16) .. +7]
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a[ks] = ld16(wrow + (16 * mt + j) * kHeadDim + 32 * ks);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b8(a[ks]), qB[ks], acc[mt], 0, 0, 0);
      }
      // RMSNorm (the 128 rows of a position sit in the 4 lanes l%16 == const),
      // * w_qnorm, rotate-half RoPE: row i < 64 pairs with row i + 64 (tile mt + 4)
      float ss = 0.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss = fmaf(acc[mt][r], acc[mt][r], ss);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      const float inv = 1.0f / sqrtf(ss * (1.0f / kGateDim) + 1e-6f);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * mt + 4 * g + r;
          const float na = acc[mt][r] * inv * wqn_l[i];
          const float nb = acc[mt + 4][r] * inv * wqn_l[i + 64];
          const float c = cosv[pos * 64 + i], s = sinv[pos * 64 + i];
          acc[mt][r] = na * c - nb * s;
          acc[mt + 4][r] = nb * c + na * s;
        }
    }
    // add into the mean gate query in head order (the items of one head
    // cover disjoint positions and add at the same time)
    for (int hh = 0; hh < kHpr; ++hh) {
      if (wave / kTiles == hh && active) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) ghat[pos * kGhatPitch + 16 * mt + 4 * g + r] += acc[mt][r] * inv_g;
      }
      __syncthreads();
    }
  }

  // ---- 3. scores.  Wave w takes both position tiles of candidate tiles w,
  // w + kWavesSel, ...  B operands: ghat of position 16nt + l%16, dims
  // 32ks + 8(l/16) .. +7, as bf16 high + low
  u32x4 bh[kTiles][4], bl[kTiles][4];
#pragma unroll
  for (int n2 = 0; n2 < kTiles; ++n2)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int nt = n2;
      const float *gp = ghat + (16 * nt + j) * kGhatPitch + 32 * ks + 8 * g;
      float hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hb = f32_to_bf16(gp[e]);
        hi[e] = __uint_as_float(hb << 16);
        lo[e] = gp[e] - hi[e];
      }
      bh[n2][ks] = u32x4{pack_bf16_rne(hi[0], hi[1]), pack_bf16_rne(hi[2], hi[3]), pack_bf16_rne(hi[4], hi[5]),
                         pack_bf16_rne(hi[6], hi[7])};
      bl[n2][ks] = u32x4{pack_bf16_rne(lo[0], lo[1]), pack_bf16_rne(lo[2], lo[3]), pack_bf16_rne(lo[4], lo[5]),
                         pack_bf16_rne(lo[6], lo[7])};
    }
  __syncthreads();  // the tables are consumed: the LDS becomes the score-key rows
  const float inv_sqrt_dg = 0.08838834764831845f;  // 1/sqrt(128)
  const uint16_t *gkh = p.gate_keys + (int64_t)kvh * kGateDim + 8 * g;
  const int64_t page_stride = (int64_t)p.n_kv_heads * kGateDim;
  for (int ct = wave; 16 * ct < nc; ct += kWavesSel) {
    const int c_lane = min(16 * ct + j, nc - 1);  // A operand row: candidate 16ct + l%16
    const uint16_t *krow = gkh + (int64_t)bt_l[c_lane] * page_stride;
    u32x4 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = ld16(krow + 32 * ks);
#pragma unroll
    for (int n2 = 0; n2 < kTiles; ++n2) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b8(a[ks]), b8(bh[n2][ks]), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b8(a[ks]), b8(bl[n2][ks]), sacc, 0, 0, 0);
      }
      // lane: position 16nt + l%16, candidates 16ct + 4(l/16) + r
      const int pos = 16 * n2 + j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * ct + 4 * g + r;
        if (c < nc) {
          const float sc = sacc[r] * inv_sqrt_dg;
          keys[pos * kRowWords + c] = score_key(sc);
          if (p.scores && pos < nq) p.scores[((int64_t)(t0 + pos) * p.n_kv_heads + kvh) * p.max_blocks + c] = sc;
        }
      }
    }
  }
  if (p.scores && p.max_blocks > nc)
    for (int e = t; e < nq * (p.max_blocks - nc); e += kThreadsSel) {
      const int pos = e / (p.max_blocks - nc), c = nc + e % (p.max_blocks - nc);
      p.scores[((int64_t)(t0 + pos) * p.n_kv_heads + kvh) * p.max_blocks + c] = -__builtin_inff();
    }
  lds_barrier();

  // ---- 4. exact Top-K per position (wave w: positions w, w + kWavesSel, ...)
  const int k_eff = min(p.n_sel - 1, nc);
  for (int pos = wave; pos < nq; pos += kWavesSel) {
    const int64_t u = (int64_t)(t0 + pos) * p.n_kv_heads + kvh;
    wave_select(keys + pos * kRowWords, nc, k_eff, p.n_sel, hist[wave], p.sel + u * p.n_sel,
                p.gates ? p.gates + u * p.n_sel : nullptr, p.cnt + u);
  }
}

hipError_t launch_prefill_select(const PrefillSelectParams &p, hipStream_t st) {
  hipLaunchKernelGGL(prefill_select_kernel, dim3((unsigned)(2 * p.n_qblocks * p.n_kv_heads)), dim3(kThreadsSel), 0, st,
                     p);
  return hipGetLastError();
}

}  // namespace sas
