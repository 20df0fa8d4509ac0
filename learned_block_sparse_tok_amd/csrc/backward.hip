// Backward of the continuous gates of a gated decode step, down to the gate
// parameters.
//
// SAS puts continuous gates on the selected blocks so that the language-model
// loss can train the ranking end to end ("Tencent released Simple-Attention-
// Sparsification ...", aigc.news; "Tencent Hunyuan open-sources SAS ...": a
// differentiable path from the LM loss to the selector).  With each selected
// block's share of the output scaled by its gate g = sigmoid(score), the
// Top-K choice passing no gradient, the local block's gate fixed at 1 and the
// bf16 gate keys passing the gradient straight through:
//   dg_i   = sum_{h in group} sum_{j in block c_i} P_hj <dO_h, v_j>
//   dS_i   = dg_i g_i (1 - g_i)                          (historical blocks)
//   dghat  = sum_i dS_i gk_{c_i} / sqrt(128),  dgk_{c_i} = dS_i ghat / sqrt(128)
// and on through the group mean, RoPE (a rotation: its transpose rotates
// back), RMSNorm and the bias-free projections to dW_q, dw_qnorm, dW_k and
// dw_knorm, summed over the batch.
//
// Three kernels:
//   gate_grad_kernel  one 8-wave workgroup per (sequence, KV head): pass 1
//     recomputes the softmax max / sum of every head over the selection
//     (S^T = K Q^T on MFMA, as the decode kernel does); pass 2 recomputes S^T
//     and D^T = V dO^T (V as the A operand, dO as the B operand) per block and
//     reduces sum P * D.  K is read twice and V once: 48 KiB per selected
//     block and KV head.
//   gate_chain_kernel one 256-thread workgroup per (sequence, KV head): the
//     chain from dg to the per-sequence factors (du of every query head with
//     its RMSNorm weight term; du, pooled statistics and RMSNorm weight term
//     of every selected historical block), recomputing the gate queries and
//     the selected blocks' pooled keys in fp32.
//   gate_param_reduce_kernel + gate_dwk_sum_kernel  the weight gradients as
//     sums over the batch of outer products of those factors, as 64 x 64
//     output tiles with the factor rows staged in LDS; dW_k's rows are split
//     into ranges whose partial tiles are then added in order (a fixed order
//     throughout: deterministic).
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {
namespace {

constexpr int kWavesG = 8;
constexpr float kInvSqrtDg = 0.08838834764831845f;  // 1/sqrt(128)

__device__ __forceinline__ bf16x8 to_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// the transpose of the rotate-half RoPE rotation at one pair (i, i+64)
__device__ __forceinline__ void rope_back(float da, float db, float c, float s, float &ga, float &gb) {
  ga = da * c + db * s;
  gb = db * c - da * s;
}

}  // namespace

// ---------------------------------------------------------------- dg per selected block
__global__ __launch_bounds__(kWavesG * 64, 1) void gate_grad_kernel(BackwardParams p) {
  __shared__ float ml[kWavesG][2][kMaxGroup];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int unit = blockIdx.x;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int G = p.group;
  const int count = p.cnt[unit];
  const int32_t L = p.seq_lens[s];

  // B operands: lane l holds q / dO of head l%16, dims 32ks + 8(l/16) .. +7
  bf16x8 qB[4], dB[4];
  {
    const int64_t row = ((int64_t)s * p.n_q_heads + kvh * G + (j < G ? j : 0)) * kHeadDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qB[ks] = to_bf16x8(j < G ? ld16(p.q + row + 32 * ks) : u32x4{0, 0, 0, 0});
      dB[ks] = to_bf16x8(j < G ? ld16(p.d_out + row + 32 * ks) : u32x4{0, 0, 0, 0});
    }
  }
  const int32_t *sel = p.sel + (int64_t)unit * p.max_sel;
  const int32_t *bt = p.block_table + (int64_t)s * p.max_blocks;
  const char *kpool = reinterpret_cast<const char *>(p.k_pool) + (int64_t)kvh * p.head_stride * 2;
  const char *vpool = reinterpret_cast<const char *>(p.v_pool) + (int64_t)kvh * p.head_stride * 2;
  // A-operand lane offset: token 16t + l%16, dims 32ks + 8(l/16)
  const int64_t lane_off = ((int64_t)j * p.tok_stride + 8 * g) * 2;
  const int64_t tile = 16 * p.tok_stride * 2;

  auto scores = [&](const char *kb, f32x4 (&sacc)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 k[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) k[ks] = ld16(kb + t * tile + 64 * ks + lane_off);
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(k[ks]), qB[ks], sacc[t], 0, 0, 0);
    }
  };

  // ---- pass 1: max and sum of exp over the whole selection, per head (column)
  float m = -__builtin_inff(), lsum = 0.f;
  for (int i = wave; i < count; i += kWavesG) {
    const int blk = sel[i];
    const int64_t off = (int64_t)bt[blk] * p.page_stride * 2;
    const int nvalid = min(kBlock, L - blk * kBlock);
    f32x4 sacc[4];
    scores(kpool + off, sacc);
    float z[4][4], mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[t][r] = 16 * t + 4 * g + r < nvalid ? sacc[t][r] * p.scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, z[t][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    float add = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) add += exp2f(z[t][r] - m_new);
    lsum = (m == -__builtin_inff() ? 0.f : lsum * exp2f(m - m_new)) + add;
    m = m_new;
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (g == 0) {
    ml[wave][0][j] = m;
    ml[wave][1][j] = lsum;
  }
  __syncthreads();
  float M = -__builtin_inff(), S = 0.f;
#pragma unroll
  for (int w = 0; w < kWavesG; ++w) M = fmaxf(M, ml[w][0][j]);
#pragma unroll
  for (int w = 0; w < kWavesG; ++w)
    if (ml[w][0][j] != -__builtin_inff()) S += ml[w][1][j] * exp2f(ml[w][0][j] - M);
  const float inv_s = j < G && S > 0.f ? 1.0f / S : 0.f;  // columns past the group contribute nothing

  // ---- pass 2: dg_i = sum over the block's tokens and the group's heads of P * <dO, v>
  for (int i = wave; i < count; i += kWavesG) {
    const int blk = sel[i];
    const int64_t off = (int64_t)bt[blk] * p.page_stride * 2;
    const int nvalid = min(kBlock, L - blk * kBlock);
    f32x4 sacc[4], dacc[4];
    scores(kpool + off, sacc);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 v[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) v[ks] = ld16(vpool + off + t * tile + 64 * ks + lane_off);
      dacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) dacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(v[ks]), dB[ks], dacc[t], 0, 0, 0);
    }
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * t + 4 * g + r < nvalid) acc += exp2f(sacc[t][r] * p.scale_log2 - M) * inv_s * dacc[t][r];
    acc = wave_sum(acc);
    if (lane == 0) p.d_gates[(int64_t)unit * p.max_sel + i] = acc;
  }
  for (int i = count + threadIdx.x; i < p.max_sel; i += kWavesG * 64) p.d_gates[(int64_t)unit * p.max_sel + i] = 0.f;
}

// ---------------------------------------------------------------- per-sequence chain
__global__ __launch_bounds__(256) void gate_chain_kernel(BackwardParams p) {
  __shared__ float qv[kMaxGroup][kHeadDim];   // the group's queries (fp32)
  __shared__ float un[kMaxGroup][kGateDim];   // u / r per head
  __shared__ float rr[kMaxGroup];             // r per head
  __shared__ float ghat[kGateDim], dghat[kGateDim];
  __shared__ float pooled[kChainBlocks][3 * kHeadDim];
  __shared__ float uk[kChainBlocks][kGateDim];
  __shared__ float rk[kChainBlocks];
  __shared__ float dwk_acc[4][kGateDim];  // per wave: the key-side norm-weight term summed over its blocks

  const int t = threadIdx.x;
  const int unit = blockIdx.x;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int G = p.group;
  const int count = p.cnt[unit];
  const int n_hist = count - 1;
  const int32_t L = p.seq_lens[s];
  const int32_t *sel = p.sel + (int64_t)unit * p.max_sel;
  const float *gts = p.gates + (int64_t)unit * p.max_sel;
  const float *dg = p.d_gates + (int64_t)unit * p.max_sel;
  const int32_t *bt = p.block_table + (int64_t)s * p.max_blocks;

  // ---- gate queries of the group: u_h = W_q[h] q_h, r_h, u_h / r_h, then the mean rotated query
  for (int e = t; e < G * kHeadDim; e += 256)
    qv[e >> 7][e & 127] = bf16_to_f32(p.q[((int64_t)s * p.n_q_heads + kvh * G) * kHeadDim + e]);
  __syncthreads();
  for (int e = t; e < G * kGateDim; e += 256) {
    const int h = e >> 7, jj = e & 127;
    const uint16_t *wrow = p.w_q + ((int64_t)(kvh * G + h) * kGateDim + jj) * kHeadDim;
    float acc = 0.f;
    for (int d = 0; d < kHeadDim; d += 8) {
      const u32x4 w = ld16(wrow + d);
      acc = fmaf(qv[h][d + 0], bf16_lo(w.x), acc);
      acc = fmaf(qv[h][d + 1], bf16_hi(w.x), acc);
      acc = fmaf(qv[h][d + 2], bf16_lo(w.y), acc);
      acc = fmaf(qv[h][d + 3], bf16_hi(w.y), acc);
      acc = fmaf(qv[h][d + 4], bf16_lo(w.z), acc);
      acc = fmaf(qv[h][d + 5], bf16_hi(w.z), acc);
      acc = fmaf(qv[h][d + 6], bf16_lo(w.w), acc);
      acc = fmaf(qv[h][d + 7], bf16_hi(w.w), acc);
    }
    un[h][jj] = acc;
  }
  __syncthreads();
  if (t < 64) {  // wave 0: per head RMS, normalise, rotate, mean over the group
    float cq, sq;
    rope_cos_sin((double)(L - 1), p.inv_freq[t], cq, sq);
    float sa = 0.f, sb = 0.f;
    for (int h = 0; h < G; ++h) {
      const float a = un[h][t], b = un[h][t + 64];
      const float r = sqrtf(wave_sum(a * a + b * b) * (1.0f / kGateDim) + 1e-6f);
      const float na = a / r, nb = b / r;
      un[h][t] = na;
      un[h][t + 64] = nb;
      if (t == 0) rr[h] = r;
      const float wa = na * p.w_qnorm[t], wb = nb * p.w_qnorm[t + 64];
      sa += wa * cq - wb * sq;
      sb += wb * cq + wa * sq;
    }
    ghat[t] = sa / (float)G;
    ghat[t + 64] = sb / (float)G;
  }
  __syncthreads();

  // ---- dghat = sum_i dS_i gk_i / sqrt(128) over the historical selection
  if (t < kGateDim) {
    float acc = 0.f;
    for (int i = 0; i < n_hist; ++i) {
      const float gi = gts[i];
      const float dS = dg[i] * gi * (1.f - gi);
      const int64_t page = bt[sel[i]];
      acc = fmaf(dS, bf16_to_f32(p.gate_keys[(page * p.n_kv_heads + kvh) * kGateDim + t]), acc);
    }
    dghat[t] = acc * kInvSqrtDg;
  }
  __syncthreads();

  // ---- query side: per head d(u/r * w) = RoPE^T(dghat / G), RMSNorm
  // backward; the norm-weight term summed over the group's heads
  if (t < 64) {
    float cq, sq;
    rope_cos_sin((double)(L - 1), p.inv_freq[t], cq, sq);
    float dna, dnb;
    rope_back(dghat[t] / (float)G, dghat[t + 64] / (float)G, cq, sq, dna, dnb);
    float wsa = 0.f, wsb = 0.f;
    for (int h = 0; h < G; ++h) {
      const float na = un[h][t], nb = un[h][t + 64];
      const float aa = dna * p.w_qnorm[t], ab = dnb * p.w_qnorm[t + 64];
      const float mean = wave_sum(aa * na + ab * nb) * (1.0f / kGateDim);
      const float r = rr[h];
      float *du = p.ws_du_q + ((int64_t)s * p.n_q_heads + kvh * G + h) * kGateDim;
      du[t] = (aa - na * mean) / r;
      du[t + 64] = (ab - nb * mean) / r;
      wsa += dna * na;
      wsb += dnb * nb;
    }
    p.ws_dwqn[(int64_t)unit * kGateDim + t] = wsa;
    p.ws_dwqn[(int64_t)unit * kGateDim + t + 64] = wsb;
  }

  // ---- key side, kChainBlocks selected historical blocks at a time
  const int64_t slot0 = (int64_t)unit * p.max_sel;
  float dwk_a = 0.f, dwk_b = 0.f;  // this lane's pair, summed over the wave's blocks
  for (int i0 = 0; i0 < p.max_sel; i0 += kChainBlocks) {
    const int nb_ = max(0, min(kChainBlocks, n_hist - i0));
    __syncthreads();
    // pooled statistics: thread (block b, dim d) scans the block's 64 rows
    for (int e = t; e < nb_ * kHeadDim; e += 256) {
      const int b = e >> 7, d = e & 127;
      const int64_t page = bt[sel[i0 + b]];
      const uint16_t *kb = p.k_pool + page * p.page_stride + (int64_t)kvh * p.head_stride + d;
      float mx = -__builtin_inff(), mn = __builtin_inff(), sum = 0.f;
#pragma unroll 16
      for (int r = 0; r < kBlock; ++r) {
        const float x = bf16_to_f32(kb[(int64_t)r * p.tok_stride]);
        mx = fmaxf(mx, x);
        mn = fminf(mn, x);
        sum += x;
      }
      pooled[b][d] = mx;
      pooled[b][kHeadDim + d] = mn;
      pooled[b][2 * kHeadDim + d] = sum * (1.0f / kBlock);
    }
    __syncthreads();
    // u = W_k[kvh] . pooled: thread (row jj, half) covers half of the chunk's blocks
    {
      const int jj = t & 127, half = t >> 7;
      const uint16_t *wrow = p.w_k + ((int64_t)kvh * kGateDim + jj) * 3 * kHeadDim;
      float acc[kChainBlocks / 2];
#pragma unroll
      for (int b = 0; b < kChainBlocks / 2; ++b) acc[b] = 0.f;
      for (int in = 0; in < 3 * kHeadDim; in += 8) {
        const u32x4 w = ld16(wrow + in);
        const float wv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                             bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
        for (int b = 0; b < kChainBlocks / 2; ++b) {
          const float *pb = pooled[half * (kChainBlocks / 2) + b] + in;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[b] = fmaf(wv[e], pb[e], acc[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < kChainBlocks / 2; ++b) uk[half * (kChainBlocks / 2) + b][jj] = acc[b];
    }
    __syncthreads();
    // per block (wave w: blocks w, w+4, ...): RMS, RoPE^T of dS * ghat / sqrt(128), RMSNorm backward
    {
      const int wave = t >> 6, lane = t & 63;
      for (int b = wave; b < kChainBlocks; b += 4) {
        const int i = i0 + b;
        float *du = p.ws_du_k + (slot0 + min(i, p.max_sel - 1)) * kGateDim;
        float *pk = p.ws_pool + (slot0 + min(i, p.max_sel - 1)) * 3 * kHeadDim;
        if (i >= p.max_sel) break;
        if (b >= nb_) {  // local block or padding: no gradient
          du[lane] = du[lane + 64] = 0.f;
          for (int e = lane; e < 3 * kHeadDim; e += 64) pk[e] = 0.f;
          continue;
        }
        const int c = sel[i];
        const float a = uk[b][lane], bb = uk[b][lane + 64];
        const float r = sqrtf(wave_sum(a * a + bb * bb) * (1.0f / kGateDim) + 1e-6f);
        const float na = a / r, nb = bb / r;
        const float gi = gts[i];
        const float dS = dg[i] * gi * (1.f - gi) * kInvSqrtDg;
        float ck, sk;
        rope_cos_sin((double)c * kBlock, p.inv_freq[lane], ck, sk);
        float dma, dmb;
        rope_back(dS * ghat[lane], dS * ghat[lane + 64], ck, sk, dma, dmb);
        const float aa = dma * p.w_knorm[lane], ab = dmb * p.w_knorm[lane + 64];
        const float mean = wave_sum(aa * na + ab * nb) * (1.0f / kGateDim);
        du[lane] = (aa - na * mean) / r;
        du[lane + 64] = (ab - nb * mean) / r;
        dwk_a += dma * na;
        dwk_b += dmb * nb;
        for (int e = lane; e < 3 * kHeadDim; e += 64) pk[e] = pooled[b][e];
      }
    }
  }
  {
    const int wave = t >> 6, lane = t & 63;
    dwk_acc[wave][lane] = dwk_a;
    dwk_acc[wave][lane + 64] = dwk_b;
  }
  __syncthreads();
  if (t < kGateDim)
    p.ws_dwkn[(int64_t)unit * kGateDim + t] = dwk_acc[0][t] + dwk_acc[1][t] + dwk_acc[2][t] + dwk_acc[3][t];
}

// ---------------------------------------------------------------- sums over the batch
// out[j][i] = sum_n a[n][j] * b[n][i] for one 64 x 64 tile: the a and b rows
// are staged in LDS 32 at a time; thread (ty, tx) owns a 4 x 4 block of the
// tile and sums the rows in order (deterministic).  b is fp32 or bf16.
template <typename TB>
__device__ __forceinline__ float load_b(const TB *b, int64_t i);
template <>
__device__ __forceinline__ float load_b<float>(const float *b, int64_t i) { return b[i]; }
template <>
__device__ __forceinline__ float load_b<uint16_t>(const uint16_t *b, int64_t i) { return bf16_to_f32(b[i]); }

template <typename TB>
__device__ void outer_sum_tile(const float *a, int64_t a_row, const TB *b, int64_t b_row, int n, int j0, int i0,
                               int i_lim, float *out, int64_t out_row, float (&as)[32][64], float (&bs)[32][64]) {
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  float acc[4][4] = {};
  for (int n0 = 0; n0 < n; n0 += 32) {
    __syncthreads();
    for (int e = t; e < 32 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const bool live = n0 + r < n;
      as[r][c] = live ? a[(int64_t)(n0 + r) * a_row + j0 + c] : 0.f;
      bs[r][c] = live && i0 + c < i_lim ? load_b(b, (int64_t)(n0 + r) * b_row + i0 + c) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int r = 0; r < 32; ++r) {
      float av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = as[r][4 * ty + u];
        bv[u] = bs[r][4 * tx + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (i0 + 4 * tx + v < i_lim) out[(int64_t)(j0 + 4 * ty + u) * out_row + i0 + 4 * tx + v] = acc[u][v];
}

// blocks [0, Hq*4): dW_q[h] tiles (2 x 2 per head), sum over the batch of
// du_q (x) q; then Hkv*12*kSplitK blocks: partial dW_k[kvh] tiles (2 x 6 per
// head, the (sequence, slot) rows split into kSplitK ranges), sums of
// du_k (x) pooled; the last block: the norm-weight gradients as sums over the
// (sequence, KV head) rows.
__global__ __launch_bounds__(256) void gate_param_reduce_kernel(BackwardParams p) {
  __shared__ float as[32][64], bs[32][64];
  const int tiles_q = p.n_q_heads * 4, tiles_k = p.n_kv_heads * 12;  // dW_k: 12 tiles of 64 x 64 per KV head
  const int bid = blockIdx.x;
  if (bid < tiles_q) {
    const int h = bid >> 2, jt = (bid >> 1) & 1, it = bid & 1;
    outer_sum_tile<uint16_t>(p.ws_du_q + (int64_t)h * kGateDim, (int64_t)p.n_q_heads * kGateDim,
                             p.q + (int64_t)h * kHeadDim, (int64_t)p.n_q_heads * kHeadDim, p.batch, 64 * jt, 64 * it,
                             kHeadDim, p.d_w_q + (int64_t)h * kGateDim * kHeadDim, kHeadDim, as, bs);
  } else if (bid < tiles_q + tiles_k * kSplitK) {
    // one of kSplitK consecutive row ranges of one dW_k tile -> a partial tile
    const int k = (bid - tiles_q) / kSplitK, part = (bid - tiles_q) % kSplitK;
    const int kvh = k / 12, jt = (k % 12) / 6, it = k % 6;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    const int n = p.batch * p.max_sel;
    const int per = (n + kSplitK - 1) / kSplitK;
    const int n_lo = part * per, n_hi = min(n, n_lo + per);
    for (int n0 = n_lo; n0 < n_hi; n0 += 32) {
      __syncthreads();
      for (int e = tid; e < 32 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;
        const int nn = n0 + r;
        const bool live = nn < n_hi;
        const int64_t slot = live ? ((int64_t)(nn / p.max_sel) * p.n_kv_heads + kvh) * p.max_sel + nn % p.max_sel : 0;
        as[r][c] = live ? p.ws_du_k[slot * kGateDim + 64 * jt + c] : 0.f;
        bs[r][c] = live ? p.ws_pool[slot * 3 * kHeadDim + 64 * it + c] : 0.f;
      }
      __syncthreads();
#pragma unroll 8
      for (int r = 0; r < 32; ++r) {
        float av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          av[u] = as[r][4 * ty + u];
          bv[u] = bs[r][4 * tx + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
      }
    }
    float *dst = p.ws_part + ((int64_t)k * kSplitK + part) * 64 * 64;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(4 * ty + u) * 64 + 4 * tx + v] = acc[u][v];
  } else if (threadIdx.x < kGateDim) {
    const int t = threadIdx.x;
    const int units = p.batch * p.n_kv_heads;
    float aq = 0.f, ak = 0.f;
    for (int u = 0; u < units; ++u) {
      aq += p.ws_dwqn[(int64_t)u * kGateDim + t];
      ak += p.ws_dwkn[(int64_t)u * kGateDim + t];
    }
    p.d_w_qnorm[t] = aq;
    p.d_w_knorm[t] = ak;
  }
}

// dW_k from its partial tiles, summed in order of the row ranges
__global__ __launch_bounds__(256) void gate_dwk_sum_kernel(BackwardParams p) {
  const int k = blockIdx.x;  // tile
  const int kvh = k / 12, jt = (k % 12) / 6, it = k % 6;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    float acc = 0.f;
    for (int part = 0; part < kSplitK; ++part) acc += p.ws_part[((int64_t)k * kSplitK + part) * 64 * 64 + e];
    p.d_w_k[((int64_t)kvh * kGateDim + 64 * jt + (e >> 6)) * 3 * kHeadDim + 64 * it + (e & 63)] = acc;
  }
}

hipError_t launch_gate_backward(const BackwardParams &p, hipStream_t st) {
  const unsigned units = (unsigned)(p.batch * p.n_kv_heads);
  hipLaunchKernelGGL(gate_grad_kernel, dim3(units), dim3(kWavesG * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_chain_kernel, dim3(units), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)(p.n_q_heads * 4 + p.n_kv_heads * 12 * kSplitK + 1);
  hipLaunchKernelGGL(gate_param_reduce_kernel, dim3(tiles), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_dwk_sum_kernel, dim3((unsigned)(p.n_kv_heads * 12)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
