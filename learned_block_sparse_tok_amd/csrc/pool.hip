// Key-block pooling -> gate keys.
//
// SAS pools each 64-token key block by max, min and average and maps the
// pooled statistics to a 128-wide gate key with Q/K normalisation and gate
// RoPE ("Tencent released Simple-Attention-Sparsification ...", aigc.news,
// the setup paragraph; "Specifications and Configuration Table" of the
// localmodelwatch model page: KV block size 64, gate hidden size 128, key
// block pooling max + min + average, Q/K normalization, gate RoPE).
//
// One workgroup (256 threads) per (listed block, KV head):
//   1. a coalesced pass over the 64 x 128 bf16 key rows: per dimension the
//      running max / min / fp32 sum of 32 rows per thread, halves combined
//      in LDS -> pooled[384] = [max | min | mean];
//   2. the 128 x 384 projection w_k[h] . pooled: 16 lanes per w_k row (every
//      load instruction reads whole rows), reduced across the lanes (DPP);
//   3. wave 0: RMSNorm (eps 1e-6) * w_knorm, rotate-half RoPE at position
//      64*c (angles formed and reduced in fp64), round to bf16, store.
// Bytes per (block, KV head): 16 KiB of keys read, 256 B of gate key written
// (w_k is 96 KiB per KV head and stays in L2).
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {

__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  const int unit = blockIdx.x;
  const int i = unit / p.n_kv_heads;
  const int kvh = unit - i * p.n_kv_heads;
  const int t = threadIdx.x;
  const int s = p.pool_seq[i], c = p.pool_blk[i];
  const int32_t page = p.block_table[(int64_t)s * p.max_blocks + c];
  const uint16_t *kb = p.k_pool + (int64_t)page * p.page_stride + (int64_t)kvh * p.head_stride;

  __shared__ float part[2][3][kHeadDim];
  __shared__ float pooled[3 * kHeadDim];
  __shared__ float upart[1][kGateDim];

  {  // 1. pooled statistics
    const int d = t & (kHeadDim - 1);
    const int half = t >> 7;
    float mx = -__builtin_inff(), mn = __builtin_inff(), sum = 0.f;
#pragma unroll 8
    for (int r = 0; r < kBlock / 2; ++r) {
      float x = bf16_to_f32(kb[(int64_t)(half * (kBlock / 2) + r) * p.tok_stride + d]);
      mx = fmaxf(mx, x);
      mn = fminf(mn, x);
      sum += x;
    }
    part[half][0][d] = mx;
    part[half][1][d] = mn;
    part[half][2][d] = sum;
  }
  __syncthreads();
  if (t < kHeadDim) {
    pooled[t] = fmaxf(part[0][0][t], part[1][0][t]);
    pooled[kHeadDim + t] = fminf(part[0][1][t], part[1][1][t]);
    pooled[2 * kHeadDim + t] = (part[0][2][t] + part[1][2][t]) * (1.0f / kBlock);
  }
  __syncthreads();
  {  // 2. projection to the gate space: each 16-lane group owns 8 output rows
     // j; a lane holds 24 of a row's 384 inputs (three 16-byte chunks), so a
     // wave reads 4 whole rows per load; the group reduces across its lanes.
    const int lane16 = t & 15, grp = t >> 4;
    const uint16_t *w = p.w_k + ((int64_t)kvh * kGateDim + 8 * grp) * 3 * kHeadDim + 8 * lane16;
    u32x4 wv[8][3];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int k = 0; k < 3; ++k) wv[r][k] = ld16(w + r * 3 * kHeadDim + 128 * k);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float *pp = pooled + 128 * k + 8 * lane16;
        acc = fmaf(pp[0], bf16_lo(wv[r][k].x), acc);
        acc = fmaf(pp[1], bf16_hi(wv[r][k].x), acc);
        acc = fmaf(pp[2], bf16_lo(wv[r][k].y), acc);
        acc = fmaf(pp[3], bf16_hi(wv[r][k].y), acc);
        acc = fmaf(pp[4], bf16_lo(wv[r][k].z), acc);
        acc = fmaf(pp[5], bf16_hi(wv[r][k].z), acc);
        acc = fmaf(pp[6], bf16_lo(wv[r][k].w), acc);
        acc = fmaf(pp[7], bf16_hi(wv[r][k].w), acc);
      }
      acc = row16_sum(acc);
      if (lane16 == 0) upart[0][8 * grp + r] = acc;
    }
  }
  __syncthreads();
  if (t < 64) {  // 3. norm + RoPE on pairs (t, t+64)
    float a = upart[0][t];
    float b = upart[0][t + 64];
    float ss = wave_sum(a * a + b * b);
    float inv = 1.0f / sqrtf(ss * (1.0f / kGateDim) + 1e-6f);
    a = a * inv * p.w_knorm[t];
    b = b * inv * p.w_knorm[t + 64];
    float cf, sf;
    rope_cos_sin((double)c * kBlock, pow(p.theta, -(double)t / 64.0), cf, sf);
    float ra = a * cf - b * sf;
    float rb = b * cf + a * sf;
    uint16_t *dst = p.gate_keys + ((int64_t)page * p.n_kv_heads + kvh) * kGateDim;
    dst[t] = (uint16_t)f32_to_bf16(ra);
    dst[t + 64] = (uint16_t)f32_to_bf16(rb);
  }
}

hipError_t launch_pool(const PoolParams &p, hipStream_t st) {
  if (p.n == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3((unsigned)(p.n * p.n_kv_heads)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
