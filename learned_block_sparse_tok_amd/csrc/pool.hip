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
//
// The same pooling also runs inside the decode step's cache write
// (append_kernel): the step that writes a block's last row pools the block
// there, instead of a second launch re-reading that row.
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {

// Gate key of one 64-token key block of one KV head.  Every thread of a
// 256-thread workgroup calls it (it holds barriers).  kb: the block's row 0 of
// this head; last_row: when non-null, row 63 is read from there instead of
// from the pool (the append kernel passes the row it is writing).
__device__ __forceinline__ void pool_unit(const uint16_t *kb, int64_t tok_stride, const uint16_t *last_row,
                                          const uint16_t *w_kh, const float *w_knorm, double theta, int c,
                                          uint16_t *dst) {
  __shared__ float part[2][3][kHeadDim];
  __shared__ float pooled[3 * kHeadDim];
  __shared__ float upart[kGateDim];
  const int t = threadIdx.x;

  {  // 1. pooled statistics
    const int d = t & (kHeadDim - 1);
    const int half = t >> 7;
    float mx = -__builtin_inff(), mn = __builtin_inff(), sum = 0.f;
#pragma unroll 8
    for (int r = 0; r < kBlock / 2; ++r) {
      const int row = half * (kBlock / 2) + r;
      const uint16_t *src = (last_row && row == kBlock - 1) ? last_row : kb + (int64_t)row * tok_stride;
      float x = bf16_to_f32(src[d]);
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
    const uint16_t *w = w_kh + (int64_t)(8 * grp) * 3 * kHeadDim + 8 * lane16;
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
      if (lane16 == 0) upart[8 * grp + r] = acc;
    }
  }
  __syncthreads();
  if (t < 64) {  // 3. norm + RoPE on pairs (t, t+64)
    float a = upart[t];
    float b = upart[t + 64];
    float ss = wave_sum(a * a + b * b);
    float inv = 1.0f / sqrtf(ss * (1.0f / kGateDim) + 1e-6f);
    a = a * inv * w_knorm[t];
    b = b * inv * w_knorm[t + 64];
    float cf, sf;
    rope_cos_sin((double)c * kBlock, pow(theta, -(double)t / 64.0), cf, sf);
    float ra = a * cf - b * sf;
    float rb = b * cf + a * sf;
    dst[t] = (uint16_t)f32_to_bf16(ra);
    dst[t + 64] = (uint16_t)f32_to_bf16(rb);
  }
}

__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  const int unit = blockIdx.x;
  const int i = unit / p.n_kv_heads;
  const int kvh = unit - i * p.n_kv_heads;
  const int s = p.pool_seq[i], c = p.pool_blk[i];
  const int32_t page = p.block_table[(int64_t)s * p.max_blocks + c];
  pool_unit(p.k_pool + (int64_t)page * p.page_stride + (int64_t)kvh * p.head_stride, p.tok_stride, nullptr,
            p.w_k + (int64_t)kvh * kGateDim * 3 * kHeadDim, p.w_knorm, p.theta, c,
            p.gate_keys + ((int64_t)page * p.n_kv_heads + kvh) * kGateDim);
}

// One workgroup per (sequence, KV head): threads 0-15 write the new key row,
// 16-31 the value row (16 bytes each); when the row completes its block
// (L % 64 == 0) the whole workgroup pools that block, taking row 63 from
// k_new.  Bytes per (sequence, KV head): 512 B read + 512 B written, plus
// 16 KiB - 256 B of keys read and 256 B written per completed block.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int unit = blockIdx.x;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int t = threadIdx.x;
  const int L = p.seq_lens[s];
  const int pos = L - 1;
  const int c = pos / kBlock, r = pos - c * kBlock;
  const int32_t page = p.block_table[(int64_t)s * p.max_blocks + c];
  const int64_t base = (int64_t)page * p.page_stride + (int64_t)kvh * p.head_stride;
  const int64_t src = ((int64_t)s * p.n_kv_heads + kvh) * kHeadDim;
  if (t < 32) {
    const int lane = t & 15;
    const uint16_t *from = (t < 16 ? p.k_new : p.v_new) + src + 8 * lane;
    uint16_t *to = (t < 16 ? p.k_pool : p.v_pool) + base + (int64_t)r * p.tok_stride + 8 * lane;
    *(u32x4 *)to = ld16(from);
  }
  if (L % kBlock == 0)
    pool_unit(p.k_pool + base, p.tok_stride, p.k_new + src, p.w_k + (int64_t)kvh * kGateDim * 3 * kHeadDim,
              p.w_knorm, p.theta, c, p.gate_keys + ((int64_t)page * p.n_kv_heads + kvh) * kGateDim);
}

hipError_t launch_pool(const PoolParams &p, hipStream_t st) {
  if (p.n == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3((unsigned)(p.n * p.n_kv_heads)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams &p, int batch, hipStream_t st) {
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)(batch * p.n_kv_heads)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
