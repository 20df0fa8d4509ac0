// Gate query, block scores and per-KV-head Top-K.
//
// SAS scores the KV blocks for each decode query through a query projection
// ("Qproj") with Q/K normalisation and gate RoPE, and keeps a Top-K of 31
// historical blocks plus the local block for the default 2,048-token budget
// (1,024 / 4,096 also) ("Tencent released Simple-Attention-Sparsification
// ...", aigc.news, setup paragraph; localmodelwatch "Specifications and
// Configuration Table").  Each selected block gets a continuous gate.
//
// Two kernels:
//   gate_query_kernel   one workgroup per (query head, 8 sequences): q @ w_q[h]
//                       with w_q[h] read once per workgroup, RMSNorm, RoPE at
//                       position L-1 (fp64 angles); fp32 result to workspace.
//   score_topk_kernel   one workgroup per (sequence, KV head): the mean gate
//                       query of the group against every candidate's gate key
//                       (16 lanes x 16 B per key, gathered through the block
//                       table, DPP row reduction), keys kept in LDS as
//                       order-preserving uint32; exact Top-K by a 4-pass
//                       8-bit radix select over the whole workgroup; ties at
//                       the threshold go to the lowest block indices; the
//                       selection is written in ascending order by two
//                       workgroup prefix sums.
// Bytes per (sequence, KV head): 256 B of gate key per candidate block.
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {

constexpr int kGqSeqs = 8;  // sequences per gate-query workgroup

__global__ __launch_bounds__(128) void gate_query_kernel(GateQueryParams p) {
  const int h = blockIdx.x;
  const int s0 = blockIdx.y * kGqSeqs;
  const int ns = min(kGqSeqs, p.batch - s0);
  const int j = threadIdx.x;  // output dimension
  __shared__ float qs[kGqSeqs][kHeadDim];
  __shared__ float vs[kGqSeqs][kGateDim];
  __shared__ float red[2][kGqSeqs];

  for (int i = 0; i < kGqSeqs; ++i)
    qs[i][j] = i < ns ? bf16_to_f32(p.q[((int64_t)(s0 + i) * p.n_q_heads + h) * kHeadDim + j]) : 0.f;
  __syncthreads();

  float acc[kGqSeqs];
#pragma unroll
  for (int i = 0; i < kGqSeqs; ++i) acc[i] = 0.f;
  const uint16_t *w = p.w_q + (int64_t)h * kHeadDim * kGateDim + j;
#pragma unroll 4
  for (int d = 0; d < kHeadDim; ++d) {
    float wv = bf16_to_f32(w[d * kGateDim]);
#pragma unroll
    for (int i = 0; i < kGqSeqs; ++i) acc[i] = fmaf(qs[i][d], wv, acc[i]);
  }
  // RMSNorm: sum of squares over the 128 dimensions (two waves)
#pragma unroll
  for (int i = 0; i < kGqSeqs; ++i) {
    float ss = wave_sum(acc[i] * acc[i]);
    if ((j & 63) == 0) red[j >> 6][i] = ss;
  }
  __syncthreads();
  const float wn = p.w_qnorm[j];
#pragma unroll
  for (int i = 0; i < kGqSeqs; ++i) {
    float inv = 1.0f / sqrtf((red[0][i] + red[1][i]) * (1.0f / kGateDim) + 1e-6f);
    vs[i][j] = acc[i] * inv * wn;
  }
  __syncthreads();
  // RoPE at the current token's position: thread j rotates pair (j & 63) of
  // the sequences i = j >> 6, (j >> 6) + 2, ...
  const int pj = j & 63;
  const double inv_freq = pow(p.theta, -(double)pj / 64.0);
  for (int i = j >> 6; i < ns; i += 2) {
    double ang = (double)(p.seq_lens[s0 + i] - 1) * inv_freq;
    double sn, cs;
    sincos(ang, &sn, &cs);
    float cf = (float)cs, sf = (float)sn;
    float a = vs[i][pj], b = vs[i][pj + 64];
    float *dst = p.gq + ((int64_t)(s0 + i) * p.n_q_heads + h) * kGateDim;
    dst[pj] = a * cf - b * sf;
    dst[pj + 64] = b * cf + a * sf;
  }
}

// Inclusive prefix sum of one uint32 per thread over a 256-thread workgroup.
__device__ __forceinline__ uint32_t wg_incl_scan(uint32_t v, uint32_t *tmp /* [4] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t n = __shfl_up(v, off, 64);
    if (lane >= off) v += n;
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int k = 0; k < w; ++k) add += tmp[k];
  __syncthreads();
  return v + add;
}

constexpr int kScoreUnroll = 8;  // gate keys in flight per 16-lane group

__global__ __launch_bounds__(256) void score_topk_kernel(ScoreTopkParams p) {
  extern __shared__ uint32_t keys[];  // [max_blocks]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_tmp[4];
  __shared__ uint32_t sh_prefix, sh_krem;

  const int sk = blockIdx.x;
  const int s = sk / p.n_kv_heads;
  const int kvh = sk - s * p.n_kv_heads;
  const int t = threadIdx.x;
  const int lane16 = t & 15, grp = t >> 4;
  const int32_t L = p.seq_lens[s];
  const int n = (L - 1) / kBlock;  // candidates: blocks before the local block
  const int k_hist = p.n_sel - 1;
  const int k_eff = min(k_hist, n);

  // mean gate query of this KV head's group, dims 8*lane16 .. +7
  float gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] = 0.f;
  for (int g = 0; g < p.group; ++g) {
    const float *src = p.gq + ((int64_t)s * p.n_q_heads + kvh * p.group + g) * kGateDim + 8 * lane16;
    f32x4 a = *reinterpret_cast<const f32x4 *>(src);
    f32x4 b = *reinterpret_cast<const f32x4 *>(src + 4);
    gm[0] += a.x; gm[1] += a.y; gm[2] += a.z; gm[3] += a.w;
    gm[4] += b.x; gm[5] += b.y; gm[6] += b.z; gm[7] += b.w;
  }
  const float inv_g = 1.0f / (float)p.group;
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] *= inv_g;

  const float inv_sqrt_dg = 0.08838834764831845f;  // 1/sqrt(128)
  const int32_t *bt = p.block_table + (int64_t)s * p.max_blocks;
  float *scores = p.scores + (int64_t)sk * p.max_blocks;
  for (int base = 0; base < n; base += 16 * kScoreUnroll) {
    u32x4 v[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      int c = base + u * 16 + grp;
      if (c < n) {
        int32_t page = bt[c];
        v[u] = ld16(p.gate_keys + ((int64_t)page * p.n_kv_heads + kvh) * kGateDim + 8 * lane16);
      } else {
        v[u] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      float d = gm[0] * bf16_lo(v[u].x);
      d = fmaf(gm[1], bf16_hi(v[u].x), d);
      d = fmaf(gm[2], bf16_lo(v[u].y), d);
      d = fmaf(gm[3], bf16_hi(v[u].y), d);
      d = fmaf(gm[4], bf16_lo(v[u].z), d);
      d = fmaf(gm[5], bf16_hi(v[u].z), d);
      d = fmaf(gm[6], bf16_lo(v[u].w), d);
      d = fmaf(gm[7], bf16_hi(v[u].w), d);
      d = row16_sum(d);
      int c = base + u * 16 + grp;
      if (lane16 == 0 && c < n) {
        float sc = d * inv_sqrt_dg;
        keys[c] = score_key(sc);
        scores[c] = sc;
      }
    }
  }
  for (int c = n + t; c < p.max_blocks; c += 256) scores[c] = -__builtin_inff();
  __syncthreads();

  // ---- exact Top-K: threshold key T and how many keys equal to T to take
  uint32_t T = 0, krem = 0;  // k_eff >= n: every candidate (all keys > 0)
  if (k_eff > 0 && k_eff < n) {
    uint32_t prefix = 0, mask = 0;
    krem = (uint32_t)k_eff;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[t] = 0;
      __syncthreads();
      for (int i = t; i < n; i += 256) {
        uint32_t k = keys[i];
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      const uint32_t dig = 255u - (uint32_t)t;
      const uint32_t hv = hist[dig];
      const uint32_t ge = wg_incl_scan(hv, scan_tmp);  // keys with digit >= dig
      if (ge >= krem && ge - hv < krem) {
        sh_prefix = prefix | (dig << shift);
        sh_krem = krem - (ge - hv);
      }
      __syncthreads();
      prefix = sh_prefix;
      krem = sh_krem;
      mask |= 0xFFu << shift;
    }
    T = prefix;
  }

  // ---- ordered compaction: thread t owns candidates [t*m, t*m + m)
  const int n_sel = p.n_sel;
  int32_t *sel = p.sel + (int64_t)sk * n_sel;
  float *gates = p.gates ? p.gates + (int64_t)sk * n_sel : nullptr;
  if (k_eff > 0) {
    const int m = (n + 255) / 256;
    const int lo = min(n, t * m), hi = min(n, lo + m);
    uint32_t eq = 0;
    for (int i = lo; i < hi; ++i) eq += keys[i] == T;
    uint32_t eq_before = wg_incl_scan(eq, scan_tmp) - eq;
    uint32_t take = 0;
    for (int i = lo; i < hi; ++i) {
      uint32_t k = keys[i];
      if (k > T || (k == T && eq_before++ < krem)) ++take;
    }
    uint32_t pos = wg_incl_scan(take, scan_tmp) - take;
    eq_before = wg_incl_scan(eq, scan_tmp) - eq;
    for (int i = lo; i < hi; ++i) {
      uint32_t k = keys[i];
      if (k > T || (k == T && eq_before++ < krem)) {
        sel[pos] = i;
        if (gates) gates[pos] = 1.0f / (1.0f + expf(-key_score(k)));
        ++pos;
      }
    }
  }
  for (int i = k_eff + t; i < n_sel; i += 256) {
    sel[i] = i == k_eff ? n : -1;
    if (gates) gates[i] = i == k_eff ? 1.0f : 0.0f;
  }
  if (t == 0) p.cnt[sk] = k_eff + 1;
}

hipError_t launch_gate_query(const GateQueryParams &p, hipStream_t st) {
  dim3 grid((unsigned)p.n_q_heads, (unsigned)((p.batch + kGqSeqs - 1) / kGqSeqs));
  hipLaunchKernelGGL(gate_query_kernel, grid, dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_score_topk(const ScoreTopkParams &p, int batch, hipStream_t st) {
  size_t lds = sizeof(uint32_t) * (size_t)p.max_blocks;
  hipLaunchKernelGGL(score_topk_kernel, dim3((unsigned)(batch * p.n_kv_heads)), dim3(256), lds, st, p);
  return hipGetLastError();
}

}  // namespace sas
