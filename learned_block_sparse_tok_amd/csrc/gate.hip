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
//   gate_query_kernel   one workgroup per (query head, 16 sequences): the
//                       16 x 128 x 128 projection q . w_q[h]^T on MFMA
//                       (v_mfma_f32_16x16x32_bf16, w_q rows are 16-byte
//                       operand loads), then RMSNorm and RoPE at position L-1
//                       (angles formed and reduced in fp64); fp32 result to
//                       workspace.
//   score_topk_kernel   one workgroup per (sequence, KV head): the block-table
//                       row is staged in LDS, every candidate's gate key is
//                       gathered at once (16 lanes x 16 B per key, up to 512
//                       keys in flight per workgroup) and dotted with the mean
//                       gate query of the group (DPP row reduction); scores
//                       become order-preserving uint32 keys in the same LDS
//                       slots; an 8-bit radix select (per-wave histograms, one
//                       wave scans) finds the threshold, usually in two or
//                       three passes; the selection is marked in an LDS bitmap
//                       and one wave writes it out in ascending block order,
//                       ties at the threshold going to the lowest indices.
// Bytes per (sequence, KV head): 256 B of gate key per candidate block.
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {

constexpr int kGqTile = 16;  // sequences per gate-query workgroup (MFMA rows)

__device__ __forceinline__ bf16x8 as_bf16x8_g(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ __launch_bounds__(256) void gate_query_kernel(GateQueryParams p) {
  const int h = blockIdx.x;
  const int s0 = blockIdx.y * kGqTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  __shared__ float g[kGqTile][kGateDim + 4];
  __shared__ double inv_freq[kGateDim / 2];
  if (threadIdx.x < kGateDim / 2) inv_freq[threadIdx.x] = pow(p.theta, -(double)threadIdx.x / 64.0);

  // A operand: q rows of 16 sequences, lane holds q[s0+row][32ks + 8kg .. +7]
  bf16x8 qa[4];
  {
    const bool valid = s0 + row < p.batch;
    const uint16_t *qrow = p.q + ((int64_t)(s0 + row) * p.n_q_heads + h) * kHeadDim + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = as_bf16x8_g(valid ? ld16(qrow + 32 * ks) : u32x4{0, 0, 0, 0});
  }
  // B operand: w_q[h] is [j][d]; lane holds w_q[h][16nt + row][32ks + 8kg .. +7]
  const uint16_t *wh = p.w_q + (int64_t)h * kGateDim * kHeadDim;
#pragma unroll
  for (int n2 = 0; n2 < 2; ++n2) {
    const int nt = 2 * wave + n2;
    const uint16_t *wrow = wh + (int64_t)(16 * nt + row) * kHeadDim + 8 * kg;
    u32x4 wb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wb[ks] = ld16(wrow + 32 * ks);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], as_bf16x8_g(wb[ks]), acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) g[4 * kg + r][16 * nt + row] = acc[r];
  }
  __syncthreads();

  // RMSNorm + RoPE: thread (sequence t/16, pairs 4(t%16) .. +3 with partners +64)
  const int sq = threadIdx.x >> 4, q4 = threadIdx.x & 15;
  float a[4], b[4], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = g[sq][4 * q4 + e];
    b[e] = g[sq][4 * q4 + e + 64];
    ss += a[e] * a[e] + b[e] * b[e];
  }
  ss = row16_sum(ss);
  if (s0 + sq < p.batch) {
    const float inv = 1.0f / sqrtf(ss * (1.0f / kGateDim) + 1e-6f);
    const double pos = (double)(p.seq_lens[s0 + sq] - 1);
    float *dst = p.gq + ((int64_t)(s0 + sq) * p.n_q_heads + h) * kGateDim;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pj = 4 * q4 + e;
      const float av = a[e] * inv * p.w_qnorm[pj];
      const float bv = b[e] * inv * p.w_qnorm[pj + 64];
      float cf, sf;
      rope_cos_sin(pos, inv_freq[pj], cf, sf);
      dst[pj] = av * cf - bv * sf;
      dst[pj + 64] = bv * cf + av * sf;
    }
  }
}

constexpr int kKeysInFlight = 32;  // gate keys per 16-lane group per pass (512 per workgroup)
constexpr int kMaxBitWords = SAS_MAX_BLOCKS_DEV / 32;

__global__ __launch_bounds__(256) void score_topk_kernel(ScoreTopkParams p) {
  extern __shared__ uint32_t slot[];  // [max_blocks]: block-table row, then score keys
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t selbits[kMaxBitWords], eqbits[kMaxBitWords];
  __shared__ uint32_t sh_T, sh_krem, sh_full;

  const int sk = blockIdx.x;
  const int s = sk / p.n_kv_heads;
  const int kvh = sk - s * p.n_kv_heads;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int lane16 = t & 15, grp = t >> 4;
  const int32_t L = p.seq_lens[s];
  const int n = (L - 1) / kBlock;  // candidates: the blocks before the local block
  const int k_eff = min(p.n_sel - 1, n);
  const int nwords = (n + 31) >> 5;

  const int32_t *bt = p.block_table + (int64_t)s * p.max_blocks;
  for (int c = t; c < n; c += 256) slot[c] = (uint32_t)bt[c];
  for (int i = t; i < nwords; i += 256) {
    selbits[i] = 0;
    eqbits[i] = 0;
  }

  // mean gate query of the group, dims 8*lane16 .. +7
  float gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] = 0.f;
  for (int g = 0; g < p.group; ++g) {
    const float *src = p.gq + ((int64_t)s * p.n_q_heads + kvh * p.group + g) * kGateDim + 8 * lane16;
    const f32x4 x = *reinterpret_cast<const f32x4 *>(src);
    const f32x4 y = *reinterpret_cast<const f32x4 *>(src + 4);
    gm[0] += x.x; gm[1] += x.y; gm[2] += x.z; gm[3] += x.w;
    gm[4] += y.x; gm[5] += y.y; gm[6] += y.z; gm[7] += y.w;
  }
  const float inv_g = 1.0f / (float)p.group;
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] *= inv_g;
  __syncthreads();

  const float inv_sqrt_dg = 0.08838834764831845f;  // 1/sqrt(128)
  float *scores = p.scores + (int64_t)sk * p.max_blocks;
  const uint16_t *gkh = p.gate_keys + (int64_t)kvh * kGateDim + 8 * lane16;
  const int64_t page_stride = (int64_t)p.n_kv_heads * kGateDim;
  for (int base = 0; base < n; base += 16 * kKeysInFlight) {
    u32x4 v[kKeysInFlight];
#pragma unroll
    for (int u = 0; u < kKeysInFlight; ++u) {
      const int c = base + 16 * u + grp;
      v[u] = c < n ? ld16(gkh + (int64_t)slot[c] * page_stride) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kKeysInFlight; ++u) {
      float d = gm[0] * bf16_lo(v[u].x);
      d = fmaf(gm[1], bf16_hi(v[u].x), d);
      d = fmaf(gm[2], bf16_lo(v[u].y), d);
      d = fmaf(gm[3], bf16_hi(v[u].y), d);
      d = fmaf(gm[4], bf16_lo(v[u].z), d);
      d = fmaf(gm[5], bf16_hi(v[u].z), d);
      d = fmaf(gm[6], bf16_lo(v[u].w), d);
      d = fmaf(gm[7], bf16_hi(v[u].w), d);
      d = row16_sum(d);
      const int c = base + 16 * u + grp;
      if (lane16 == 0 && c < n) {
        const float sc = d * inv_sqrt_dg;
        slot[c] = score_key(sc);
        scores[c] = sc;
      }
    }
  }
  for (int c = n + t; c < p.max_blocks; c += 256) scores[c] = -__builtin_inff();
  __syncthreads();

  // ---- threshold: take every key > T, and the krem lowest-index keys == T
  uint32_t T = 0, krem = 0;  // k_eff >= n: every candidate (all keys are > 0)
  if (k_eff > 0 && k_eff < n) {
    uint32_t prefix = 0, mask = 0;
    krem = (uint32_t)k_eff;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = t; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int i = t; i < n; i += 256) {
        const uint32_t k = slot[i];
        if ((k & mask) == prefix) atomicAdd(&hist[wave][(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns digits 255-4l .. 252-4l (descending)
        uint32_t cnt[4], tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 255 - (4 * lane + e);
          cnt[e] = hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d];
          tot += cnt[e];
        }
        uint32_t incl = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        uint32_t run = incl - tot;  // keys in higher digits
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (run < krem && run + cnt[e] >= krem) {
            const uint32_t d = 255u - (uint32_t)(4 * lane + e);
            sh_T = prefix | (d << shift);
            sh_krem = krem - run;
            sh_full = cnt[e] == krem - run;
          }
          run += cnt[e];
        }
      }
      __syncthreads();
      prefix = sh_T;
      krem = sh_krem;
      mask |= 0xFFu << shift;
      if (sh_full) {  // the whole bin is taken: every key >= prefix
        T = prefix - 1u;  // prefix > 0 here: some keys lie below the bin
        krem = 0;
        break;
      }
      T = prefix;
    }
  }

  // ---- mark the selection, then write it in ascending block order
  const int n_sel = p.n_sel;
  int32_t *sel = p.sel + (int64_t)sk * n_sel;
  float *gates = p.gates ? p.gates + (int64_t)sk * n_sel : nullptr;
  if (k_eff > 0) {
    for (int i = t; i < n; i += 256) {
      const uint32_t k = slot[i];
      if (k > T) atomicOr(&selbits[i >> 5], 1u << (i & 31));
      else if (k == T && krem > 0) atomicOr(&eqbits[i >> 5], 1u << (i & 31));
    }
    __syncthreads();
    if (wave == 0) {
      const int wpl = (nwords + 63) / 64;
      const int w0 = min(nwords, lane * wpl), w1 = min(nwords, w0 + wpl);
      if (krem > 0) {  // the krem lowest-index keys equal to T
        uint32_t c = 0;
        for (int i = w0; i < w1; ++i) c += __popc(eqbits[i]);
        uint32_t incl = c;
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        uint32_t before = incl - c;
        for (int i = w0; i < w1 && before < krem; ++i) {
          uint32_t bits = eqbits[i];
          while (bits && before < krem) {
            const uint32_t low = bits & (0u - bits);
            selbits[i] |= low;
            bits ^= low;
            ++before;
          }
        }
      }
      uint32_t c = 0;
      for (int i = w0; i < w1; ++i) c += __popc(selbits[i]);
      uint32_t incl = c;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      uint32_t pos = incl - c;
      for (int i = w0; i < w1; ++i) {
        uint32_t bits = selbits[i];
        while (bits) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          const int idx = 32 * i + b;
          sel[pos] = idx;
          if (gates) gates[pos] = 1.0f / (1.0f + expf(-key_score(slot[idx])));
          ++pos;
        }
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
  dim3 grid((unsigned)p.n_q_heads, (unsigned)((p.batch + kGqTile - 1) / kGqTile));
  hipLaunchKernelGGL(gate_query_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_score_topk(const ScoreTopkParams &p, int batch, hipStream_t st) {
  const size_t lds = sizeof(uint32_t) * (size_t)p.max_blocks;
  // allow the largest block-table row (64 KiB of LDS); set once per process
  static const hipError_t attr = hipFuncSetAttribute((const void *)score_topk_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)(sizeof(uint32_t) * SAS_MAX_BLOCKS_DEV));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(score_topk_kernel, dim3((unsigned)(batch * p.n_kv_heads)), dim3(256), lds, st, p);
  return hipGetLastError();
}

}  // namespace sas
