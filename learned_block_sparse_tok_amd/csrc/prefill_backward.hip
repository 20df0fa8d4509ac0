// Backward of the continuous gates of the training-time forward of one
// sequence, down to the gate parameters.
//
// SAS trains its gates with the language-model loss on 32,768-token
// sequences, every query selecting its own blocks ("Tencent released
// Simple-Attention-Sparsification ...", aigc.news: training Top-K of 31
// historical blocks, the LM loss ranking the context end to end; "Tencent
// Hunyuan open-sources SAS ...": per-query selection, a differentiable path
// from the loss to the selector).  Position t is the decode step whose cache
// holds its first t+1 tokens, so the loss is a sum over positions and the
// gradient is the sum of the per-step gradients (the decode-step form is in
// backward.hip):
//   dg_{t,i}  = sum_{h in group} sum_{j in block c_i, j <= t} P_thj <dO_th, v_j>
//   dS_{t,i}  = dg_{t,i} g_{t,i} (1 - g_{t,i})                (historical blocks)
//   dghat_t   = sum_i dS_{t,i} gk_{c_i} / sqrt(128)
//   dgk_c     = sum over the (t, i) that selected c of dS_{t,i} ghat_t / sqrt(128)
// then RoPE^T, RMSNorm backward and the bias-free projections, summed over
// the positions (query side) and over the blocks (key side).
//
// Kernels, in launch order:
//   prefill_grad_kernel (prefill.hip)  dg per (position, KV head, slot), per
//     workgroup head group, from the walk of the forward with the forward's
//     log-sum-exp.
//   prefill_pool_stats_kernel  max / min / mean of every block that can be
//     historical, per KV head (the inputs of the gate-key projection).
//   prefill_chain_kernel  per (64 positions, KV head): dg and dS of the
//     positions' slots, the gate queries recomputed on MFMA and their group
//     mean, dghat, the query side down to d(pre-norm gate query) and the
//     query-norm weight terms, and the rows of the dense matrix A (position x
//     block, dS / sqrt(128) where the position selected the block) through
//     which dgk becomes a plain contraction: dgk = A^T ghat.
//   prefill_tiles_kernel  128 x 128 tiles of dW_q = sum_t du_q (x) q and of
//     dgk = A^T ghat as partial sums over kPrefillSplit ranges of positions
//     (A is lower-triangular by blocks: a column tile of blocks starts at the
//     first position that can select it).
//   prefill_sums_kernel  the partial tiles added in order; dw_qnorm.
//   prefill_key_chain_kernel  per (16 blocks, KV head): the pre-norm gate key
//     recomputed on MFMA from the pooled statistics, RoPE^T and RMSNorm
//     backward of dgk, the key-norm weight terms.
//   prefill_final_kernel  dW_k = sum_c du_k (x) pooled, and dw_knorm.
// Every sum runs in a fixed order: the result is deterministic.
#include "backward_common.h"
#include "prefill_backward.h"

namespace sas {
namespace {

constexpr int kUnPitch = kGateDim + 4;  // LDS row of one position's 128 projection outputs (floats)
constexpr int kMaxSelP = 64;            // selection slots per position (budgets up to 4,096 tokens)

// sum over the 4 lanes 4p .. 4p+3 that hold one position's dims
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  return x;
}

}  // namespace

// ---------------------------------------------------------------- pooled statistics
// One 256-thread workgroup per (block, KV head); thread t scans rows
// 32(t/128) .. +31 of dim t%128, and the two halves are combined in LDS.
__global__ __launch_bounds__(256) void prefill_pool_stats_kernel(PrefillBackwardParams p) {
  __shared__ float red[2][3][kHeadDim];
  const int kvh = blockIdx.x % p.n_kv_heads, c = blockIdx.x / p.n_kv_heads;
  const int d = threadIdx.x & (kHeadDim - 1), half = threadIdx.x >> 7;
  const uint16_t *kr = p.k_pool + (int64_t)p.block_table[c] * p.page_stride + (int64_t)kvh * p.head_stride + d;
  float mx = -__builtin_inff(), mn = __builtin_inff(), sm = 0.f;
#pragma unroll 8
  for (int r = 32 * half; r < 32 * half + 32; ++r) {
    const float v = bf16_to_f32(kr[(int64_t)r * p.tok_stride]);
    mx = fmaxf(mx, v);
    mn = fminf(mn, v);
    sm += v;
  }
  red[half][0][d] = mx;
  red[half][1][d] = mn;
  red[half][2][d] = sm;
  __syncthreads();
  if (half == 0) {
    float *dst = p.ws_pool + ((int64_t)kvh * p.n_hist + c) * 3 * kHeadDim;
    dst[d] = fmaxf(red[0][0][d], red[1][0][d]);
    dst[kHeadDim + d] = fminf(red[0][1][d], red[1][1][d]);
    dst[2 * kHeadDim + d] = (red[0][2][d] + red[1][2][d]) * (1.0f / kBlock);
  }
}

// ---------------------------------------------------------------- per 64 positions: the chain
// Thread (p = t/4, o = t%4) owns position t0 + p and the dims
// 16o + e, 64 + 16o + e (e < 16): the RoPE pairs (d, d + 64) of its 16 dims.
// The gate-query projections u = W_q[h] q_t of the 64 positions run on MFMA
// (wave w: outputs 32w .. 32w+31, positions as the B operand's columns) and
// reach the thread layout through LDS.
__global__ __launch_bounds__(256) void prefill_chain_kernel(PrefillBackwardParams p) {
  __shared__ __attribute__((aligned(16))) float un[kBlock][kUnPitch];
  // the positions' selections, first; then the query-norm weight terms
  // (dn * n summed over the heads) of the positions' dims
  __shared__ __attribute__((aligned(16))) uint8_t slots[kBlock * kMaxSelP * (2 + 4 + 4)];
  static_assert(sizeof(slots) >= sizeof(float) * kBlock * kUnPitch, "weight terms exceed the selection buffer");
  auto sel_l = reinterpret_cast<int16_t(*)[kMaxSelP]>(slots);  // historical blocks of each position, ascending
  auto page_l = reinterpret_cast<int32_t(*)[kMaxSelP]>(slots + kBlock * kMaxSelP * 2);
  auto ds_l = reinterpret_cast<float(*)[kMaxSelP]>(slots + kBlock * kMaxSelP * 6);  // dS / sqrt(128)
  auto wsum_l = reinterpret_cast<float(*)[kUnPitch]>(slots);
  __shared__ int nh_l[kBlock];                 // historical blocks per position
  __shared__ float wqn_l[kGateDim];            // w_qnorm

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int pp = tid >> 2, o = tid & 3;
  const int kvh = blockIdx.x % p.n_kv_heads, tau = blockIdx.x / p.n_kv_heads;  // KV head fastest: one per XCD
  const int G = p.group, Hq = p.n_q_heads, Hkv = p.n_kv_heads, S = p.max_sel, T = p.seq_len;
  const int t0 = tau * kBlock;
  const int nq = min(kBlock, T - t0);
  const int t = t0 + pp;
  const bool valid = pp < nq;

  // ---- dg (the head groups' terms in order), dS, the historical slots.
  // Thread t takes the (position, slot) items t + 256k: their dg terms,
  // blocks and gates are all loaded before the first is used (they do not
  // depend on the counts), then the blocks' pages, then LDS.
  constexpr int kItems = kBlock * kMaxSelP / 256;
  const int n_items = nq * S;
  const int64_t hg_stride = (int64_t)T * Hkv * S;
  float dgv[kItems], gv[kItems];
  int cv[kItems];
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int e = tid + 256 * k;
    if (e < n_items) {
      const int q = e / S, i = e - q * S;
      const int64_t u = ((int64_t)(t0 + q) * Hkv + kvh) * S + i;
      dgv[k] = p.ws_dgp[u];
      cv[k] = p.sel[u];
      gv[k] = p.gates[u];
    }
  }
  if (tid < kBlock) nh_l[tid] = tid < nq ? p.cnt[(int64_t)(t0 + tid) * Hkv + kvh] - 1 : 0;
  if (tid < kGateDim) wqn_l[tid] = p.w_qnorm[tid];
  __syncthreads();
  int pg[kItems];
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int e = tid + 256 * k;
    if (e < n_items) {
      const int q = e / S, i = e - q * S;
      const int64_t u = ((int64_t)(t0 + q) * Hkv + kvh) * S + i;
      for (int hg = 1; hg < p.head_groups; ++hg) dgv[k] += p.ws_dgp[hg * hg_stride + u];
      p.d_gates[u] = dgv[k];
      // a historical block precedes the position's own (trusted; clamped)
      cv[k] = (unsigned)cv[k] < (unsigned)tau ? cv[k] : 0;
      if (i < nh_l[q]) pg[k] = p.block_table[cv[k]];
    }
  }
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int e = tid + 256 * k;
    if (e < n_items) {
      const int q = e / S, i = e - q * S;
      if (i < nh_l[q]) {
        sel_l[q][i] = (int16_t)cv[k];
        page_l[q][i] = pg[k];
        ds_l[q][i] = dgv[k] * gv[k] * (1.f - gv[k]) * kInvSqrtDg;
      }
    }
  }

  // RoPE at the position for this thread's 16 pairs
  float cs[16], sn[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) rope_cos_sin((double)t, p.inv_freq[16 * o + e], cs[e], sn[e]);
  // w_qnorm of this thread's dim e (e < 16: 16o + e; else 64 + 16o + e - 16)
  auto wqn = [&](int e) { return wqn_l[e < 16 ? 16 * o + e : 64 + 16 * o + (e - 16)]; };

  // u = W_q[hq] q_t for the 64 positions into un[position][dim]
  auto project = [&](int hq) {
    u32x4 a[2][4], b[4][4];
    const uint16_t *wq = p.w_q + ((int64_t)hq * kGateDim + 32 * wave + (lane & 15)) * kHeadDim + 8 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[mt][ks] = ld16(wq + 16 * mt * kHeadDim + 32 * ks);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int pos = t0 + 16 * nt + (lane & 15);
      const bool ok = pos < T;
      const uint16_t *qr = p.q + ((int64_t)(ok ? pos : 0) * Hq + hq) * kHeadDim + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) b[nt][ks] = ok ? ld16(qr + 32 * ks) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(a[mt][ks]), to_bf16x8(b[nt][ks]), acc, 0, 0, 0);
        *reinterpret_cast<f32x4 *>(&un[16 * nt + (lane & 15)][32 * wave + 16 * mt + 4 * (lane >> 4)]) = acc;
      }
  };
  // this thread's 32 dims of un[pp]: x[e] = dim 16o + e, x[16 + e] = dim 64 + 16o + e
  auto read_un = [&](float (&x)[32]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 lo = *reinterpret_cast<const f32x4 *>(&un[pp][16 * o + 4 * k]);
      const f32x4 hi = *reinterpret_cast<const f32x4 *>(&un[pp][64 + 16 * o + 4 * k]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[4 * k + v] = lo[v];
        x[16 + 4 * k + v] = hi[v];
      }
    }
  };

  // ---- dghat = sum_i dS_i gk_{c_i} / sqrt(128) over the position's historical selection
  float dgh[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) dgh[e] = 0.f;
  {
    const int nh = valid ? nh_l[pp] : 0;
    const uint16_t *gk0 = p.gate_keys + (int64_t)kvh * kGateDim + 16 * o;
    const int64_t gk_page = (int64_t)Hkv * kGateDim;
    // four selections' keys loaded together (one round trip per four), then
    // added in slot order
    auto add_key = [&](const u32x4 (&w)[4], float dsv) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int e = 8 * (k & 1) + 2 * v + 16 * (k >> 1);
          dgh[e] = fmaf(dsv, bf16_lo(w[k][v]), dgh[e]);
          dgh[e + 1] = fmaf(dsv, bf16_hi(w[k][v]), dgh[e + 1]);
        }
    };
    int i = 0;
    for (; i + 4 <= nh; i += 4) {
      u32x4 w[4][4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint16_t *gk = gk0 + page_l[pp][i + b] * gk_page;
        w[b][0] = ld16(gk);
        w[b][1] = ld16(gk + 8);
        w[b][2] = ld16(gk + 64);
        w[b][3] = ld16(gk + 72);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) add_key(w[b], ds_l[pp][i + b]);
    }
    for (; i < nh; ++i) {
      const uint16_t *gk = gk0 + page_l[pp][i] * gk_page;
      const u32x4 w[4] = {ld16(gk), ld16(gk + 8), ld16(gk + 64), ld16(gk + 72)};
      add_key(w, ds_l[pp][i]);
    }
  }

  // ---- rows of A: columns [0, cols) of the tile's positions (every column a
  // dgk tile reads for these positions), dS / sqrt(128) where the position
  // selected the block, else 0.  512 columns at a time, through a map in LDS
  // (the projection buffer, free here) of each (position, column)'s slot.
  {
    const int cols = tau >= 1 ? min(p.a_cols, kBlock * ((tau - 1) / kBlock + 1)) : 0;
    constexpr int kMapCols = 512;
    static_assert(kBlock * kMapCols <= (int)sizeof(un), "slot map exceeds the projection buffer");
    int8_t *map = reinterpret_cast<int8_t *>(&un[0][0]);
    for (int c0 = 0; c0 < cols; c0 += kMapCols) {
      const int nc = min(kMapCols, cols - c0);
      __syncthreads();  // earlier reads of the buffer are done
      for (int e = tid; e < kBlock * kMapCols / 16; e += 256)
        reinterpret_cast<u32x4 *>(map)[e] = u32x4{~0u, ~0u, ~0u, ~0u};  // slot -1
      __syncthreads();
      for (int e = tid; e < kBlock * kMaxSelP; e += 256) {
        const int q = e / kMaxSelP, i = e - q * kMaxSelP;
        if (i < nh_l[q]) {
          const int c = sel_l[q][i] - c0;
          if ((unsigned)c < (unsigned)nc) map[q * kMapCols + c] = (int8_t)i;
        }
      }
      __syncthreads();
      // four columns per item (nc and the column offsets are multiples of 64)
      const int nc4 = nc >> 2;
      for (int e = tid; e < nq * nc4; e += 256) {
        const int q = e / nc4, c = 4 * (e - q * nc4);
        const uint32_t m4 = *reinterpret_cast<const uint32_t *>(map + q * kMapCols + c);
        f32x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = (int8_t)(m4 >> (8 * k));
          v[k] = i >= 0 ? ds_l[q][i] : 0.f;
        }
        *reinterpret_cast<f32x4 *>(p.ws_a + ((int64_t)kvh * T + t0 + q) * p.a_cols + c0 + c) = v;
      }
    }
  }

  // ---- one pass over the group's heads: u = W_q[h] q_t, its RMS r and
  // n = u / r; the gate query's terms (n * w_qnorm, rotated) summed in head
  // order into the group mean; and the query side of the backward:
  // d(n w) = RoPE^T(dghat / G), the same for every head of the group (it
  // depends on the selection's dS only), RMSNorm backward to du_q, and
  // dn * n summed over the heads in order
  float dn[32];
#pragma unroll
  for (int e = 0; e < 16; ++e) rope_back(dgh[e] / (float)G, dgh[16 + e] / (float)G, cs[e], sn[e], dn[e], dn[16 + e]);
  float gh[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) gh[e] = 0.f;
  for (int h = 0; h < G; ++h) {
    __syncthreads();  // the previous head's reads of un (and, at h = 0, of the selections) are done
    project(kvh * G + h);
    __syncthreads();
    float x[32], ss = 0.f;
    read_un(x);
#pragma unroll
    for (int e = 0; e < 32; ++e) ss += x[e] * x[e];
    const float r = sqrtf(quad_sum(ss) * (1.0f / kGateDim) + 1e-6f);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = x[e] / r;
      dot += dn[e] * wqn(e) * x[e];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float wa = x[e] * wqn(e), wb = x[16 + e] * wqn(16 + e);
      gh[e] += wa * cs[e] - wb * sn[e];
      gh[16 + e] += wb * cs[e] + wa * sn[e];
    }
    const float mean = quad_sum(dot) * (1.0f / kGateDim);
    float du[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) du[e] = (dn[e] * wqn(e) - x[e] * mean) / r;
    // this thread's own entries: no other thread touches them
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      f32x4 *ws = reinterpret_cast<f32x4 *>(&wsum_l[pp][(k < 4 ? 0 : 64) + 16 * o + 4 * (k & 3)]);
      const int e0 = (k < 4 ? 0 : 16) + 4 * (k & 3);
      const f32x4 term = {dn[e0] * x[e0], dn[e0 + 1] * x[e0 + 1], dn[e0 + 2] * x[e0 + 2], dn[e0 + 3] * x[e0 + 3]};
      *ws = h == 0 ? term : *ws + term;
    }
    if (valid) {
      float *dst = p.ws_du_q + ((int64_t)t * Hq + kvh * G + h) * kGateDim;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        *reinterpret_cast<f32x4 *>(dst + 16 * o + 4 * k) = f32x4{du[4 * k], du[4 * k + 1], du[4 * k + 2], du[4 * k + 3]};
        *reinterpret_cast<f32x4 *>(dst + 64 + 16 * o + 4 * k) =
            f32x4{du[16 + 4 * k], du[17 + 4 * k], du[18 + 4 * k], du[19 + 4 * k]};
      }
    }
  }
  if (valid) {
    float *dst = p.ws_ghat + ((int64_t)kvh * T + t) * kGateDim;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      *reinterpret_cast<f32x4 *>(dst + 16 * o + 4 * k) =
          f32x4{gh[4 * k], gh[4 * k + 1], gh[4 * k + 2], gh[4 * k + 3]} * (1.0f / G);
      *reinterpret_cast<f32x4 *>(dst + 64 + 16 * o + 4 * k) =
          f32x4{gh[16 + 4 * k], gh[17 + 4 * k], gh[18 + 4 * k], gh[19 + 4 * k]} * (1.0f / G);
    }
  }
  // ---- the query-norm weight terms summed over the 64 positions in order
  // (those of positions past the sequence end are zero: q = 0 there)
  __syncthreads();
  if (tid < kGateDim) {
    float a = 0.f;
    for (int q = 0; q < nq; ++q) a += wsum_l[q][tid];
    p.ws_dwqn[((int64_t)tau * Hkv + kvh) * kGateDim + tid] = a;
  }
}

// ---------------------------------------------------------------- long sums over positions: partial tiles
// blocks [0, Hq*kPrefillSplit): dW_q[h] (128 x 128) over one of
// kPrefillSplit ranges of positions, the sum of du_q (x) q (q is bf16: no
// low parts on that side); then Hkv*ceil(a_cols/128)*kPrefillSplit blocks:
// dgk tiles (128 blocks x 128 dims) of A^T ghat over one range of the
// positions that can select the tile's blocks.  A is taken as zero for a
// block at or after a position's own, which the position cannot select.
__global__ __launch_bounds__(256) void prefill_tiles_kernel(PrefillBackwardParams p) {
  __shared__ __attribute__((aligned(16))) OuterLds128 ls;
  const int k = blockIdx.x / kPrefillSplit, part = blockIdx.x % kPrefillSplit;
  const int Hq = p.n_q_heads, T = p.seq_len;
  f32x4 acc[4][4];
  auto range = [&](int n0, int n) {  // part's share of rows [n0, n)
    const int len = max(0, n - n0), per = (len + kPrefillSplit - 1) / kPrefillSplit;
    return make_int2(n0 + min(len, part * per), n0 + min(len, part * per + per));
  };
  if (k < Hq) {
    const int64_t rs = (int64_t)Hq * kHeadDim;
    const float *a = p.ws_du_q + (int64_t)k * kGateDim;
    const uint16_t *b = p.q + (int64_t)k * kHeadDim;
    const int2 r = range(0, T);
    outer_sum_tile128<true>([&](int n, int c) { return *reinterpret_cast<const f32x4 *>(a + n * rs + c); },
                            [&](int n, int c) {
                              const u32x2 v = *reinterpret_cast<const u32x2 *>(b + n * rs + c);
                              return f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
                            },
                            r.x, r.y, acc, ls);
  } else {
    const int k2 = k - Hq, kvh = k2 % p.n_kv_heads, c0 = 128 * (k2 / p.n_kv_heads);
    const float *a = p.ws_a + (int64_t)kvh * T * p.a_cols + c0;
    const float *b = p.ws_ghat + (int64_t)kvh * T * kGateDim;
    const int2 r = range(min(T, kBlock * (c0 + 1)), T);
    // columns c0 + c .. +3 lie in A's row whenever the first is a block the
    // position can select (a_cols is a multiple of 64)
    outer_sum_tile128<false>(
        [&](int n, int c) {
          const int own = n >> 6;
          f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
          if (c0 + c < own) {
            v = *reinterpret_cast<const f32x4 *>(a + (int64_t)n * p.a_cols + c);
#pragma unroll
            for (int k = 1; k < 4; ++k) v[k] = c0 + c + k < own ? v[k] : 0.f;
          }
          return v;
        },
        [&](int n, int c) { return *reinterpret_cast<const f32x4 *>(b + (int64_t)n * kGateDim + c); }, r.x, r.y, acc,
        ls);
  }
  store_tile128(acc, p.ws_part + ((int64_t)k * kPrefillSplit + part) * 128 * 128);
}

// the partial tiles added in order, a quarter tile (32 rows) per block:
// dW_q (Hq*4 blocks), dgk (Hkv*ceil(a_cols/128)*4 blocks, rows past a_cols
// dropped); then 32 blocks for the query-norm weight terms, block b summing
// dims 4b .. 4b+3 over the (64 positions, KV head) rows: thread t takes rows
// t, t+256, ..., then a fixed tree over the threads
__global__ __launch_bounds__(256) void prefill_sums_kernel(PrefillBackwardParams p) {
  __shared__ f32x4 red[256];
  const int Hq = p.n_q_heads;
  const int n_tiles = Hq + p.n_kv_heads * ((p.a_cols + 127) / 128);
  const int k = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  if (k < n_tiles) {
    const float *src = p.ws_part + (int64_t)k * kPrefillSplit * 128 * 128;
    float *dst;
    int rows = 128;
    if (k < Hq) {
      dst = p.d_w_q + (int64_t)k * kGateDim * kHeadDim;
    } else {
      const int k2 = k - Hq, kvh = k2 % p.n_kv_heads, c0 = 128 * (k2 / p.n_kv_heads);
      dst = p.ws_dgk + ((int64_t)kvh * p.a_cols + c0) * kGateDim;
      rows = min(128, p.a_cols - c0);
    }
    // thread t owns elements 4(t + 256q) .. +3 of the quarter's 32 x 128
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 32 * 128 * quarter + 4 * (threadIdx.x + 256 * q);
      if ((e >> 7) >= rows) continue;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int part = 0; part < kPrefillSplit; ++part) acc += *reinterpret_cast<const f32x4 *>(src + part * 128 * 128 + e);
      *reinterpret_cast<f32x4 *>(dst + e) = acc;
    }
  } else {
    const int b = blockIdx.x - 4 * n_tiles;
    const int rows = p.n_qblocks * p.n_kv_heads;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int u = threadIdx.x; u < rows; u += 256)
      sum += *reinterpret_cast<const f32x4 *>(p.ws_dwqn + (int64_t)u * kGateDim + 4 * b);
    red[threadIdx.x] = sum;
    __syncthreads();
    for (int half = 128; half > 0; half >>= 1) {
      if ((int)threadIdx.x < half) red[threadIdx.x] += red[threadIdx.x + half];
      __syncthreads();
    }
    if (threadIdx.x == 0) *reinterpret_cast<f32x4 *>(p.d_w_qnorm + 4 * b) = red[0];
  }
}

// ---------------------------------------------------------------- key side, 16 blocks per workgroup
// Thread (row = t/16, o = t%16) owns block c0 + row and dims o + 16k
// (k < 8), i.e. the RoPE pairs (o + 16k, o + 16k + 64), k < 4.
__global__ __launch_bounds__(256) void prefill_key_chain_kernel(PrefillBackwardParams p) {
  __shared__ __attribute__((aligned(16))) float pooled[kChainBlocks][kPoolPitch];
  __shared__ float uk[kChainBlocks][kUkPitch];
  __shared__ float rows16[kChainBlocks][kGateDim];
  const int tid = threadIdx.x;
  const int kvh = blockIdx.x % p.n_kv_heads, chunk = blockIdx.x / p.n_kv_heads;
  const int c0 = chunk * kChainBlocks, nb = min(kChainBlocks, p.n_hist - c0);
  u32x4 wk[2][12];
  load_wk_rows(p.w_k, kvh, wk);
  const float *pool = p.ws_pool + ((int64_t)kvh * p.n_hist + c0) * 3 * kHeadDim;
  for (int e4 = tid; e4 < kChainBlocks * 3 * kHeadDim / 4; e4 += 256) {
    const int b = e4 / (3 * kHeadDim / 4), c4 = e4 - b * (3 * kHeadDim / 4);
    *reinterpret_cast<f32x4 *>(&pooled[b][4 * c4]) =
        b < nb ? *reinterpret_cast<const f32x4 *>(pool + 4 * e4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  project_pooled<kChainBlocks>(wk, pooled, uk);
  __syncthreads();
  const int row = tid >> 4, o = tid & 15, c = c0 + row;
  float dw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) dw[k] = 0.f;
  if (row < nb) {
    float x[8], ss = 0.f, g[8];
    const float *dgk = p.ws_dgk + ((int64_t)kvh * p.a_cols + c) * kGateDim;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = uk[row][o + 16 * k];
      ss += x[k] * x[k];
      g[k] = dgk[o + 16 * k];
    }
    const float r = sqrtf(row16_sum(ss) * (1.0f / kGateDim) + 1e-6f);
    float dm[8], dot = 0.f, wkn[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float ck, sk;
      rope_cos_sin((double)c * kBlock, p.inv_freq[o + 16 * k], ck, sk);
      rope_back(g[k], g[k + 4], ck, sk, dm[k], dm[k + 4]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      wkn[k] = p.w_knorm[o + 16 * k];
      x[k] = x[k] / r;
      dot += dm[k] * wkn[k] * x[k];
    }
    const float mean = row16_sum(dot) * (1.0f / kGateDim);
    float *du = p.ws_du_k + ((int64_t)kvh * p.n_hist + c) * kGateDim;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      du[o + 16 * k] = (dm[k] * wkn[k] - x[k] * mean) / r;
      dw[k] = dm[k] * x[k];
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) rows16[row][o + 16 * k] = dw[k];
  __syncthreads();
  if (tid < kGateDim) {
    float a = 0.f;
#pragma unroll
    for (int b = 0; b < kChainBlocks; ++b) a += rows16[b][tid];
    p.ws_dwkn[((int64_t)kvh * p.key_chunks + chunk) * kGateDim + tid] = a;
  }
}

// blocks [0, Hkv*12): dW_k[kvh] tile (jt, it) = sum over the blocks c of
// du_k (x) pooled; the last block: dw_knorm over the (KV head, 16 blocks) rows
__global__ __launch_bounds__(256) void prefill_final_kernel(PrefillBackwardParams p) {
  __shared__ __attribute__((aligned(16))) OuterLds ls;
  const int k = blockIdx.x;
  if (k < p.n_kv_heads * 12) {
    const int kvh = k % p.n_kv_heads, tile = k / p.n_kv_heads, jt = tile / 6, it = tile % 6;
    const float *a = p.ws_du_k + (int64_t)kvh * p.n_hist * kGateDim + 64 * jt;
    const float *b = p.ws_pool + (int64_t)kvh * p.n_hist * 3 * kHeadDim + 64 * it;
    f32x4 acc[2][2];
    outer_sum_tile([&](int n, int c) { return a[(int64_t)n * kGateDim + c]; },
                   [&](int n, int c) { return b[(int64_t)n * 3 * kHeadDim + c]; }, 0, p.n_hist, acc, ls);
    store_tile(acc, p.d_w_k + ((int64_t)kvh * kGateDim + 64 * jt) * 3 * kHeadDim + 64 * it, 3 * kHeadDim);
  } else {
    float *slices = reinterpret_cast<float *>(&ls);  // [8][kGateDim]
    const int q = threadIdx.x & 31, sl = threadIdx.x >> 5;
    const int rows = p.n_kv_heads * p.key_chunks;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int u = sl; u < rows; u += 8) sum += *reinterpret_cast<const f32x4 *>(p.ws_dwkn + (int64_t)u * kGateDim + 4 * q);
    *reinterpret_cast<f32x4 *>(slices + sl * kGateDim + 4 * q) = sum;
    __syncthreads();
    if (threadIdx.x < kGateDim) {
      float a = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) a += slices[g * kGateDim + threadIdx.x];
      p.d_w_knorm[threadIdx.x] = a;
    }
  }
}

hipError_t launch_prefill_gate_backward(const PrefillBackwardParams &p, hipStream_t st) {
  hipError_t e = launch_prefill_grad(p, st);
  if (e != hipSuccess) return e;
  if (p.n_hist > 0) {
    hipLaunchKernelGGL(prefill_pool_stats_kernel, dim3((unsigned)(p.n_hist * p.n_kv_heads)), dim3(256), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(prefill_chain_kernel, dim3((unsigned)(p.n_qblocks * p.n_kv_heads)), dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int tiles = p.n_q_heads + p.n_kv_heads * ((p.a_cols + 127) / 128);
  hipLaunchKernelGGL(prefill_tiles_kernel, dim3((unsigned)(tiles * kPrefillSplit)), dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_sums_kernel, dim3((unsigned)(4 * tiles + kGateDim / 4)), dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.n_hist > 0) {
    hipLaunchKernelGGL(prefill_key_chain_kernel, dim3((unsigned)(p.key_chunks * p.n_kv_heads)), dim3(256), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(prefill_final_kernel, dim3((unsigned)(p.n_kv_heads * 12 + 1)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
