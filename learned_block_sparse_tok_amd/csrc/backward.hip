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
//   gate_grad_kernel  one 8-wave workgroup per (sequence, KV head), one pass
//     over the selection: per block S^T = K Q^T (as the decode kernel does)
//     and D^T = V dO^T (V as the A operand, dO as the B operand) on MFMA,
//     reduced to per-head sums relative to the block's own score maximum;
//     the softmax normaliser is applied once the selection's maximum and sum
//     are known.  K and V are read once: 32 KiB per selected block and KV
//     head.  The pooled statistics of the historical blocks (the inputs of
//     the gate-key projection) are taken from the K registers on the way.
//   gate_chain_kernel one 256-thread workgroup per (sequence, KV head): the
//     chain from dg to the per-sequence factors (du of every query head with
//     its RMSNorm weight term; du and RMSNorm weight term of every selected
//     historical block), recomputing the gate queries and the selected
//     blocks' pre-norm gate keys on MFMA.
//   gate_param_reduce_kernel + gate_dwk_sum_kernel  the weight gradients as
//     sums over the batch of outer products of those factors, as 64 x 64
//     output tiles on bf16 MFMA over high/low splits of the fp32 factors,
//     the factor rows staged in LDS; dW_k's
//     rows are split into ranges whose partial tiles are then added in order
//     (a fixed order throughout: deterministic).
#include <type_traits>

#include "backward_common.h"
#include "sas_kernels.h"

namespace sas {
namespace {

constexpr int kWavesG = 8;
// K and V bytes, each read once per launch: non-temporal loads keep them out
// of the caches (≈3 µs of the grad kernel's 61 at the Qwen3-8B shape)
__device__ __forceinline__ u32x4 ld16_once(const char *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// One butterfly step over n value pairs (v[c], v[c + n]): a lane keeps the
// half picked by its bit, takes the same half from its partner lane and
// combines the two.
template <int kCtrl, int n>
__device__ __forceinline__ void keep_half(bool bit, float (&mx)[2 * n], float (&mn)[2 * n], float (&sm)[2 * n]) {
#pragma unroll
  for (int c = 0; c < n; ++c) {
    const float kx = bit ? mx[c + n] : mx[c], sx = bit ? mx[c] : mx[c + n];
    const float kn = bit ? mn[c + n] : mn[c], sn = bit ? mn[c] : mn[c + n];
    const float ks = bit ? sm[c + n] : sm[c], ss = bit ? sm[c] : sm[c + n];
    mx[c] = fmaxf(kx, row_dpp<kCtrl>(sx));
    mn[c] = fminf(kn, row_dpp<kCtrl>(sn));
    sm[c] = ks + row_dpp<kCtrl>(ss);
  }
}

}  // namespace

// ---------------------------------------------------------------- dg per selected block
// One pass over the selection: per block and head, the block's own score
// maximum m_ih and a_ih = sum_j 2^(z_hj - m_ih) <dO_h, v_j> (z = score in
// log2 units) go to LDS, and each wave keeps an online max / sum per head.
// Once the waves' sums are combined into the selection's M_h and S_h,
//   dg_i = sum_h a_ih 2^(m_ih - M_h) / S_h.
__global__ __launch_bounds__(kWavesG * 64, 1) void gate_grad_kernel(BackwardParams p) {
  __shared__ float ml[kWavesG][2][kMaxGroup];
  __shared__ float fin[2][kMaxGroup];                    // per head: M_h, 1 / S_h
  __shared__ float bm[kMaxSelBackward][kMaxGroup];       // per block and head: m_ih
  __shared__ float ba[kMaxSelBackward][kMaxGroup];       // per block and head: a_ih
  __shared__ int32_t page_l[kMaxSelBackward], nvalid_l[kMaxSelBackward];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int unit = blockIdx.x;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int G = p.group;
  const int count = p.cnt[unit];
  const int32_t L = p.seq_lens[s];
  const int32_t *sel = p.sel + (int64_t)unit * p.max_sel;
  const int32_t *bt = p.block_table + (int64_t)s * p.max_blocks;
  for (int i = threadIdx.x; i < count; i += kWavesG * 64) {
    const int blk = sel[i];
    page_l[i] = bt[blk];
    nvalid_l[i] = min(kBlock, L - blk * kBlock);
  }

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
  const char *kpool = reinterpret_cast<const char *>(p.k_pool) + (int64_t)kvh * p.head_stride * 2;
  const char *vpool = reinterpret_cast<const char *>(p.v_pool) + (int64_t)kvh * p.head_stride * 2;
  // A-operand lane offset: token 16t + l%16, dims 32ks + 8(l/16)
  const int64_t lane_off = ((int64_t)j * p.tok_stride + 8 * g) * 2;
  const int64_t tile = 16 * p.tok_stride * 2;
  lds_barrier();

  // each wave keeps the next block's 32 KiB in flight while it works on the
  // current one: K(next) is issued once S^T has consumed K, V(next) once D^T
  // has consumed V
  u32x4 k[4][4], v[4][4];
  auto load_k = [&](int i) {
    const char *kb = kpool + (int64_t)page_l[i] * p.page_stride * 2 + lane_off;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) k[t][ks] = ld16_once(kb + t * tile + 64 * ks);
  };
  auto load_v = [&](int i) {
    const char *vb = vpool + (int64_t)page_l[i] * p.page_stride * 2 + lane_off;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) v[t][ks] = ld16_once(vb + t * tile + 64 * ks);
  };
  // The pooled statistics (max, min, mean over the 64 rows of every dim) of
  // a historical block, taken from the K registers for the key-side chain.
  // Lane (g, j) holds rows j, 16+j, 32+j, 48+j of dims 32ks + 8g + e; after
  // the in-lane reduction over its 4 rows, three butterfly steps over the
  // 16 lanes of its row split e (lane bits 2, 3, 1; the first step may pair
  // by a rotation since every lane still holds the same dims), and a fourth
  // splits ks (lane bit 0): lane j ends with ks = 2 b0 + {0, 1},
  // e = 4 b2 + 2 b3 + b1 reduced over all 64 rows.
  const bool b0 = j & 1, b1 = j & 2, b2 = j & 4, b3 = j & 8;
  auto pooled_stats = [&](int i) {
    float fx[4], fn[4], fs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float mx[8], mn[8], sm[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = (e & 1) ? bf16_hi(k[t][ks][e >> 1]) : bf16_lo(k[t][ks][e >> 1]);
        mx[e] = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mn[e] = fminf(fminf(x[0], x[1]), fminf(x[2], x[3]));
        sm[e] = (x[0] + x[1]) + (x[2] + x[3]);
      }
      keep_half<kRor4, 4>(b2, mx, mn, sm);
      float mx2[4] = {mx[0], mx[1], mx[2], mx[3]}, mn2[4] = {mn[0], mn[1], mn[2], mn[3]},
            sm2[4] = {sm[0], sm[1], sm[2], sm[3]};
      keep_half<kRor8, 2>(b3, mx2, mn2, sm2);
      float mx3[2] = {mx2[0], mx2[1]}, mn3[2] = {mn2[0], mn2[1]}, sm3[2] = {sm2[0], sm2[1]};
      keep_half<kXor2, 1>(b1, mx3, mn3, sm3);
      fx[ks] = mx3[0];
      fn[ks] = mn3[0];
      fs[ks] = sm3[0];
    }
    keep_half<kXor1, 2>(b0, fx, fn, fs);
    float *dst = p.ws_pool + ((int64_t)unit * p.max_sel + i) * 3 * kHeadDim;
    const int e = 4 * b2 + 2 * b3 + b1;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int dim = 32 * (2 * b0 + kk) + 8 * g + e;
      dst[dim] = fx[kk];
      dst[kHeadDim + dim] = fn[kk];
      dst[2 * kHeadDim + dim] = fs[kk] * (1.0f / kBlock);
    }
  };
  float m = -__builtin_inff(), lsum = 0.f;  // this wave's online max / sum of head (column) j
  // One block of the wave's share; kMore: a later block follows, whose loads
  // go out here.  Every block but the wave's last runs with kMore, so the
  // steady-state loop issues its loads unconditionally and the load counters
  // wait for exactly the block being consumed (a load issued on one branch
  // only makes the counter wait at the join cover the other branch too,
  // which held D^T until the next block's K had landed).
  auto block = [&](int i, auto more) {
    constexpr bool kMore = decltype(more)::value;
    const int nvalid = nvalid_l[i];
    // S^T = K Q^T and D^T = V dO^T: lane holds rows 16t + 4g + r of column j
    f32x4 sacc[4], dacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(k[t][ks]), qB[ks], sacc[t], 0, 0, 0);
    }
    // every block before the local one (the selection's last) is historical
    if (kMore || i < count - 1) pooled_stats(i);
    if (kMore) load_k(i + kWavesG);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) dacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(v[t][ks]), dB[ks], dacc[t], 0, 0, 0);
    }
    if (kMore) load_v(i + kWavesG);
    float z[4][4], mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[t][r] = 16 * t + 4 * g + r < nvalid ? sacc[t][r] * p.scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, z[t][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // the block's maximum for head j (row 0 is always valid)
    float es = 0.f, a = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(z[t][r] - mx);  // z - mx <= 0; 2^-inf = 0
        es += e;
        // rows past the sequence end: e = 0 and their V is not read into the sum
        a += 16 * t + 4 * g + r < nvalid ? e * dacc[t][r] : 0.f;
      }
    es += __shfl_xor(es, 16, 64);
    es += __shfl_xor(es, 32, 64);
    a += __shfl_xor(a, 16, 64);
    a += __shfl_xor(a, 32, 64);
    if (g == 0) {
      bm[i][j] = mx;
      ba[i][j] = a;
    }
    const float m_new = fmaxf(m, mx);
    lsum = (m == -__builtin_inff() ? 0.f : lsum * exp2f(m - m_new)) + es * exp2f(mx - m_new);
    m = m_new;
  };
  if (wave < count) {
    load_k(wave);
    load_v(wave);
    int i = wave;
    for (; i + kWavesG < count; i += kWavesG) block(i, std::true_type{});
    block(i, std::false_type{});
  }
  if (g == 0) {
    ml[wave][0][j] = m;
    ml[wave][1][j] = lsum;
  }
  lds_barrier();
  if (threadIdx.x < kMaxGroup) {
    const int h = threadIdx.x;
    float M = -__builtin_inff(), S = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesG; ++w) M = fmaxf(M, ml[w][0][h]);
#pragma unroll
    for (int w = 0; w < kWavesG; ++w)
      if (ml[w][0][h] != -__builtin_inff()) S += ml[w][1][h] * exp2f(ml[w][0][h] - M);
    fin[0][h] = M;
    fin[1][h] = h < G && S > 0.f ? 1.0f / S : 0.f;
  }
  lds_barrier();
  for (int i = threadIdx.x; i < p.max_sel; i += kWavesG * 64) {
    float acc = 0.f;
    if (i < count)
      for (int h = 0; h < G; ++h) acc += ba[i][h] * exp2f(bm[i][h] - fin[0][h]) * fin[1][h];
    p.d_gates[(int64_t)unit * p.max_sel + i] = acc;
  }
}

// ---------------------------------------------------------------- per-sequence chain
// The element-wise steps work on (row, dim slice) items: thread (row t / 16,
// o = t % 16) holds dims o + 16k, k = 0..7, i.e. the RoPE pairs
// (o + 16k, o + 16k + 64) for k = 0..3, and a sum over a row's 128 dims is a
// DPP sum over its 16 lanes.  Rows are query heads on the query side and
// selected blocks on the key side.  The two projections run on MFMA:
// u_h = W_q[h] q_h with q_h as the only non-zero column of the B operand,
// and U^T = W_k[kvh] P^T for 16 blocks' pooled statistics P at a time.  The
// max and min rows of P are bf16 values; the mean rows are split into bf16
// high and low parts (about 16 significant bits).

__global__ __launch_bounds__(256) void gate_chain_kernel(BackwardParams p) {
  __shared__ float un[kMaxGroup][kGateDim];    // u per head, then u / r
  __shared__ float part[kMaxGroup][kGateDim];  // per head: rotated weighted query, then the norm-weight term
  __shared__ float rr[kMaxGroup];              // r per head
  __shared__ float ghat[kGateDim], dghat[kGateDim];
  __shared__ float rows16[16][kGateDim];       // dghat partial sums per slot group, then dw_knorm per block row
  __shared__ __attribute__((aligned(16))) float pooled[kChainBlocks][kPoolPitch];
  __shared__ float uk[kChainBlocks][kUkPitch];
  __shared__ int32_t page_l[kMaxSelBackward], blk_l[kMaxSelBackward];  // per slot: page, block index
  __shared__ float ds_l[kMaxSelBackward];                               // per slot: dL/dscore = dg g (1 - g)
  __shared__ float wqn_l[kGateDim], wkn_l[kGateDim];
  __shared__ double invf_l[kGateDim / 2];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int row = t >> 4, o = t & 15;
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

  // W_q[h] A operands (row 16mt + l%16, inputs 32ks + 8(l/16) .. +7) and q_h
  // as column 0 of the B operand
  auto load_wq = [&](int h, u32x4 (&a)[8][4], bf16x8 (&qb)[4]) {
    const uint16_t *wq = p.w_q + ((int64_t)(kvh * G + h) * kGateDim + (lane & 15)) * kHeadDim + 8 * (lane >> 4);
    const uint16_t *qh = p.q + ((int64_t)s * p.n_q_heads + kvh * G + h) * kHeadDim + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = to_bf16x8((lane & 15) == 0 ? ld16(qh + 32 * ks) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[mt][ks] = ld16(wq + (int64_t)16 * mt * kHeadDim + 32 * ks);
  };

  // the historical slots' pages, block indices and score gradients (one slot
  // per thread: at most 255 historical slots), the norm weights and the RoPE
  // frequencies, gathered into LDS.  Every load is issued unconditionally
  // from clamped, valid addresses (a padding slot's -1 reads block 0's
  // page), so that none waits for the selection count, and the first head's
  // W_q loads go out right after the slots, ahead of the dependent
  // block-table gather: the W_q stream and the slot -> page chain overlap.
  const int ti = min(t, p.max_sel - 1);
  const int slot_blk = sel[ti];
  const float slot_g = gts[ti], slot_dg = dg[ti];
  u32x4 a[8][4];
  bf16x8 qb[4];
  load_wq(min(wave, G - 1), a, qb);
  const float wqn = p.w_qnorm[t & (kGateDim - 1)], wkn = p.w_knorm[t & (kGateDim - 1)];
  const double invf = p.inv_freq[t & (kGateDim / 2 - 1)];
  const int slot_page = bt[max(slot_blk, 0)];
  const bool has_slot = t < n_hist;
  if (has_slot) {
    blk_l[t] = slot_blk;
    page_l[t] = slot_page;
    ds_l[t] = slot_dg * slot_g * (1.f - slot_g);
  }
  if (t < kGateDim) {
    wqn_l[t] = wqn;
    wkn_l[t] = wkn;
  }
  if (t < kGateDim / 2) invf_l[t] = invf;

  // ---- u_h = W_q[h] q_h, one head per wave at a time
  for (int h = wave; h < G; h += 4) {
    if (h != wave) load_wq(h, a, qb);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(a[mt][ks]), qb[ks], acc, 0, 0, 0);
      if ((lane & 15) == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) un[h][16 * mt + 4 * (lane >> 4) + r] = acc[r];
    }
  }
  // W_k A operands of this wave's 32 rows (row 32w + 16mt + l%16, inputs
  // 32ks + 8(l/16) .. +7), kept in registers for every chunk
  u32x4 wk[2][12];
  load_wk_rows(p.w_k, kvh, wk);
  // the pooled statistics of the historical blocks, written by
  // gate_grad_kernel, kChainBlocks blocks at a time: 96 float4 per block,
  // thread t takes float4 t + 256k.  The first chunk is fetched here, each
  // next one while the current one is processed.
  const int64_t slot0 = (int64_t)unit * p.max_sel;
  constexpr int kQuads = kChainBlocks * 3 * kHeadDim / 4 / 256;
  f32x4 pv[kQuads];
  auto fetch_pooled = [&](int i0) {
    const int nb_ = max(0, min(kChainBlocks, n_hist - i0));
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.ws_pool + (slot0 + i0) * 3 * kHeadDim);
#pragma unroll
    for (int k = 0; k < kQuads; ++k)
      if (t + 256 * k < nb_ * 3 * kHeadDim / 4) pv[k] = src[t + 256 * k];
  };
  fetch_pooled(0);
  lds_barrier();
  // the gate keys of the first two historical slots of this thread's slot
  // group (dghat below), fetched ahead of the query side
  const uint16_t *gk = p.gate_keys + (int64_t)kvh * kGateDim + 8 * o;
  const int64_t gk_page = (int64_t)p.n_kv_heads * kGateDim;
  u32x4 gk_first[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (row + 16 * k < n_hist) gk_first[k] = ld16(gk + page_l[row + 16 * k] * gk_page);

  // ---- per head: RMS, normalise, weight, rotate; the mean over the group in head order
  float cq[4], sq[4];  // RoPE at the query's position for pairs o + 16k
#pragma unroll
  for (int k = 0; k < 4; ++k) rope_cos_sin((double)(L - 1), invf_l[o + 16 * k], cq[k], sq[k]);
  for (int h = row; h < G; h += 16) {
    float x[8], ss = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = un[h][o + 16 * k];
      ss += x[k] * x[k];
    }
    const float r = sqrtf(row16_sum(ss) * (1.0f / kGateDim) + 1e-6f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = x[k] / r;
      un[h][o + 16 * k] = x[k];
    }
    if (o == 0) rr[h] = r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = o + 16 * k;
      const float wa = x[k] * wqn_l[d], wb = x[k + 4] * wqn_l[d + 64];
      part[h][d] = wa * cq[k] - wb * sq[k];
      part[h][d + 64] = wb * cq[k] + wa * sq[k];
    }
  }
  lds_barrier();
  if (t < kGateDim) {
    float a = 0.f;
    for (int h = 0; h < G; ++h) a += part[h][t];
    ghat[t] = a / (float)G;
  }

  // ---- dghat = sum_i dS_i gk_i / sqrt(128) over the historical selection:
  // thread (slot group row, dims 8o .. 8o+7), then the 16 groups in order
  {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 2
    for (int i = row; i < n_hist; i += 16) {
      const u32x4 w = i < row + 32 ? gk_first[(i - row) >> 4] : ld16(gk + page_l[i] * gk_page);
      const float d = ds_l[i];
      acc[0] = fmaf(d, bf16_lo(w.x), acc[0]);
      acc[1] = fmaf(d, bf16_hi(w.x), acc[1]);
      acc[2] = fmaf(d, bf16_lo(w.y), acc[2]);
      acc[3] = fmaf(d, bf16_hi(w.y), acc[3]);
      acc[4] = fmaf(d, bf16_lo(w.z), acc[4]);
      acc[5] = fmaf(d, bf16_hi(w.z), acc[5]);
      acc[6] = fmaf(d, bf16_lo(w.w), acc[6]);
      acc[7] = fmaf(d, bf16_hi(w.w), acc[7]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) rows16[row][8 * o + e] = acc[e];
  }
  lds_barrier();
  if (t < kGateDim) {
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) a += rows16[g][t];
    dghat[t] = a * kInvSqrtDg;
  }
  lds_barrier();

  // ---- query side: per head d(n w) = RoPE^T(dghat / G), RMSNorm backward;
  // the norm-weight term dn * n summed over the heads in order
  for (int h = row; h < G; h += 16) {
    float dn[8], n[8], dot = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = o + 16 * k;
      rope_back(dghat[d] / (float)G, dghat[d + 64] / (float)G, cq[k], sq[k], dn[k], dn[k + 4]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      n[k] = un[h][o + 16 * k];
      dot += dn[k] * wqn_l[o + 16 * k] * n[k];
    }
    const float mean = row16_sum(dot) * (1.0f / kGateDim);
    const float r = rr[h];
    float *du = p.ws_du_q + ((int64_t)s * p.n_q_heads + kvh * G + h) * kGateDim;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = o + 16 * k;
      du[d] = (dn[k] * wqn_l[d] - n[k] * mean) / r;
      part[h][d] = dn[k] * n[k];
    }
  }
  lds_barrier();
  if (t < kGateDim) {
    float a = 0.f;
    for (int h = 0; h < G; ++h) a += part[h][t];
    p.ws_dwqn[(int64_t)unit * kGateDim + t] = a;
  }

  // ---- key side, kChainBlocks selected historical blocks at a time
  float dwk[8];  // dm * n of this thread's dims, summed over its block rows
#pragma unroll
  for (int k = 0; k < 8; ++k) dwk[k] = 0.f;
  for (int i0 = 0; i0 < p.max_sel; i0 += kChainBlocks) {
    const int nb_ = max(0, min(kChainBlocks, n_hist - i0));
    lds_barrier();
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
      const int e4 = t + 256 * k, b = e4 / (3 * kHeadDim / 4), c4 = e4 - b * (3 * kHeadDim / 4);
      if (e4 < nb_ * 3 * kHeadDim / 4) *reinterpret_cast<f32x4 *>(&pooled[b][4 * c4]) = pv[k];
    }
    lds_barrier();
    if (i0 + kChainBlocks < p.max_sel) fetch_pooled(i0 + kChainBlocks);
    // U^T = W_k P^T (columns of blocks not in the chunk hold stale values and are not read)
    project_pooled<kChainBlocks>(wk, pooled, uk);
    lds_barrier();
    // per block row: RMS, RoPE^T of dS ghat / sqrt(128), RMSNorm backward
    {
      const int b = row, i = i0 + b;
      if (i < p.max_sel) {
        float *du = p.ws_du_k + (slot0 + i) * kGateDim;
        if (b >= nb_) {  // local block or padding: no gradient, and zero pooled rows for the sums
          float *pk = p.ws_pool + (slot0 + i) * 3 * kHeadDim;
#pragma unroll
          for (int k = 0; k < 8; ++k) du[o + 16 * k] = 0.f;
#pragma unroll
          for (int k = 0; k < 24; ++k) pk[o + 16 * k] = 0.f;
        } else {
          float x[8], ss = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            x[k] = uk[b][o + 16 * k];
            ss += x[k] * x[k];
          }
          const float r = sqrtf(row16_sum(ss) * (1.0f / kGateDim) + 1e-6f);
          const float dS = ds_l[i] * kInvSqrtDg;
          const double pos = (double)blk_l[i] * kBlock;
          float dm[8], dot = 0.f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int d = o + 16 * k;
            float ck, sk;
            rope_cos_sin(pos, invf_l[d], ck, sk);
            rope_back(dS * ghat[d], dS * ghat[d + 64], ck, sk, dm[k], dm[k + 4]);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            x[k] = x[k] / r;
            dot += dm[k] * wkn_l[o + 16 * k] * x[k];
          }
          const float mean = row16_sum(dot) * (1.0f / kGateDim);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int d = o + 16 * k;
            du[d] = (dm[k] * wkn_l[d] - x[k] * mean) / r;
            dwk[k] += dm[k] * x[k];
          }
        }
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < 8; ++k) rows16[row][o + 16 * k] = dwk[k];
  lds_barrier();
  if (t < kGateDim) {
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) a += rows16[g][t];
    p.ws_dwkn[(int64_t)unit * kGateDim + t] = a;
  }
}

// ---------------------------------------------------------------- sums over the batch
// blocks [0, Hq*4): dW_q[h] tiles (2 x 2 per head), sums over the batch of
// du_q (x) q; then Hkv*12*kSplitK blocks: partial dW_k[kvh] tiles (2 x 6 per
// head, the (sequence, slot) rows split into kSplitK ranges), sums of
// du_k (x) pooled; the last two blocks: the query- and key-side norm-weight
// gradients as sums over the (sequence, KV head) rows.
__global__ __launch_bounds__(256) void gate_param_reduce_kernel(BackwardParams p) {
  __shared__ __attribute__((aligned(16))) OuterLds ls;
  const int tiles_q = p.n_q_heads * 4, tiles_k = p.n_kv_heads * 12;  // dW_k: 12 tiles of 64 x 64 per KV head
  const int bid = blockIdx.x;
  const int tid = threadIdx.x;
  f32x4 acc[2][2];
  if (bid < tiles_q) {
    const int h = bid >> 2, jt = (bid >> 1) & 1, it = bid & 1;
    const int64_t rs = (int64_t)p.n_q_heads * kHeadDim;  // row stride of du_q and q over the batch
    const float *a = p.ws_du_q + (int64_t)h * kGateDim + 64 * jt;
    const uint16_t *b = p.q + (int64_t)h * kHeadDim + 64 * it;
    outer_sum_tile([&](int n, int c) { return a[n * rs + c]; }, [&](int n, int c) { return bf16_to_f32(b[n * rs + c]); },
                   0, p.batch, acc, ls);
    store_tile(acc, p.d_w_q + ((int64_t)h * kGateDim + 64 * jt) * kHeadDim + 64 * it, kHeadDim);
  } else if (bid < tiles_q + tiles_k * kSplitK) {
    // one of kSplitK consecutive row ranges of one dW_k tile -> a partial
    // tile.  The KV head is the fastest-varying index, so that with
    // workgroups dealt round-robin to the 8 XCDs all blocks of one KV head
    // share an L2 (the one that also ran its units' chain, for 8 KV heads).
    const int kb = bid - tiles_q, kvh = kb % p.n_kv_heads, rest = kb / p.n_kv_heads;
    const int tile = rest / kSplitK, part = rest % kSplitK;
    const int k = kvh * 12 + tile, jt = tile / 6, it = tile % 6;
    const int n = p.batch * p.max_sel;
    const int per = (n + kSplitK - 1) / kSplitK;
    const int n_lo = min(n, part * per), n_hi = min(n, n_lo + per);
    auto slot = [&](int nn) { return ((int64_t)(nn / p.max_sel) * p.n_kv_heads + kvh) * p.max_sel + nn % p.max_sel; };
    outer_sum_tile([&](int nn, int c) { return p.ws_du_k[slot(nn) * kGateDim + 64 * jt + c]; },
                   [&](int nn, int c) { return p.ws_pool[slot(nn) * 3 * kHeadDim + 64 * it + c]; }, n_lo, n_hi, acc,
                   ls);
    store_tile(acc, p.ws_part + ((int64_t)k * kSplitK + part) * 64 * 64, 64);
  } else {
    // thread (dims 4q .. 4q+3, slice sl) sums rows u = sl, sl + 8, ...; the
    // eight slices are then added in order
    const bool key = bid > tiles_q + tiles_k * kSplitK;
    const float *src = key ? p.ws_dwkn : p.ws_dwqn;
    const int q = tid & 31, sl = tid >> 5;
    const int units = p.batch * p.n_kv_heads;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
    for (int u = sl; u < units; u += 8) sum += *reinterpret_cast<const f32x4 *>(src + (int64_t)u * kGateDim + 4 * q);
    float *slices = reinterpret_cast<float *>(&ls);  // [8][kGateDim] within the tile buffers
    *reinterpret_cast<f32x4 *>(slices + sl * kGateDim + 4 * q) = sum;
    lds_barrier();
    if (tid < kGateDim) {
      float a = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) a += slices[g * kGateDim + tid];
      (key ? p.d_w_knorm : p.d_w_qnorm)[tid] = a;
    }
  }
}

// dW_k from its partial tiles, summed in order of the row ranges: thread t
// owns elements 4(t + 256q) .. +3 of the tile
__global__ __launch_bounds__(256) void gate_dwk_sum_kernel(BackwardParams p) {
  const int kvh = blockIdx.x % p.n_kv_heads, tile = blockIdx.x / p.n_kv_heads;  // KV head fastest, as above
  const int k = kvh * 12 + tile, jt = tile / 6, it = tile % 6;
  sum_tile_parts(p.ws_part + (int64_t)k * kSplitK * 64 * 64, kSplitK, 64 * 64,
                 p.d_w_k + ((int64_t)kvh * kGateDim + 64 * jt) * 3 * kHeadDim + 64 * it, 3 * kHeadDim);
}

hipError_t launch_gate_backward(const BackwardParams &p, hipStream_t st) {
  const unsigned units = (unsigned)(p.batch * p.n_kv_heads);
  hipLaunchKernelGGL(gate_grad_kernel, dim3(units), dim3(kWavesG * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_chain_kernel, dim3(units), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)(p.n_q_heads * 4 + p.n_kv_heads * 12 * kSplitK + 2);
  hipLaunchKernelGGL(gate_param_reduce_kernel, dim3(tiles), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_dwk_sum_kernel, dim3((unsigned)(p.n_kv_heads * 12)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
