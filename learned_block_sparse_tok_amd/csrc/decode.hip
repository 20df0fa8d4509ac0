// Block-sparse flash-decode over the selected KV blocks.
//
// SAS decodes with attention restricted to the selected 64-token blocks,
// optionally scaling each selected block by its continuous gate
// ("Tencent released Simple-Attention-Sparsification ...", aigc.news: sparse
// decode budget, continuous gates on selected KV blocks; "Tencent Hunyuan
// open-sources SAS ...": block-sparse decoding).
//
// Split-K over the selection: each wave of a 256-thread workgroup owns a
// contiguous slice of one (sequence, KV head)'s selected blocks and keeps a
// running (max, sum, output) for the G query heads of the group; a second
// kernel merges the slices.  Per 64-token block a wave
//   - gathers K (16 KiB) straight into MFMA A-operand registers: lane l holds
//     token 16t + l%16, dims 32ks + 8(l/16) .. +7 (16-byte loads);
//   - gathers V (16 KiB) with fully coalesced 16-byte loads and parks it in a
//     per-wave LDS tile whose 16-byte chunks are XOR-swizzled by row;
//   - S^T (64 tokens x 16 heads, heads >= G zero) = K . Q^T with
//     v_mfma_f32_16x16x32_bf16 (4 token tiles x 4 k-steps);
//   - online softmax in the log2 domain; lane l holds head l%16, tokens
//     16t + 4(l/16) + r, so the probabilities are already laid out as the
//     B operand of the next product (the k index of P.V is that token order);
//   - O^T (128 dims x 16 heads) += V^T . P^T with V^T read by
//     ds_read_b64_tr_b16 (8 dim tiles x 2 k-steps).
// MFMA only serves the grouped-query tiles; the kernel is HBM-bound
// (32 KiB of K/V per selected block and KV head).
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {

constexpr int kWaves = 4;
constexpr int kVTileBytes = kBlock * kHeadDim * 2;  // 16 KiB

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);  // RNE
  return __builtin_bit_cast(uint32_t, b);
}

// Byte offset of (row, 16-byte chunk) in a swizzled 64 x 256-byte V tile.
__device__ __forceinline__ int vtile_off(int row, int chunk) {
  return row * 256 + ((chunk ^ ((row & 7) << 1)) << 4);
}

template <bool kGated>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t vlds[kWaves][kVTileBytes];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int unit = blockIdx.x / p.wg_per_unit;  // (sequence, KV head)
  const int wg = blockIdx.x - unit * p.wg_per_unit;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int G = p.group;
  const int W = p.wg_per_unit * kWaves;
  const int ws = wg * kWaves + wave;
  const int count = p.cnt[unit];
  const int i0 = ws * p.blocks_per_wave;
  const int i1 = min(count, i0 + p.blocks_per_wave);
  const int32_t L = p.seq_lens[s];

  // B operand of S^T = K Q^T: lane l holds q[head l%16][32ks + 8(l/16) .. +7]
  bf16x8 qB[4];
  {
    const uint16_t *qrow = p.q + ((int64_t)s * p.n_q_heads + kvh * G + j) * kHeadDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qB[ks] = as_bf16x8(j < G ? ld16(qrow + 32 * ks) : u32x4{0, 0, 0, 0});
  }

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff();  // running max, log2 domain
  float lsum = 0.f;             // this lane's share of the softmax denominator
  uint8_t *vt = vlds[wave];
  const int32_t *sel = p.sel + (int64_t)unit * p.max_sel;
  const int32_t *bt = p.block_table + (int64_t)s * p.max_blocks;

  // tr-read lane roles: within the 16-lane group g, lane 4e+q4 addresses
  // row 4g+e (+16 for the upper half of the k-step), columns 16dt+4q4 .. +3
  const int tr_e = (lane & 15) >> 2, tr_q = lane & 3;

  for (int i = i0; i < i1; ++i) {
    const int blk = sel[i];
    const int32_t page = bt[blk];
    const uint16_t *kb = p.k_pool + (int64_t)page * p.page_stride + (int64_t)kvh * p.head_stride;
    const uint16_t *vb = p.v_pool + (int64_t)page * p.page_stride + (int64_t)kvh * p.head_stride;
    const int nvalid = min(kBlock, L - blk * kBlock);

    u32x4 ka[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[t][ks] = ld16(kb + (int64_t)(16 * t + j) * p.tok_stride + 32 * ks + 8 * g);
    u32x4 vr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) vr[r] = ld16(vb + (int64_t)(4 * r + g) * p.tok_stride + 8 * j);

    f32x4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[t][ks]), qB[ks], sacc[t], 0, 0, 0);
    }

    float z[4][4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tau = 16 * t + 4 * g + r;
        z[t][r] = tau < nvalid ? sacc[t][r] * p.scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, z[t][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const bool live = m_new != -__builtin_inff();
    const float alpha = live ? exp2f(m - m_new) : 1.0f;
    const float gate = kGated ? p.gates[(int64_t)unit * p.max_sel + i] : 1.0f;
    float psum = 0.f;
    u32x4 pB[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 2 * s2 + (e >> 2), r = e & 3;
        float pe = live ? exp2f(z[t][r] - m_new) : 0.f;
        psum += pe;
        pv[e] = kGated ? pe * gate : pe;
      }
      pB[s2] = u32x4{pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]), pack2(pv[6], pv[7])};
    }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;

    // V -> LDS; rows past the cache end are zeroed
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 4 * r + g;
      *reinterpret_cast<u32x4 *>(vt + vtile_off(row, j)) = row < nvalid ? vr[r] : u32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int row0 = 32 * s2 + 4 * g + tr_e;
      const int row1 = row0 + 16;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int chunk = 2 * dt + (tr_q >> 1);
        const int sub = (tr_q & 1) * 8;
        i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(vt + vtile_off(row0, chunk) + sub));
        i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(vt + vtile_off(row1, chunk) + sub));
        u32x2 lo = __builtin_bit_cast(u32x2, a0), hi = __builtin_bit_cast(u32x2, a1);
        u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pB[s2]), o[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (j < G) {
    const int64_t slot = ((int64_t)unit * W + ws) * G + j;
    float *po = p.part_o + slot * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4 *>(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0) {
      p.part_ml[slot * 2] = m;
      p.part_ml[slot * 2 + 1] = lsum;
    }
  }
}

// Merge the W partial (max, sum, output) triples of each query head.
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams p) {
  const int unit = blockIdx.x;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int G = p.group;
  const int W = p.wg_per_unit * kWaves;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += blockDim.x) {
    const int j = idx >> 7, d = idx & (kHeadDim - 1);
    const int64_t base = (int64_t)unit * W * G + j;
    float M = -__builtin_inff();
    for (int w = 0; w < W; ++w) M = fmaxf(M, p.part_ml[(base + (int64_t)w * G) * 2]);
    float den = 0.f, num = 0.f;
    for (int w = 0; w < W; ++w) {
      const int64_t slot = base + (int64_t)w * G;
      const float mw = p.part_ml[slot * 2];
      const float f = mw == -__builtin_inff() ? 0.f : exp2f(mw - M);
      den = fmaf(f, p.part_ml[slot * 2 + 1], den);
      num = fmaf(f, p.part_o[slot * kHeadDim + d], num);
    }
    p.out[((int64_t)s * p.n_q_heads + kvh * G + j) * kHeadDim + d] = (uint16_t)f32_to_bf16(num / den);
  }
}

DecodeSplit decode_split(int batch, int n_kv_heads, int max_sel) {
  const int units = batch * n_kv_heads;
  const int target_waves = 2048;  // 8 waves per CU on 256 CUs
  int wg = target_waves / (kWaves * units);
  const int max_wg = (max_sel + kWaves - 1) / kWaves;
  wg = wg < 1 ? 1 : wg;
  wg = wg > max_wg ? max_wg : wg;
  wg = wg < 1 ? 1 : wg;
  const int waves = wg * kWaves;
  return DecodeSplit{wg, waves, (max_sel + waves - 1) / waves};
}

hipError_t launch_decode(const DecodeParams &p, int batch, hipStream_t st) {
  const unsigned units = (unsigned)(batch * p.n_kv_heads);
  if (p.gates)
    hipLaunchKernelGGL(decode_split_kernel<true>, dim3(units * p.wg_per_unit), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, dim3(units * p.wg_per_unit), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(units), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
