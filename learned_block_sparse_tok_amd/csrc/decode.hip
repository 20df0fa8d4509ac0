// Block-sparse flash-decode over the selected KV blocks.
//
// SAS decodes with attention restricted to the selected 64-token blocks,
// optionally scaling each selected block by its continuous gate
// ("Tencent released Simple-Attention-Sparsification ...", aigc.news: sparse
// decode budget, continuous gates on selected KV blocks; "Tencent Hunyuan
// open-sources SAS ...": block-sparse decoding).
//
// Split-K over the selection of each (sequence, KV head): every wave of a
// 512-thread workgroup owns a contiguous slice of the selected blocks and
// keeps a running (max, sum, output) for the G query heads of the group.  Per
// 64-token block a wave
//   - gathers K (16 KiB) straight into MFMA A-operand registers: lane l holds
//     token 16t + l%16, dims 32ks + 8(l/16) .. +7 (16-byte loads);
//   - gathers V (16 KiB) with fully coalesced 16-byte nontemporal loads (read
//     once per step, kept out of the caches) and parks it in a per-wave LDS
//     tile with a padded row pitch (conflict-free writes and reads);
//   - S^T (64 tokens x 16 heads, heads >= G zero) = K . Q^T with
//     v_mfma_f32_16x16x32_bf16 (4 token tiles x 4 k-steps);
//   - online softmax in the log2 domain; lane l holds head l%16, tokens
//     16t + 4(l/16) + r, which is already the B-operand layout of P.V once
//     the k index of that product is taken in this token order;
//   - O^T (128 dims x 16 heads) += V^T . P^T with V^T read by
//     ds_read_b64_tr_b16 (8 dim tiles x 2 k-steps).
// Each wave keeps the next block's 32 KiB in flight while it works on the
// current one: V(next) is issued as soon as V(current) sits in LDS, K(next)
// as soon as the QK product has consumed K(current); block-table and
// selection lookups are scalar loads.  The waves merge in LDS at the end and
// write the bf16
// output; when a (sequence, KV head) spans several workgroups (fewer units
// than CUs) each writes a partial and a small second kernel merges them.
// MFMA only serves the grouped-query tiles; the kernel is HBM-bound (32 KiB
// of K/V per selected block and KV head).
#include "attend.h"

namespace sas {

template <int kMode>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t vlds[kWaves][kVTileBytes];
  // the wave index is uniform: keep it (and everything derived) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x / p.wg_per_unit;  // (sequence, KV head)
  const int wg = blockIdx.x - unit * p.wg_per_unit;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int32_t *sel = p.sel + (int64_t)unit * p.max_sel;
  const float *gts = kMode ? p.gates + (int64_t)unit * p.max_sel : nullptr;
  const int32_t *bt = p.block_table + (int64_t)s * p.max_blocks;
  // scalar lookups, in bounds for any i (slots past cnt hold -1)
  auto source = [&](int i) {
    i = min(i, p.max_sel - 1);
    const int blk = max(sel[i], 0);
    return BlockRef{bt[blk], blk, kMode ? gts[i] : 1.0f};
  };
  BlockRegs b;
  attend_unit<kMode>(p, vlds, s, kvh, unit, wg, wave, (wg * kWaves + wave) * p.blocks_per_wave, p.cnt[unit],
                     p.seq_lens[s], source, b, false);
}

// Merge the wg_per_unit partials of each (sequence, KV head) into the bf16
// output (only launched when a unit spans several workgroups; the kernel
// boundary orders the partial writes before these reads).
// kW >= wg_per_unit: every partial's (max, sum, output) is loaded before any
// is used (unconditional loads, the slots past wg_per_unit clamped to the
// last one and ignored), so the merge costs one round trip to memory, not
// one per partial.
constexpr int kMaxWgPerUnit = 32;

template <int kW>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  const int unit = blockIdx.x;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int G = p.group;
  const int nwg = p.wg_per_unit;
  const int64_t ubase = (int64_t)unit * nwg * G;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int jj = idx >> 7, d = idx & (kHeadDim - 1);
    float mw[kW], lw[kW], ow[kW];
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const int64_t slot = ubase + (int64_t)min(w, nwg - 1) * G + jj;
      mw[w] = p.part_ml[slot * 2];
      lw[w] = p.part_ml[slot * 2 + 1];
      ow[w] = p.part_o[slot * kHeadDim + d];
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kW; ++w)
      if (w < nwg) M = fmaxf(M, mw[w]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      if (w >= nwg || mw[w] == -__builtin_inff()) continue;
      const float f = exp2f(mw[w] - M);
      den = fmaf(f, lw[w], den);
      num = fmaf(f, ow[w], num);
    }
    p.out[((int64_t)s * p.n_q_heads + kvh * G + jj) * kHeadDim + d] = (uint16_t)f32_to_bf16(num / den);
  }
}

DecodeSplit decode_split(int batch, int n_kv_heads, int max_sel, int cus) {
  // one 8-wave workgroup per CU; a (sequence, KV head) spans several
  // workgroups only when there are fewer units than CUs
  const int units = batch * n_kv_heads;
  int wg = cus / units;
  const int max_wg = (max_sel + kWaves - 1) / kWaves;  // >= 1 block per wave
  wg = wg > max_wg ? max_wg : wg;
  wg = wg > kMaxWgPerUnit ? kMaxWgPerUnit : wg;  // the merge kernel's largest instance
  wg = wg < 1 ? 1 : wg;
  const int waves = wg * kWaves;
  return DecodeSplit{wg, waves, (max_sel + waves - 1) / waves};
}

hipError_t launch_decode_merge(const DecodeParams &p, int batch, hipStream_t st) {
  const dim3 grid((unsigned)(batch * p.n_kv_heads));
  if (p.wg_per_unit <= 4) hipLaunchKernelGGL((decode_merge_kernel<4>), grid, dim3(256), 0, st, p);
  else if (p.wg_per_unit <= 8) hipLaunchKernelGGL((decode_merge_kernel<8>), grid, dim3(256), 0, st, p);
  else if (p.wg_per_unit <= 16) hipLaunchKernelGGL((decode_merge_kernel<16>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((decode_merge_kernel<32>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams &p, int batch, hipStream_t st) {
  const unsigned units = (unsigned)(batch * p.n_kv_heads);
  const dim3 grid(units * (unsigned)p.wg_per_unit);
  if (!p.gates)
    hipLaunchKernelGGL((decode_kernel<0>), grid, dim3(kWaves * 64), 0, st, p);
  else if (p.gate_mode == 0)
    hipLaunchKernelGGL((decode_kernel<1>), grid, dim3(kWaves * 64), 0, st, p);
  else
    hipLaunchKernelGGL((decode_kernel<2>), grid, dim3(kWaves * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.wg_per_unit == 1) return e;
  return launch_decode_merge(p, batch, st);
}

}  // namespace sas
