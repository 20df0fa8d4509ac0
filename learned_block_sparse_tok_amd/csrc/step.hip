// The whole SAS decode step of one (sequence, KV head) in one workgroup:
// gate query, block scores, per-KV-head Top-K, then the block-sparse
// flash-decode over the selection ("Tencent released Simple-Attention-
// Sparsification ...", aigc.news: learned block selection within the token
// budget, continuous gates on the selected KV blocks; "Tencent Hunyuan
// open-sources SAS ...": block-sparse decoding).
//
// The selection and the page of every selected block stay in LDS, so the
// attention's first K/V gathers are issued as soon as the Top-K is known:
// no kernel boundary, no second dispatch ramp and no dependent lookups of
// the selection and the block table in global memory.  The outputs (sel,
// gates, cnt, scores, out) are those of the gate kernel followed by the
// decode kernel, bit for bit: the selection runs the same arithmetic in the
// same order, and the attention is the decode kernel's own device code.
//
// One 512-thread workgroup (8 waves, one per CU at the decode kernel's
// register budget) per (sequence, KV head), or, with fewer pairs than CUs,
// several per pair (each makes the pair's selection, then attends its share
// of the blocks and stores a partial result that the decode merge kernel
// combines):
//   1. loads: the group's queries, RoPE frequencies and norm weights, the
//      block-table row (to LDS), and one batch of 16 query-projection rows
//      per 16-lane group (32 groups; w_q stays in L2);
//   2. all 512 first candidates' gate keys are gathered at once (16 per lane
//      group), the projection runs while they arrive (transposing row sums),
//      then RMSNorm, RoPE and the group mean as in the gate kernel;
//   3. scores (one row sum per key, finished by lane 0 of its group, so that
//      equal keys get equal scores) become order-preserving keys in LDS;
//   4. wave 0 selects (radix select, ascending order, lowest index at the
//      threshold) straight into LDS arrays of the selection, pages and
//      gates; the last wave stores the selection outputs from there;
//   5. the 8 waves attend the selection exactly as the decode kernel does
//      (its V tiles reuse the LDS the gate phase held).
#include "attend.h"
#include "select.h"
#include "step_layout.h"

namespace sas {

// blockIdx -> (pair, workgroup of the pair).  One workgroup per pair: the
// pair is the block index.  Several: when the pair count is a multiple of 8,
// the workgroups of one pair are placed on one XCD (workgroups are dealt to
// the 8 XCDs round-robin), so that their repeated selections read the pair's
// block-table row and gate keys through one L2; else consecutive.
namespace {
__device__ __forceinline__ void split_unit(int nwg, int &unit, int &wg) {
  const int b = (int)blockIdx.x;
  const int units = (int)gridDim.x / nwg;
  if (nwg > 1 && (units & 7) == 0) {
    const int x = b & 7, k = b >> 3;
    unit = x + 8 * (k / nwg);
    wg = k - (k / nwg) * nwg;
  } else {
    unit = nwg == 1 ? b : b / nwg;
    wg = b - unit * nwg;
  }
}
}  // namespace

constexpr int kStepKeys = step_layout::kKeysPerGroup;  // gate keys per 16-lane group per pass (512 per workgroup)
constexpr int kStepMaxSel = 256;      // selection slots per (sequence, KV head)
constexpr int kStepBtUnroll = 2;      // block-table entries per thread staged without a loop
// the gate phase's arrays inside the V tiles: score keys, block-table row,
// gate queries (step_layout.h, checked on the host for every width)
constexpr int kStepKeysOff = step_layout::kKeysOff;
constexpr int kStepBtOff = step_layout::kBtOff;
constexpr int kStepVsOff = step_layout::kVsOff;
static_assert(step_layout::kMaxBlocks == SAS_MAX_BLOCKS_DEV && step_layout::kMaxGroup == kMaxGroup &&
                  step_layout::kGateDim == kGateDim && step_layout::kVTilesBytes == kWaves * kVTileBytes,
              "step layout constants disagree with the kernels'");
static_assert(step_layout::kGroups * 16 == kWaves * 64, "one 16-lane group per 16 threads");
static_assert(3 * 4 * kMaxSlices * kStepMaxSel <= kWaves * kVTileBytes, "slice lists exceed the V tiles");
static_assert(3 * 4 * 512 <= kWaves * kVTileBytes, "padded slice lists exceed the V tiles");

// seq_lens, block_table, n_kv_heads and max_blocks also come as leading
// scalar arguments (copies of sp.g's): the first loads need only these, and
// they arrive in the first kernel-argument fetch.
template <bool kMax, int kMode>
__global__ __launch_bounds__(kWaves * 64, 1) void step_kernel(const int32_t *__restrict__ seq_lens_a,
                                                              const int32_t *__restrict__ block_table_a,
                                                              int32_t n_kv_heads_a, int32_t max_blocks_a,
                                                              StepParams sp) {
  __shared__ __attribute__((aligned(16))) uint8_t vlds[kWaves][kVTileBytes];
  __shared__ float qs[kMaxGroup][kHeadDim];
  __shared__ float part[4][kGateDim];
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  __shared__ int32_t sel_l[kStepMaxSel], page_l[kStepMaxSel];
  __shared__ float gate_l[kStepMaxSel];
  uint8_t *const gate_lds = &vlds[0][0];
  uint32_t *keys = reinterpret_cast<uint32_t *>(gate_lds + kStepKeysOff);  // [max(max_blocks, 512)]
  int32_t *btl = reinterpret_cast<int32_t *>(gate_lds + kStepBtOff);      // [max_blocks]
  float(*vs)[kGateDim] = reinterpret_cast<float(*)[kGateDim]>(gate_lds + kStepVsOff);

  const GateParams &p = sp.g;
  // (sequence, KV head) and its share: with fewer pairs than CUs each pair
  // spans wg_per_unit workgroups, each making the pair's selection and
  // attending its share of the blocks as the decode kernel splits them
  const int nwg = sp.d.wg_per_unit;
  int unit, wg;
  split_unit(nwg, unit, wg);  // KV head = unit % Hkv
  const int s = unit / n_kv_heads_a;
  const int kvh = unit - s * n_kv_heads_a;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane16 = t & 15, grp = t >> 4;  // 32 groups of 16 lanes
  const int G = p.group;
  const int32_t L = seq_lens_a[s];
  const int n = (L - 1) / kBlock;  // candidates: the blocks before the local block
  const int k_eff = min(p.n_sel - 1, n);

  // ---- 1. loads (nothing waits before all are issued)
  const uint16_t *qg = p.q + ((int64_t)s * p.n_q_heads + kvh * G) * kHeadDim;
  const bool has_q = 8 * t < G * kHeadDim;
  const u32x4 qpiece = ld16(qg + (has_q ? 8 * t : 0));
  const double inv_freq = p.inv_freq[lane];
  const float wqn_a = p.w_qnorm[lane], wqn_b = p.w_qnorm[lane + 64];
  const int32_t *bt = block_table_a + (int64_t)s * max_blocks_a;
  int32_t btv[kStepBtUnroll];
#pragma unroll
  for (int k = 0; k < kStepBtUnroll; ++k) btv[k] = bt[min(t + 512 * k, max_blocks_a - 1)];
  // projection batch b: rows 16b .. 16b+15 of the group's heads (head b/8);
  // lane group grp takes batches grp, grp + 32, ...  (one batch for G <= 4)
  const int n_batches = 8 * G;
  const uint16_t *wq_lane = p.w_q + ((int64_t)kvh * G * kGateDim) * kHeadDim + 8 * lane16;
  u32x4 wv[16];
  auto load_batch = [&](int b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[r] = ld16(wq_lane + (int64_t)min(16 * b + r, G * kGateDim - 1) * kHeadDim);
  };
  load_batch(grp);

  if (has_q) {
    float *qd = &qs[0][0] + 8 * t;
    qd[0] = bf16_lo(qpiece.x); qd[1] = bf16_hi(qpiece.x); qd[2] = bf16_lo(qpiece.y); qd[3] = bf16_hi(qpiece.y);
    qd[4] = bf16_lo(qpiece.z); qd[5] = bf16_hi(qpiece.z); qd[6] = bf16_lo(qpiece.w); qd[7] = bf16_hi(qpiece.w);
  }
#pragma unroll
  for (int k = 0; k < kStepBtUnroll; ++k)
    if (t + 512 * k < p.max_blocks) btl[t + 512 * k] = btv[k];
  for (int c = t + 512 * kStepBtUnroll; c < p.max_blocks; c += 512) btl[c] = bt[c];
  lds_barrier();

  // ---- 2. the first 512 candidates' gate keys, then the projection
  const uint16_t *gkh = p.gate_keys + (int64_t)kvh * kGateDim + 8 * lane16;
  const int64_t page_stride = (int64_t)p.n_kv_heads * kGateDim;
  // unconditional loads (no branch per key, so the load counters stay exact):
  // a slot past the candidates reads the local block's key (page btl[n],
  // which the scores never overwrite: they live in their own array)
  u32x4 v[kStepKeys];
  auto gather = [&](int base) {
#pragma unroll
    for (int u = 0; u < kStepKeys; ++u)
      v[u] = __builtin_nontemporal_load(  // read once: kept out of the caches
          reinterpret_cast<const u32x4 *>(gkh + (int64_t)btl[step_layout::gather_slot(base, u, grp, n)] * page_stride));
  };
  gather(0);
  auto project = [&](int b) {  // lane o of the group ends with row o of batch b
    const int h = min(b >> 3, G - 1);
    const float *qq = qs[h] + 8 * lane16;
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qq[e];
    float pp[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const u32x4 &w = wv[r];
      float acc = qv[0] * bf16_lo(w.x);
      acc = fmaf(qv[1], bf16_hi(w.x), acc);
      acc = fmaf(qv[2], bf16_lo(w.y), acc);
      acc = fmaf(qv[3], bf16_hi(w.y), acc);
      acc = fmaf(qv[4], bf16_lo(w.z), acc);
      acc = fmaf(qv[5], bf16_hi(w.z), acc);
      acc = fmaf(qv[6], bf16_lo(w.w), acc);
      acc = fmaf(qv[7], bf16_hi(w.w), acc);
      pp[row16_slot(r)] = acc;
    }
    const float tot = row16_transpose_sum(pp);
    if (b < n_batches) vs[b >> 3][16 * (b & 7) + lane16] = tot;
  };
  project(grp);
  // G > 4 only; n_batches is a multiple of 8, so a wave's 4 groups agree
  for (int b = grp + 32; b < n_batches; b += 32) {
    load_batch(b);
    project(b);
  }
  lds_barrier();
  if (wave < 4) {  // RMSNorm + RoPE per head (wave w: heads w, w+4, ...; lane i: pair (i, i+64))
    float cf, sf;
    rope_cos_sin((double)(L - 1), inv_freq, cf, sf);
    float sa = 0.f, sb = 0.f;
    for (int g = wave; g < G; g += 4) {
      const float a = vs[g][lane], b = vs[g][lane + 64];
      const float inv = 1.0f / sqrtf(wave_sum(a * a + b * b) * (1.0f / kGateDim) + 1e-6f);
      const float na = a * inv * wqn_a, nb = b * inv * wqn_b;
      const float ra = na * cf - nb * sf, rb = nb * cf + na * sf;
      sa += ra;
      sb += rb;
      if (kMax) {
        vs[g][lane] = ra;
        vs[g][lane + 64] = rb;
      }
    }
    part[wave][lane] = sa;
    part[wave][lane + 64] = sb;
  }
  lds_barrier();
  float gm[8];  // mean gate query of the group, dims 8*lane16 .. +7
  {
    const float inv_g = 1.0f / (float)G;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lane16 + e;
      gm[e] = (part[0][d] + part[1][d] + part[2][d] + part[3][d]) * inv_g;
    }
  }
  float gh[kMax ? 8 : 1][8];  // kMax: per-head gate queries
  if (kMax) {
#pragma unroll
    for (int h = 0; h < (kMax ? 8 : 1); ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) gh[h][e] = h < G ? vs[h][8 * lane16 + e] : 0.f;
  }

  // ---- 3. scores
  const float inv_sqrt_dg = 0.08838834764831845f;  // 1/sqrt(128)
  float *scores = p.scores && wg == 0 ? p.scores + (int64_t)unit * p.max_blocks : nullptr;
  for (int base = 0; base < n; base += 32 * kStepKeys) {
    if (base > 0) gather(base);
#pragma unroll
    for (int u = 0; u < kStepKeys; ++u) {
      auto dot8 = [&](const float(&w)[8]) {
        float d = w[0] * bf16_lo(v[u].x);
        d = fmaf(w[1], bf16_hi(v[u].x), d);
        d = fmaf(w[2], bf16_lo(v[u].y), d);
        d = fmaf(w[3], bf16_hi(v[u].y), d);
        d = fmaf(w[4], bf16_lo(v[u].z), d);
        d = fmaf(w[5], bf16_hi(v[u].z), d);
        d = fmaf(w[6], bf16_lo(v[u].w), d);
        d = fmaf(w[7], bf16_hi(v[u].w), d);
        return row16_sum(d);
      };
      float d;
      if (kMax) {
        d = -__builtin_inff();
#pragma unroll
        for (int h = 0; h < (kMax ? 8 : 1); ++h)
          if (h < G) d = fmaxf(d, dot8(gh[h]));
      } else {
        d = dot8(gm);
      }
      const int c = base + 32 * u + grp;
      if (lane16 == 0 && c < n) {
        const float sc = d * inv_sqrt_dg;
        keys[c] = score_key(sc);
        if (scores) scores[c] = sc;
      }
    }
  }
  if (scores)
    for (int c = n + t; c < p.max_blocks; c += 512) scores[c] = -__builtin_inff();
  lds_barrier();

  // the local block is selected whatever the scores: the wave whose share of
  // the selection ends with it (and takes it first) issues its K/V loads now,
  // so that they arrive while wave 0 selects
  const int bpw = sp.d.blocks_per_wave;
  const int gwave = wg * kWaves + wave;  // this wave's share among the pair's waves
  const bool prefetch = gwave == k_eff / bpw;
  BlockRegs b;
  if (prefetch) issue_block(b, block_rows(sp.d, kvh, BlockRef{btl[n], n, 1.0f}, L), lane_offsets(sp.d));

  // ---- 4. wave 0 selects straight into the LDS selection, pages and gates
  if (wave == 0) {
    wave_select_emit(keys, n, k_eff, hist, [&](uint32_t pos, int c, uint32_t key) {
      sel_l[pos] = c;
      gate_l[pos] = __uint_as_float(key);  // the score key for now
    });
    // pages and gates one slot per lane, off the emit's serial path
    for (int i = lane; i < k_eff; i += 64) {
      page_l[i] = btl[sel_l[i]];
      gate_l[i] = 1.0f / (1.0f + __expf(-key_score(__float_as_uint(gate_l[i]))));
    }
    if (lane == 0) {  // the local block closes the selection
      sel_l[k_eff] = n;
      page_l[k_eff] = btl[n];
      gate_l[k_eff] = 1.0f;
    }
  }
  lds_barrier();
  if (wg == 0 && wave == kWaves - 1) {  // the selection's outputs, from the LDS arrays (the V tiles overwrite the keys)
    int32_t *sel = p.sel + (int64_t)unit * p.n_sel;
    float *gates = p.gates ? p.gates + (int64_t)unit * p.n_sel : nullptr;
    for (int i = lane; i < p.n_sel; i += 64) {
      const bool in = i <= k_eff;
      sel[i] = in ? sel_l[i] : -1;
      if (gates) gates[i] = in ? gate_l[i] : 0.0f;
    }
    if (lane == 0) p.cnt[unit] = k_eff + 1;
  }

  // ---- 5. attention over the selection (the V tiles now overwrite the gate phase's LDS)
  auto source = [&](int i) {
    i = min(i, kStepMaxSel - 1);
    return BlockRef{__builtin_amdgcn_readfirstlane(page_l[i]), __builtin_amdgcn_readfirstlane(sel_l[i]),
                    kMode ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gate_l[i]))) : 1.0f};
  };
  attend_unit<kMode>(sp.d, vlds, s, kvh, unit, wg, wave, gwave * bpw, k_eff + 1, L, source, b, prefetch);
}

// The second half of the sliced step (fewer pairs than CUs): the slices'
// Top-K lists of one pair (launch_gate_slices) are merged into the pair's
// selection by the same radix select, with the slice lists concatenated in
// ascending block order so that the lowest-index rule at the threshold is
// unchanged; then the attention, each pair split over wg_per_unit
// workgroups as in the decode kernel (partials merged by the decode merge
// kernel).  Every workgroup of a pair makes the same selection; the first
// stores it.
template <int kMode>
__global__ __launch_bounds__(kWaves * 64, 1) void select_decode_kernel(StepParams sp) {
  __shared__ __attribute__((aligned(16))) uint8_t vlds[kWaves][kVTileBytes];
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  __shared__ int32_t sel_l[kStepMaxSel], page_l[kStepMaxSel];
  __shared__ float gate_l[kStepMaxSel];
  __shared__ int32_t local_page;
  const GateParams &p = sp.g;
  const int nwg = sp.d.wg_per_unit;
  int unit, wg;
  split_unit(nwg, unit, wg);
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int32_t L = p.seq_lens[s];
  const int n = (L - 1) / kBlock;
  const int k_eff = min(p.n_sel - 1, n);
  // the pair's candidate lists (slices x n_sel entries) in the V tiles' space
  const int m = p.slices * p.n_sel;
  const int m_pad = max(m, 512);
  uint32_t *keys = reinterpret_cast<uint32_t *>(&vlds[0][0]);
  int32_t *cblk = reinterpret_cast<int32_t *>(keys + m_pad);
  int32_t *cpage = cblk + m_pad;
  const int64_t base = (int64_t)unit * m;
  for (int i = t; i < m_pad; i += kWaves * 64) {
    const bool in = i < m;
    keys[i] = in ? p.cand_key[base + i] : 0u;
    cblk[i] = in ? p.cand_blk[base + i] : 0;
    cpage[i] = in ? p.cand_page[base + i] : 0;
  }
  if (t == 0) local_page = p.block_table[(int64_t)s * p.max_blocks + n];
  __syncthreads();
  if (wave == 0) {
    wave_select_emit(keys, m, k_eff, hist, [&](uint32_t pos, int c, uint32_t key) {
      sel_l[pos] = cblk[c];
      page_l[pos] = cpage[c];
      gate_l[pos] = 1.0f / (1.0f + __expf(-key_score(key)));
    });
    if (lane == 0) {
      sel_l[k_eff] = n;
      page_l[k_eff] = local_page;
      gate_l[k_eff] = 1.0f;
    }
  }
  lds_barrier();
  if (wg == 0 && wave == kWaves - 1) {
    int32_t *sel = p.sel + (int64_t)unit * p.n_sel;
    float *gates = p.gates ? p.gates + (int64_t)unit * p.n_sel : nullptr;
    for (int i = lane; i < p.n_sel; i += 64) {
      const bool in = i <= k_eff;
      sel[i] = in ? sel_l[i] : -1;
      if (gates) gates[i] = in ? gate_l[i] : 0.0f;
    }
    if (lane == 0) p.cnt[unit] = k_eff + 1;
  }
  auto source = [&](int i) {
    i = min(i, kStepMaxSel - 1);
    return BlockRef{__builtin_amdgcn_readfirstlane(page_l[i]), __builtin_amdgcn_readfirstlane(sel_l[i]),
                    kMode ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gate_l[i]))) : 1.0f};
  };
  BlockRegs b;
  attend_unit<kMode>(sp.d, vlds, s, kvh, unit, wg, wave, (wg * kWaves + wave) * sp.d.blocks_per_wave, k_eff + 1, L,
                     source, b, false);
}

hipError_t launch_select_decode(const StepParams &p, int batch, hipStream_t st) {
  const unsigned units = (unsigned)(batch * p.g.n_kv_heads);
  const dim3 grid(units * (unsigned)p.d.wg_per_unit);
  const int mode = !p.d.gates ? 0 : (p.d.gate_mode == 0 ? 1 : 2);
  if (mode == 0) hipLaunchKernelGGL((select_decode_kernel<0>), grid, dim3(kWaves * 64), 0, st, p);
  else if (mode == 1) hipLaunchKernelGGL((select_decode_kernel<1>), grid, dim3(kWaves * 64), 0, st, p);
  else hipLaunchKernelGGL((select_decode_kernel<2>), grid, dim3(kWaves * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.d.wg_per_unit == 1) return e;
  return launch_decode_merge(p.d, batch, st);
}

bool step_fits(int group, int max_blocks, int n_sel) {
  return group <= kMaxGroup && max_blocks <= SAS_MAX_BLOCKS_DEV && n_sel <= kStepMaxSel;
}

hipError_t launch_step(const StepParams &p, int batch, hipStream_t st) {
  const dim3 grid((unsigned)(batch * p.g.n_kv_heads * p.d.wg_per_unit));
  const bool mx = p.g.aggregate != 0;
  const int mode = !p.d.gates ? 0 : (p.d.gate_mode == 0 ? 1 : 2);
  const int32_t *sl = p.g.seq_lens, *btab = p.g.block_table;  // the leading arguments
  const int32_t hkv = p.g.n_kv_heads, mb = p.g.max_blocks;
  if (!mx) {
    if (mode == 0) hipLaunchKernelGGL((step_kernel<false, 0>), grid, dim3(kWaves * 64), 0, st, sl, btab, hkv, mb, p);
    else if (mode == 1) hipLaunchKernelGGL((step_kernel<false, 1>), grid, dim3(kWaves * 64), 0, st, sl, btab, hkv, mb, p);
    else hipLaunchKernelGGL((step_kernel<false, 2>), grid, dim3(kWaves * 64), 0, st, sl, btab, hkv, mb, p);
  } else {
    if (mode == 0) hipLaunchKernelGGL((step_kernel<true, 0>), grid, dim3(kWaves * 64), 0, st, sl, btab, hkv, mb, p);
    else if (mode == 1) hipLaunchKernelGGL((step_kernel<true, 1>), grid, dim3(kWaves * 64), 0, st, sl, btab, hkv, mb, p);
    else hipLaunchKernelGGL((step_kernel<true, 2>), grid, dim3(kWaves * 64), 0, st, sl, btab, hkv, mb, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.d.wg_per_unit == 1) return e;
  return launch_decode_merge(p.d, batch, st);
}

}  // namespace sas
