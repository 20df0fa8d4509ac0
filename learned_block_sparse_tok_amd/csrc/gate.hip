// Gate query, block scores and per-KV-head Top-K, fused in one kernel.
//
// SAS scores the KV blocks for each decode query through a query projection
// (Qproj) with Q/K normalisation and gate RoPE, and keeps a Top-K of 31
// historical blocks plus the local block for the default 2,048-token budget
// (1,024 / 4,096 also) ("Tencent released Simple-Attention-Sparsification
// ...", aigc.news, setup paragraph; localmodelwatch "Specifications and
// Configuration Table").  Each selected block gets a continuous gate.
//
// One 256-thread workgroup per (sequence, KV head):
//   1. the block-table row is staged in LDS while the group's queries and
//      query-projection rows arrive (w_q rows from L2, 16 lanes x 16 B per
//      row, so every load instruction reads whole rows);
//   2. gate queries: q . w_q[h]^T per head, RMSNorm, RoPE at position L-1
//      (angles formed and reduced in fp64 from host-computed frequencies),
//      averaged over the group (the KV head's score is the mean of its query
//      heads' scores);
//   3. every candidate's gate key is gathered (16 lanes x 16 B per key, up to
//      512 keys in flight) and dotted with the mean gate query (DPP row
//      reduction); scores become order-preserving uint32 keys in the LDS
//      slots the block table occupied;
//   4. one wave selects: an 8-bit radix select (wave-private histogram, DPP
//      prefix sums, no workgroup barriers) finds the threshold key, usually
//      in two or three passes; a second sweep writes the selection in
//      ascending block order, ties at the threshold going to the lowest
//      block indices.
// Bytes per (sequence, KV head): 256 B of gate key per candidate block (the
// projection weights come from L2: 32 KiB per query head).
#include "sas_device.h"
#include "sas_kernels.h"
#include "select.h"

namespace sas {

constexpr int kKeysInFlight = 32;  // gate keys per 16-lane group per pass (512 per workgroup)
constexpr int kKeysEarly = 16;     // of those, issued before the projection

// kMax: a candidate's score is the maximum over the group's query heads of
// <gate query, gate key> / sqrt(128) (group <= 8) instead of their mean.
// kPositions: batch entry s is position s of one sequence (length s + 1, the
// sequence's one block-table row, scores optional), for the training-time
// forward.  kSlice: the workgroup scores one slice of a (sequence, KV head)'s
// candidates, [slice * slice_len, +slice_len), and writes its own Top-K of
// them (score key, block, page; ascending block order, key 0 padding up to
// n_sel) instead of the selection: the pair's Top-K is then the Top-K of the
// slices' lists, since every block of the pair's Top-K is in its slice's.
// Compile-time switches keep the decode path's code unchanged.
template <bool kMax, bool kPositions, bool kSlice>
__global__ __launch_bounds__(256) void gate_topk_kernel(GateParams p) {
  // [max(rows, 512)]: block-table row (or slice), then score keys; with
  // kSlice the pages stay in a second array of the same size
  extern __shared__ __attribute__((aligned(16))) uint32_t slot[];
  __shared__ float qs[kMaxGroup][kHeadDim];
  __shared__ float vs[kMaxGroup][kGateDim];
  __shared__ float part[4][kGateDim];
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];

  // (sequence, KV head) pair; KV head = workgroup % Hkv, so one KV head's
  // workgroups share an XCD's L2 for their w_q rows
  const int kvh = kSlice ? (int)(blockIdx.x % p.n_kv_heads) : (int)blockIdx.x % p.n_kv_heads;
  const int slice = kSlice ? (int)(blockIdx.x / p.n_kv_heads) % p.slices : 0;
  const int s = kSlice ? (int)(blockIdx.x / p.n_kv_heads) / p.slices : (int)blockIdx.x / p.n_kv_heads;
  const int sk = s * p.n_kv_heads + kvh;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane16 = t & 15, grp = t >> 4;
  const int G = p.group;
  const int32_t L = kPositions ? s + 1 : p.seq_lens[s];
  const int n_all = (L - 1) / kBlock;  // candidates: the blocks before the local block
  const int k_eff = min(p.n_sel - 1, n_all);
  // this workgroup's candidates: [lo, lo + n), staged rows [lo, lo + rows)
  const int lo = kSlice ? slice * p.slice_len : 0;
  const int n = kSlice ? max(0, min(n_all - lo, p.slice_len)) : n_all;
  const int rows = kSlice ? min(p.slice_len, p.max_blocks - lo) : p.max_blocks;
  uint32_t *pg = kSlice ? slot + p.slot_len : slot;

  // ---- 1. issue every load the gate-query phase needs before anything
  // waits (so in-order load counters never hold it behind the gate-key
  // gather): the group's queries, the RoPE frequency and norm weights of
  // this lane's pair, the block-table row (its whole width, independent of
  // the sequence length), and the query-projection rows.  The G*128
  // projection outputs form 8G batches of 16 rows of one head (batch b: head
  // b/8, rows 16(b%8) .. +15, i.e. rows 16b .. 16b+15 of the group's heads);
  // lane group grp takes batches grp, grp+16, ...  A group reads a row as
  // 16 x 16 B (so a wave reads 4 whole rows per load), and a transposing row
  // sum leaves lane o of the group with row o of the batch.
  const uint16_t *qg = p.q + ((int64_t)s * p.n_q_heads + kvh * G) * kHeadDim;
  const bool has_q = 8 * t < G * kHeadDim;  // G <= 16: one 16-byte piece per thread
  // (kSlice: the gate queries come precomputed, gate_query_kernel)
  const u32x4 qpiece = kSlice ? u32x4{0, 0, 0, 0} : ld16(qg + (has_q ? 8 * t : 0));
  const double inv_freq = kSlice ? 0.0 : p.inv_freq[lane];
  const float wqn_a = kSlice ? 0.f : p.w_qnorm[lane], wqn_b = kSlice ? 0.f : p.w_qnorm[lane + 64];
  const int32_t *bt = (kPositions ? p.block_table : p.block_table + (int64_t)s * p.max_blocks) + lo;
  constexpr int kBtUnroll = 4;  // rows of up to 1,024 blocks staged without a loop
  int32_t btv[kBtUnroll];
#pragma unroll
  for (int k = 0; k < kBtUnroll; ++k) btv[k] = bt[min(t + 256 * k, rows - 1)];
  constexpr int kRowsInFlight = 32;  // two batches per group: all rows for G <= 4
  const int n_batches = 8 * G;
  const uint16_t *wq_lane = p.w_q + ((int64_t)kvh * G * kGateDim) * kHeadDim + 8 * lane16;
  u32x4 wv[kRowsInFlight];
  auto load_batches = [&](int round) {  // batches grp + 16(2 round), grp + 16(2 round + 1), clamped rows
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int row = 16 * (grp + 16 * (2 * round + u / 16)) + u % 16;
      wv[u] = ld16(wq_lane + (int64_t)min(row, G * kGateDim - 1) * kHeadDim);
    }
  };
  if (!kSlice) load_batches(0);

  if (!kSlice && has_q) {
    float *qd = &qs[0][0] + 8 * t;
    qd[0] = bf16_lo(qpiece.x); qd[1] = bf16_hi(qpiece.x); qd[2] = bf16_lo(qpiece.y); qd[3] = bf16_hi(qpiece.y);
    qd[4] = bf16_lo(qpiece.z); qd[5] = bf16_hi(qpiece.z); qd[6] = bf16_lo(qpiece.w); qd[7] = bf16_hi(qpiece.w);
  }
#pragma unroll
  for (int k = 0; k < kBtUnroll; ++k)
    if (t + 256 * k < rows) pg[t + 256 * k] = (uint32_t)btv[k];
  for (int c = t + 256 * kBtUnroll; c < rows; c += 256) pg[c] = (uint32_t)bt[c];
  lds_barrier();

  // ---- 1b. issue the first 256 candidates' gate keys now (they arrive
  // during the projection); the other 256 follow it (keeping all 512 in
  // registers across the projection would cost occupancy)
  const uint16_t *gkh = p.gate_keys + (int64_t)kvh * kGateDim + 8 * lane16;
  const int64_t page_stride = (int64_t)p.n_kv_heads * kGateDim;
  u32x4 v[kKeysInFlight];
  auto gather_key = [&](int c) -> u32x4 {
    // each gate key is read once per launch: non-temporal loads keep them out of the caches
    return c < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(gkh + (int64_t)pg[c] * page_stride))
                 : u32x4{0, 0, 0, 0};
  };
#pragma unroll
  for (int u = 0; u < kKeysEarly; ++u) v[u] = gather_key(16 * u + grp);

  // ---- 2. gate queries: v[g][j] = sum_d w_q[h][j][d] q[h][d], batch by
  // batch: lane o of the group ends with row o of the batch
  auto project_batches = [&](int round) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = grp + 16 * (2 * round + i);
      const int h = min(b >> 3, G - 1);
      const float *qq = qs[h] + 8 * lane16;
      float qv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = qq[e];
      float pp[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const u32x4 &w = wv[16 * i + r];
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
    }
  };
  if (!kSlice) {
    project_batches(0);
    for (int round = 1; 32 * round < n_batches; ++round) {  // G > 4 only
      load_batches(round);
      project_batches(round);
    }
  }
  // ---- 2b. issue candidates 256 .. 511; they arrive while the gate queries
  // are normalised and rotated
#pragma unroll
  for (int u = kKeysEarly; u < kKeysInFlight; ++u) v[u] = gather_key(16 * u + grp);
  lds_barrier();
  if (!kSlice) {  // RMSNorm + RoPE per head (wave w: heads w, w+4, ...; lane i: pair (i, i+64)); sum over heads
    float cf, sf;
    rope_cos_sin((double)(L - 1), inv_freq, cf, sf);
    const float wa = wqn_a, wb = wqn_b;
    float sa = 0.f, sb = 0.f;
    for (int g = wave; g < G; g += 4) {
      const float a = vs[g][lane], b = vs[g][lane + 64];
      const float inv = 1.0f / sqrtf(wave_sum(a * a + b * b) * (1.0f / kGateDim) + 1e-6f);
      const float na = a * inv * wa, nb = b * inv * wb;
      const float ra = na * cf - nb * sf, rb = nb * cf + na * sf;
      sa += ra;
      sb += rb;
      if (kMax) {  // each head's gate query, for the per-head scores
        vs[g][lane] = ra;
        vs[g][lane + 64] = rb;
      }
    }
    part[wave][lane] = sa;
    part[wave][lane + 64] = sb;
  }
  lds_barrier();
  float gm[8];  // mean gate query of the group, dims 8*lane16 .. +7
  float gh[kMax ? 8 : 1][8];  // kMax: per-head gate queries, dims 8*lane16 .. +7
  if (kSlice) {
    // the precomputed rotated gate queries, summed over heads exactly as
    // above: heads w, w+4, ... into partial w (from 0), then the partials
    const float *gq = p.gq + ((int64_t)s * p.n_q_heads + kvh * G) * kGateDim + 8 * lane16;
    float pw[4][8];
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) pw[w][e] = 0.f;
    for (int g = 0; g < G; ++g) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(gq + g * kGateDim);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(gq + g * kGateDim + 4);
      const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if ((g & 3) == w)
#pragma unroll
          for (int e = 0; e < 8; ++e) pw[w][e] += x[e];
      if (kMax) {
#pragma unroll
        for (int h = 0; h < (kMax ? 8 : 1); ++h)
          if (h == g)
#pragma unroll
            for (int e = 0; e < 8; ++e) gh[h][e] = x[e];
      }
    }
    if (kMax) {
#pragma unroll
      for (int h = 0; h < (kMax ? 8 : 1); ++h)
        if (h >= G)
#pragma unroll
          for (int e = 0; e < 8; ++e) gh[h][e] = 0.f;
    }
    const float inv_g = 1.0f / (float)G;
#pragma unroll
    for (int e = 0; e < 8; ++e) gm[e] = (pw[0][e] + pw[1][e] + pw[2][e] + pw[3][e]) * inv_g;
  } else {
    const float inv_g = 1.0f / (float)G;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lane16 + e;
      gm[e] = (part[0][d] + part[1][d] + part[2][d] + part[3][d]) * inv_g;
    }
    if (kMax) {
#pragma unroll
      for (int h = 0; h < (kMax ? 8 : 1); ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) gh[h][e] = h < G ? vs[h][8 * lane16 + e] : 0.f;
    }
  }

  // ---- 3. scores of every candidate (first 512 already in flight)
  const float inv_sqrt_dg = 0.08838834764831845f;  // 1/sqrt(128)
  float *scores = (!kPositions || p.scores) ? p.scores + (int64_t)sk * p.max_blocks + lo : nullptr;
  for (int base = 0; base < n; base += 16 * kKeysInFlight) {
    if (base > 0) {
#pragma unroll
      for (int u = 0; u < kKeysInFlight; ++u) v[u] = gather_key(base + 16 * u + grp);
    }
    // one row sum per candidate, always finished by lane 0 of the group, so
    // that equal gate keys get bit-equal scores wherever they sit (exact
    // ties break by block index)
#pragma unroll
    for (int u = 0; u < kKeysInFlight; ++u) {
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
      const int c = base + 16 * u + grp;
      if (lane16 == 0 && c < n) {
        const float sc = d * inv_sqrt_dg;
        slot[c] = score_key(sc);
        if (!kPositions || scores) scores[c] = sc;
      }
    }
  }
  if (!kPositions || scores)
    for (int c = n + t; c < rows; c += 256) scores[c] = -__builtin_inff();
  lds_barrier();
  if (wave != 0) return;

  // ---- 4. one wave selects
  if (kSlice) {  // this slice's Top-K, with pages, for the pair's final selection
    const int k_s = min(k_eff, n);
    const int64_t base = ((int64_t)sk * p.slices + slice) * p.n_sel;
    wave_select_emit(slot, n, k_s, hist, [&](uint32_t pos, int c, uint32_t key) {
      p.cand_key[base + pos] = key;
      p.cand_blk[base + pos] = lo + c;
      p.cand_page[base + pos] = (int32_t)pg[c];
    });
    for (int i = k_s + lane; i < p.n_sel; i += 64) p.cand_key[base + i] = 0u;
  } else {
    wave_select(slot, n, k_eff, p.n_sel, hist, p.sel + (int64_t)sk * p.n_sel,
                p.gates ? p.gates + (int64_t)sk * p.n_sel : nullptr, p.cnt + sk);
  }
}

// The rotated gate queries of the sliced selection, one query head of up to
// kGqSeqs sequences per workgroup: gq[s][h][:] = RoPE(RMSNorm(W_q[h] q[s][h])
// * w_qnorm, position L_s - 1), fp32.  The arithmetic and its order are the
// gate kernel's (16-row batches reduced by transposing row sums, the norm
// summed over the whole wave), so the slices score with the same bits.
// Computed once per (sequence, head) instead of once per slice: every slice
// would otherwise read the head group's whole w_q.
constexpr int kGqSeqs = 8;

__global__ __launch_bounds__(256) void gate_query_kernel(GateParams p) {
  __shared__ float qs[kGqSeqs][kHeadDim];
  __shared__ float us[kGqSeqs][kGateDim];
  const int h = blockIdx.x % p.n_q_heads;  // heads of one KV head share an XCD for their w_q rows
  const int s0 = (int)(blockIdx.x / p.n_q_heads) * kGqSeqs;
  const int ns = min(kGqSeqs, p.batch - s0);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane16 = t & 15, grp = t >> 4;
  // loads: the chunk's query rows of head h, this lane's norm weights and
  // RoPE frequency, batch grp % 8 of the head's projection rows
  const bool has_q = t < 16 * ns;
  const u32x4 qpiece = ld16(p.q + ((int64_t)(s0 + (has_q ? t >> 4 : 0)) * p.n_q_heads + h) * kHeadDim + 8 * lane16);
  const double inv_freq = p.inv_freq[lane];
  const float wqn_a = p.w_qnorm[lane], wqn_b = p.w_qnorm[lane + 64];
  const int b = grp & 7;
  const uint16_t *wq_rows = p.w_q + ((int64_t)h * kGateDim + 16 * b) * kHeadDim + 8 * lane16;
  u32x4 wv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wv[r] = ld16(wq_rows + (int64_t)r * kHeadDim);
  if (has_q) {
    float *qd = &qs[t >> 4][8 * lane16];
    qd[0] = bf16_lo(qpiece.x); qd[1] = bf16_hi(qpiece.x); qd[2] = bf16_lo(qpiece.y); qd[3] = bf16_hi(qpiece.y);
    qd[4] = bf16_lo(qpiece.z); qd[5] = bf16_hi(qpiece.z); qd[6] = bf16_lo(qpiece.w); qd[7] = bf16_hi(qpiece.w);
  }
  lds_barrier();
  // projection: groups grp and grp + 8 take batch b of alternate sequences;
  // lane o of the group ends with row 16b + o
  for (int j = grp >> 3; j < ns; j += 2) {
    const float *qq = &qs[j][8 * lane16];
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
    us[j][16 * b + lane16] = row16_transpose_sum(pp);
  }
  lds_barrier();
  // RMSNorm + RoPE per sequence (wave w: sequences w, w+4; lane i: pair (i, i+64))
  for (int j = wave; j < ns; j += 4) {
    const int s = s0 + j;
    float cf, sf;
    rope_cos_sin((double)(p.seq_lens[s] - 1), inv_freq, cf, sf);
    const float a = us[j][lane], c = us[j][lane + 64];
    const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) * (1.0f / kGateDim) + 1e-6f);
    const float na = a * inv * wqn_a, nb = c * inv * wqn_b;
    float *out = p.gq + ((int64_t)s * p.n_q_heads + h) * kGateDim;
    out[lane] = na * cf - nb * sf;
    out[lane + 64] = nb * cf + na * sf;
  }
}

hipError_t launch_gate_query(const GateParams &p, hipStream_t st) {
  const dim3 grid((unsigned)(p.n_q_heads * ((p.batch + kGqSeqs - 1) / kGqSeqs)));
  hipLaunchKernelGGL(gate_query_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gate_topk(const GateParams &p, int batch, hipStream_t st) {
  // the selecting wave reads the first 512 slots as whole vectors
  const size_t lds = sizeof(uint32_t) * (size_t)(p.max_blocks > 512 ? (p.max_blocks + 7) / 8 * 8 : 512);
  // allow the largest block-table row (64 KiB of LDS); set once per process
  static const hipError_t attr = [] {
    const int most = (int)(sizeof(uint32_t) * SAS_MAX_BLOCKS_DEV);
    const void *kernels[] = {(const void *)gate_topk_kernel<false, false, false>,
                             (const void *)gate_topk_kernel<true, false, false>,
                             (const void *)gate_topk_kernel<false, true, false>};
    for (const void *k : kernels) {
      hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, most);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)(batch * p.n_kv_heads));
  if (p.bt_row_stride == 0)
    hipLaunchKernelGGL((gate_topk_kernel<false, true, false>), grid, dim3(256), lds, st, p);
  else if (p.aggregate)
    hipLaunchKernelGGL((gate_topk_kernel<true, false, false>), grid, dim3(256), lds, st, p);
  else
    hipLaunchKernelGGL((gate_topk_kernel<false, false, false>), grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

void gate_slice_layout(int batch, int n_kv_heads, int max_blocks, int cus, int *slices, int *slice_len) {
  // about two workgroups per CU over the pairs, slices of at least 64
  // candidates, and every slice starting inside the block-table row
  const int pairs = batch * n_kv_heads;
  int sl = (2 * cus + pairs - 1) / pairs;
  const int most = (max_blocks + 63) / 64;
  sl = sl > most ? most : sl;
  sl = sl > kMaxSlices ? kMaxSlices : sl;
  sl = sl < 1 ? 1 : sl;
  int len = (max_blocks + sl - 1) / sl;
  while (sl > 1 && (sl - 1) * len >= max_blocks) {
    --sl;
    len = (max_blocks + sl - 1) / sl;
  }
  *slices = sl;
  *slice_len = len;
}

hipError_t launch_gate_slices(const GateParams &p, int batch, hipStream_t st) {
  // score keys and pages of one slice, each at least 512 entries
  const size_t lds = 2 * sizeof(uint32_t) * (size_t)p.slot_len;
  static const hipError_t attr = [] {
    const int most = (int)(2 * sizeof(uint32_t) * SAS_MAX_BLOCKS_DEV);
    const void *kernels[] = {(const void *)gate_topk_kernel<false, false, true>,
                             (const void *)gate_topk_kernel<true, false, true>};
    for (const void *k : kernels) {
      hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, most);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)(batch * p.slices * p.n_kv_heads));
  if (p.aggregate)
    hipLaunchKernelGGL((gate_topk_kernel<true, false, true>), grid, dim3(256), lds, st, p);
  else
    hipLaunchKernelGGL((gate_topk_kernel<false, false, true>), grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

}  // namespace sas
