// Parameter block and launcher of the continuous-gate backward of the
// training-time forward (internal to the library).
#pragma once
#include "sas_kernels.h"

namespace sas {

constexpr int kPrefillSplit = 16;  // row ranges of each long sum over positions, added in order afterwards

// Query heads per MFMA column group of the training-time walks (a wave's 16
// columns are 16/h queries x h heads), for a group of G query heads; a
// workgroup covers one group of h heads, so a KV head's G heads take
// ceil(G / h) workgroups per 64 queries.
__host__ __device__ inline int prefill_heads_per_wave(int group) { return group >= 3 ? 4 : group; }

struct PrefillBackwardParams {
  const uint16_t *q, *k_pool, *v_pool, *d_out;  // q, d_out [T][Hq][128]
  const uint16_t *gate_keys, *w_q, *w_k;
  const int32_t *block_table;                   // the sequence's row
  const int32_t *sel, *cnt;                     // [T][Hkv][max_sel], [T][Hkv]
  const float *gates, *lse;                     // gates as sel; lse [T][Hq] (natural log)
  const float *w_qnorm, *w_knorm;
  float *d_gates;                               // [T][Hkv][max_sel]
  float *d_w_q, *d_w_qnorm, *d_w_k, *d_w_knorm;
  // workspace
  float *ws_dgp;   // [head_groups][T][Hkv][max_sel]  dL/dg, one term per workgroup head group
  float *ws_ghat;  // [Hkv][T][128]                   group-mean gate query of every position
  float *ws_a;     // [Hkv][T][a_cols]                dS / sqrt(128) at each historical block's column, else 0
  float *ws_du_q;  // [T][Hq][128]                    d(pre-norm gate query)
  float *ws_dwqn;  // [n_qblocks][Hkv][128]           query-norm weight terms per 64 positions
  float *ws_pool;  // [Hkv][n_hist][384]              pooled statistics of the blocks that can be historical
  float *ws_dgk;   // [Hkv][a_cols][128]              d(gate key) of every such block
  float *ws_du_k;  // [Hkv][n_hist][128]              d(pre-norm gate key)
  float *ws_dwkn;  // [Hkv][key_chunks][128]          key-norm weight terms per 16 blocks
  float *ws_part;  // [part_tiles][kPrefillSplit][64][64] partial sums of the long outer-product tiles
  int64_t page_stride, tok_stride, head_stride;
  int32_t n_q_heads, n_kv_heads, group, head_groups, max_sel, seq_len, n_qblocks;
  int32_t n_hist;      // blocks that some position can select as historical: (T - 1) / 64
  int32_t a_cols;      // n_hist rounded up to 64
  int32_t key_chunks;  // ceil(n_hist / 16)
  float scale_log2;    // sm_scale * log2(e)
  double inv_freq[kGateDim / 2];
};

hipError_t launch_prefill_grad(const PrefillBackwardParams &p, hipStream_t st);
hipError_t launch_prefill_gate_backward(const PrefillBackwardParams &p, hipStream_t st);

}  // namespace sas
