// Kernel parameter blocks and launchers of libsas (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sas_device.h"

namespace sas {

struct PoolParams {
  const uint16_t *k_pool;
  const int32_t *block_table;
  const int32_t *pool_seq, *pool_blk;
  const uint16_t *w_k;      // [Hkv][384][128]
  const float *w_knorm;     // [128]
  uint16_t *gate_keys;      // [P][Hkv][128]
  int64_t page_stride, tok_stride, head_stride;
  int32_t n, n_kv_heads, max_blocks;
  double theta;
};

struct AppendParams {
  const uint16_t *k_new, *v_new;  // [B][Hkv][128]
  uint16_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_lens;
  const uint16_t *w_k;            // [Hkv][128][384]
  const float *w_knorm;           // [128]
  uint16_t *gate_keys;            // [P][Hkv][128]
  int64_t page_stride, tok_stride, head_stride;
  int32_t n_kv_heads, max_blocks;
  double theta;
};

struct GateParams {
  const uint16_t *q;        // [B][Hq][128]
  const uint16_t *w_q;      // [Hq][128 out][128 in]
  const float *w_qnorm;     // [128]
  const uint16_t *gate_keys;
  const int32_t *block_table, *seq_lens;  // seq_lens NULL: entry s is position s of one sequence (L = s + 1)
  int32_t *sel;
  float *gates;             // nullable
  int32_t *cnt;
  float *scores;            // [B][Hkv][max_blocks], nullable
  int32_t n_q_heads, n_kv_heads, group, max_blocks, n_sel;
  int32_t bt_row_stride;    // max_blocks, or 0 when every entry shares one block-table row
  int32_t aggregate;        // 0: mean of the group's per-head scores, 1: their maximum (group <= 8)
  // sliced selection (launch_gate_slices): each pair's candidates in `slices`
  // slices of slice_len; per (pair, slice) n_sel entries of the slice's
  // Top-K (score key, 0 = padding; block; page); slot_len = LDS rows per slice
  int32_t slices, slice_len, slot_len, batch;
  float *gq;                // [B][Hq][128] rotated gate queries (gate_query_kernel)
  uint32_t *cand_key;
  int32_t *cand_blk, *cand_page;
  double inv_freq[kGateDim / 2];  // rope_theta^(-i/64)
};

struct DecodeParams {
  const uint16_t *q;
  const uint16_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_lens, *sel, *cnt;
  const float *gates;       // null: plain Top-K mode
  float *part_o;            // [B*Hkv][wg_per_unit][G][128] unnormalised partial outputs
  float *part_ml;           // [B*Hkv][wg_per_unit][G][2]   (max, sum) per partial
  uint16_t *out;            // [B][Hq][128]
  int64_t page_stride, tok_stride, head_stride;
  int32_t n_q_heads, n_kv_heads, group, max_blocks, max_sel;
  int32_t wg_per_unit;      // workgroups per (sequence, KV head)
  int32_t blocks_per_wave;  // selected blocks each wave handles
  int32_t gate_mode;        // with gates: 0 scale each block's share, 1 log-gate bias on the logits
  float scale_log2;         // sm_scale * log2(e)
};

// Decode work split: waves per (sequence, KV head) and blocks per wave, for
// a device of `cus` compute units (one 8-wave workgroup per CU).
struct DecodeSplit {
  int wg_per_unit, waves_per_unit, blocks_per_wave;
};
DecodeSplit decode_split(int batch, int n_kv_heads, int max_sel, int cus);

// The fused decode step: the selection's and the attention's parameter blocks
// (the attention with one workgroup per (sequence, KV head)).
struct StepParams {
  GateParams g;
  DecodeParams d;
};
bool step_fits(int group, int max_blocks, int n_sel);

constexpr int kMaxSlices = 16;  // slices of one pair's candidates in the sliced selection
// Slices per pair and their length for the sliced selection (about two
// workgroups per compute unit of a `cus`-CU device); every slice starts
// inside the block-table row ((slices - 1) * slice_len < max_blocks).
void gate_slice_layout(int batch, int n_kv_heads, int max_blocks, int cus, int *slices, int *slice_len);

struct PrefillParams {
  const uint16_t *q;            // [T][Hq][128]
  const uint16_t *k_pool, *v_pool;
  const int32_t *block_table;   // the sequence's row [max_blocks]
  const int32_t *sel;           // [T][Hkv][max_sel]
  const float *gates;           // nullable
  const int32_t *cnt;           // [T][Hkv]
  uint16_t *out;                // [T][Hq][128]
  float *lse;                   // [T][Hq] log-sum-exp of the logits, nullable
  int64_t page_stride, tok_stride, head_stride;
  int32_t n_q_heads, n_kv_heads, group, head_groups, max_sel, seq_len, n_qblocks;
  float scale_log2;
};

constexpr int kChainBlocks = 16;  // selected blocks the backward chain handles at a time
constexpr int kSplitK = 8;        // row ranges of each dW_k tile summed separately, then in order
constexpr int kMaxSelBackward = 256;  // selection slots per (sequence, KV head) the backward accepts

struct BackwardParams {
  const uint16_t *q, *k_pool, *v_pool, *d_out, *gate_keys, *w_q, *w_k;
  const int32_t *block_table, *seq_lens, *sel, *cnt;
  const float *gates, *w_qnorm, *w_knorm;
  float *d_gates;                 // [B][Hkv][max_sel]
  float *d_w_q, *d_w_qnorm, *d_w_k, *d_w_knorm;
  // workspace: per-sequence factors of the weight gradients
  float *ws_du_q;                 // [B][Hq][128]
  float *ws_du_k;                 // [B][Hkv][max_sel][128]
  float *ws_pool;                 // [B][Hkv][max_sel][384]
  float *ws_dwqn, *ws_dwkn;       // [B][Hkv][128]: norm-weight terms summed per (sequence, KV head)
  float *ws_part;                 // [Hkv*12][kSplitK][64][64]: partial dW_k tiles
  int64_t page_stride, tok_stride, head_stride;
  int32_t batch, n_q_heads, n_kv_heads, group, max_blocks, max_sel;
  float scale_log2;
  double inv_freq[kGateDim / 2];
};

constexpr int kMaxCandBatched = 512;  // candidates per position the batched prefill selection holds

struct PrefillSelectParams {
  const uint16_t *q;            // [T][Hq][128]
  const uint16_t *w_q;          // [Hq][128 out][128 in]
  const float *w_qnorm;
  const uint16_t *gate_keys;    // [P][Hkv][128]
  const int32_t *block_table;   // the sequence's row
  int32_t *sel;                 // [T][Hkv][n_sel]
  float *gates;                 // nullable
  int32_t *cnt;                 // [T][Hkv]
  float *scores;                // [T][Hkv][max_blocks], nullable
  int32_t n_q_heads, n_kv_heads, group, max_blocks, n_sel, seq_len, n_qblocks;
  double inv_freq[kGateDim / 2];
};

hipError_t launch_pool(const PoolParams &p, hipStream_t st);
hipError_t launch_prefill_select(const PrefillSelectParams &p, hipStream_t st);
hipError_t launch_gate_backward(const BackwardParams &p, hipStream_t st);
hipError_t launch_prefill_attend(const PrefillParams &p, hipStream_t st);
hipError_t launch_append(const AppendParams &p, int batch, hipStream_t st);
hipError_t launch_gate_topk(const GateParams &p, int batch, hipStream_t st);
hipError_t launch_gate_query(const GateParams &p, hipStream_t st);
hipError_t launch_gate_slices(const GateParams &p, int batch, hipStream_t st);
hipError_t launch_decode(const DecodeParams &p, int batch, hipStream_t st);
hipError_t launch_step(const StepParams &p, int batch, hipStream_t st);
hipError_t launch_select_decode(const StepParams &p, int batch, hipStream_t st);
hipError_t launch_decode_merge(const DecodeParams &p, int batch, hipStream_t st);

}  // namespace sas
