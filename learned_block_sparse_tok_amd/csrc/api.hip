// C ABI of libsas: argument checks, workspace carving, kernel launches.
#include <math.h>
#include <stdarg.h>

#include <atomic>
#include <mutex>
#include <stdio.h>
#include <string.h>

#include "../../include/sas.h"
#include "prefill_backward.h"
#include "sas_device.h"
#include "sas_kernels.h"

static_assert(SAS_MAX_BLOCKS == SAS_MAX_BLOCKS_DEV, "block-table limit mismatch");

namespace sas {
// the read-bandwidth probe (probe.hip), a measurement utility
hipError_t launch_read_probe(const uint64_t *addr, int32_t n, int32_t per, void *sink, hipStream_t st);
}  // namespace sas

namespace {

thread_local char g_last_error[512] = "";

sas_status fail(sas_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

sas_status ok() {
  g_last_error[0] = '\0';
  return SAS_OK;
}

sas_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(SAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device, read once per device and cached (the
// decode split and the sliced selection size their grids by it).  256, the
// MI355X's count, when no device is visible (host-only workspace queries).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int c = g_cus[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  g_cus[dev].store(c, std::memory_order_relaxed);
  return c;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

sas_status check_shape(const sas_shape *sh, bool need_kv_strides) {
  if (!sh) return fail(SAS_ERR_INVALID_ARG, "shape is NULL");
  if (sh->batch <= 0 || sh->n_q_heads <= 0 || sh->n_kv_heads <= 0 || sh->max_blocks <= 0)
    return fail(SAS_ERR_INVALID_ARG, "batch, n_q_heads, n_kv_heads and max_blocks must be positive");
  if (sh->n_q_heads % sh->n_kv_heads != 0)
    return fail(SAS_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", sh->n_q_heads,
                sh->n_kv_heads);
  if (sh->n_q_heads / sh->n_kv_heads > SAS_MAX_GROUP)
    return fail(SAS_ERR_UNSUPPORTED, "group size %d exceeds %d", sh->n_q_heads / sh->n_kv_heads, SAS_MAX_GROUP);
  if (sh->max_blocks > SAS_MAX_BLOCKS)
    return fail(SAS_ERR_UNSUPPORTED, "max_blocks %d exceeds %d", sh->max_blocks, SAS_MAX_BLOCKS);
  if (need_kv_strides) {
    if (sh->page_stride <= 0 || sh->tok_stride <= 0 || sh->head_stride <= 0)
      return fail(SAS_ERR_INVALID_ARG, "KV strides must be positive");
    if (sh->page_stride % 8 || sh->tok_stride % 8 || sh->head_stride % 8)
      return fail(SAS_ERR_UNSUPPORTED, "KV strides must be multiples of 8 elements");
    if (sh->tok_stride < SAS_HEAD_DIM)
      return fail(SAS_ERR_INVALID_ARG, "tok_stride must be at least %d", SAS_HEAD_DIM);
  }
  return SAS_OK;
}

}  // namespace

extern "C" {

const char *sas_status_str(sas_status st) {
  switch (st) {
    case SAS_OK: return "SAS_OK";
    case SAS_ERR_INVALID_ARG: return "SAS_ERR_INVALID_ARG";
    case SAS_ERR_UNSUPPORTED: return "SAS_ERR_UNSUPPORTED";
    case SAS_ERR_WORKSPACE: return "SAS_ERR_WORKSPACE";
    case SAS_ERR_HIP: return "SAS_ERR_HIP";
    default: return "SAS_ERR_UNKNOWN";
  }
}

const char *sas_last_error(void) { return g_last_error; }

int32_t sas_version(void) { return 100; }

sas_status sas_probe_read(const uint64_t *chunk_addr, int32_t n_chunks, int32_t chunks_per_wg, void *sink,
                          size_t sink_bytes, void *stream) {
  if (n_chunks < 0) return fail(SAS_ERR_INVALID_ARG, "n_chunks is negative");
  if (chunks_per_wg < 1 || chunks_per_wg > 64) return fail(SAS_ERR_INVALID_ARG, "chunks_per_wg must be in 1..64");
  if (n_chunks == 0) return ok();
  if (!chunk_addr || !sink) return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(sink)) return fail(SAS_ERR_INVALID_ARG, "sink must be 16-byte aligned");
  const size_t need = (size_t)((n_chunks + chunks_per_wg - 1) / chunks_per_wg) * 16;
  if (sink_bytes < need) return fail(SAS_ERR_INVALID_ARG, "sink %zu bytes < required %zu", sink_bytes, need);
  return hip_status(sas::launch_read_probe(chunk_addr, n_chunks, chunks_per_wg, sink, (hipStream_t)stream),
                    "read probe");
}

sas_status sas_pool_blocks(const sas_shape *shape, const void *k_pool, const int32_t *block_table,
                           const int32_t *pool_seq, const int32_t *pool_blk, int32_t n, const void *w_k,
                           const float *w_knorm, double rope_theta, void *gate_keys, void *stream) {
  sas_status st = check_shape(shape, true);
  if (st) return st;
  if (n < 0) return fail(SAS_ERR_INVALID_ARG, "n is negative");
  if (n == 0) return ok();
  if (!k_pool || !block_table || !pool_seq || !pool_blk || !w_k || !w_knorm || !gate_keys)
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!(rope_theta > 1.0)) return fail(SAS_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!aligned16(gate_keys)) return fail(SAS_ERR_UNSUPPORTED, "gate_keys must be 16-byte aligned");
  sas::PoolParams p;
  p.k_pool = (const uint16_t *)k_pool;
  p.block_table = block_table;
  p.pool_seq = pool_seq;
  p.pool_blk = pool_blk;
  p.w_k = (const uint16_t *)w_k;
  p.w_knorm = w_knorm;
  p.gate_keys = (uint16_t *)gate_keys;
  p.page_stride = shape->page_stride;
  p.tok_stride = shape->tok_stride;
  p.head_stride = shape->head_stride;
  p.n = n;
  p.n_kv_heads = shape->n_kv_heads;
  p.max_blocks = shape->max_blocks;
  p.theta = rope_theta;
  return hip_status(sas::launch_pool(p, (hipStream_t)stream), "sas_pool_blocks launch");
}

sas_status sas_append_kv(const sas_shape *shape, const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                         const int32_t *block_table, const int32_t *seq_lens, const void *w_k, const float *w_knorm,
                         double rope_theta, void *gate_keys, void *stream) {
  sas_status st = check_shape(shape, true);
  if (st) return st;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !seq_lens || !w_k || !w_knorm || !gate_keys)
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!(rope_theta > 1.0)) return fail(SAS_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(gate_keys))
    return fail(SAS_ERR_UNSUPPORTED, "k_new, v_new, k_pool, v_pool and gate_keys must be 16-byte aligned");
  sas::AppendParams p;
  p.k_new = (const uint16_t *)k_new;
  p.v_new = (const uint16_t *)v_new;
  p.k_pool = (uint16_t *)k_pool;
  p.v_pool = (uint16_t *)v_pool;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.w_k = (const uint16_t *)w_k;
  p.w_knorm = w_knorm;
  p.gate_keys = (uint16_t *)gate_keys;
  p.page_stride = shape->page_stride;
  p.tok_stride = shape->tok_stride;
  p.head_stride = shape->head_stride;
  p.n_kv_heads = shape->n_kv_heads;
  p.max_blocks = shape->max_blocks;
  p.theta = rope_theta;
  return hip_status(sas::launch_append(p, shape->batch, (hipStream_t)stream), "sas_append_kv launch");
}

namespace {
// Checks the selection arguments and fills its parameter block (scores
// nullable only where the caller supplies another buffer or skips them).
sas_status gate_params(const sas_shape *shape, const void *q, const void *w_q, const float *w_qnorm,
                       const void *gate_keys, const int32_t *block_table, const int32_t *seq_lens, double rope_theta,
                       int32_t budget_tokens, int32_t aggregate, int32_t *sel, float *gates, int32_t *cnt,
                       float *scores, bool scores_nullable, sas::GateParams &p) {
  sas_status st = check_shape(shape, false);
  if (st) return st;
  if (aggregate != SAS_AGG_MEAN && aggregate != SAS_AGG_MAX)
    return fail(SAS_ERR_INVALID_ARG, "unknown score aggregation %d", aggregate);
  if (aggregate == SAS_AGG_MAX && shape->n_q_heads / shape->n_kv_heads > 8)
    return fail(SAS_ERR_UNSUPPORTED, "max aggregation supports groups of at most 8 query heads");
  if (!q || !w_q || !w_qnorm || !gate_keys || !block_table || !seq_lens || !sel || !cnt ||
      (!scores && !scores_nullable))
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (budget_tokens < SAS_BLOCK || budget_tokens % SAS_BLOCK)
    return fail(SAS_ERR_INVALID_ARG, "budget_tokens (%d) must be a positive multiple of %d", budget_tokens,
                SAS_BLOCK);
  if (budget_tokens / SAS_BLOCK > 256)
    return fail(SAS_ERR_UNSUPPORTED, "budget_tokens (%d) exceeds %d", budget_tokens, 256 * SAS_BLOCK);
  if (!(rope_theta > 1.0)) return fail(SAS_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!aligned16(gate_keys) || !aligned16(w_q))
    return fail(SAS_ERR_UNSUPPORTED, "gate_keys and w_q must be 16-byte aligned");
  p.q = (const uint16_t *)q;
  p.w_q = (const uint16_t *)w_q;
  p.w_qnorm = w_qnorm;
  p.gate_keys = (const uint16_t *)gate_keys;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.sel = sel;
  p.gates = gates;
  p.cnt = cnt;
  p.scores = scores;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.group = shape->n_q_heads / shape->n_kv_heads;
  p.max_blocks = shape->max_blocks;
  p.n_sel = budget_tokens / SAS_BLOCK;
  p.bt_row_stride = shape->max_blocks;
  p.aggregate = aggregate;
  for (int i = 0; i < SAS_GATE_DIM / 2; ++i) p.inv_freq[i] = pow(rope_theta, -(double)i / (SAS_GATE_DIM / 2));
  return SAS_OK;
}
}  // namespace

sas_status sas_gate_topk_ex(const sas_shape *shape, const void *q, const void *w_q, const float *w_qnorm,
                            const void *gate_keys, const int32_t *block_table, const int32_t *seq_lens,
                            double rope_theta, int32_t budget_tokens, int32_t aggregate, int32_t *sel, float *gates,
                            int32_t *cnt, float *scores, void *stream) {
  sas::GateParams p;
  sas_status st = gate_params(shape, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, rope_theta, budget_tokens,
                              aggregate, sel, gates, cnt, scores, false, p);
  if (st) return st;
  return hip_status(sas::launch_gate_topk(p, shape->batch, (hipStream_t)stream), "sas_gate_topk launch");
}

sas_status sas_gate_topk(const sas_shape *shape, const void *q, const void *w_q, const float *w_qnorm,
                         const void *gate_keys, const int32_t *block_table, const int32_t *seq_lens,
                         double rope_theta, int32_t budget_tokens, int32_t *sel, float *gates, int32_t *cnt,
                         float *scores, void *stream) {
  return sas_gate_topk_ex(shape, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, rope_theta, budget_tokens,
                          SAS_AGG_MEAN, sel, gates, cnt, scores, stream);
}

namespace {
sas_status check_prefill(const sas_shape *shape, bool need_kv_strides, int32_t seq_len) {
  sas_status st = check_shape(shape, need_kv_strides);
  if (st) return st;
  if (shape->batch != 1) return fail(SAS_ERR_INVALID_ARG, "prefill calls take one sequence (batch %d)", shape->batch);
  if (seq_len < 1) return fail(SAS_ERR_INVALID_ARG, "seq_len must be positive");
  if ((seq_len + SAS_BLOCK - 1) / SAS_BLOCK > shape->max_blocks)
    return fail(SAS_ERR_INVALID_ARG, "seq_len %d needs more than max_blocks (%d) blocks", seq_len, shape->max_blocks);
  return SAS_OK;
}
}  // namespace

sas_status sas_prefill_select(const sas_shape *shape, const void *q, const void *w_q, const float *w_qnorm,
                              const void *gate_keys, const int32_t *block_table_row, int32_t seq_len,
                              double rope_theta, int32_t budget_tokens, int32_t *sel, float *gates, int32_t *cnt,
                              float *scores, void *stream) {
  sas_status st = check_prefill(shape, false, seq_len);
  if (st) return st;
  if (!q || !w_q || !w_qnorm || !gate_keys || !block_table_row || !sel || !cnt)
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (budget_tokens < SAS_BLOCK || budget_tokens % SAS_BLOCK)
    return fail(SAS_ERR_INVALID_ARG, "budget_tokens (%d) must be a positive multiple of %d", budget_tokens,
                SAS_BLOCK);
  if (budget_tokens / SAS_BLOCK > 256)
    return fail(SAS_ERR_UNSUPPORTED, "budget_tokens (%d) exceeds %d", budget_tokens, 256 * SAS_BLOCK);
  if (!(rope_theta > 1.0)) return fail(SAS_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!aligned16(gate_keys) || !aligned16(w_q))
    return fail(SAS_ERR_UNSUPPORTED, "gate_keys and w_q must be 16-byte aligned");
  const int n_qblocks = (seq_len + SAS_BLOCK - 1) / SAS_BLOCK;
  if (n_qblocks - 1 <= sas::kMaxCandBatched) {  // one workgroup per 64 positions and KV head
    sas::PrefillSelectParams b;
    b.q = (const uint16_t *)q;
    b.w_q = (const uint16_t *)w_q;
    b.w_qnorm = w_qnorm;
    b.gate_keys = (const uint16_t *)gate_keys;
    b.block_table = block_table_row;
    b.sel = sel;
    b.gates = gates;
    b.cnt = cnt;
    b.scores = scores;
    b.n_q_heads = shape->n_q_heads;
    b.n_kv_heads = shape->n_kv_heads;
    b.group = shape->n_q_heads / shape->n_kv_heads;
    b.max_blocks = shape->max_blocks;
    b.n_sel = budget_tokens / SAS_BLOCK;
    b.seq_len = seq_len;
    b.n_qblocks = n_qblocks;
    for (int i = 0; i < SAS_GATE_DIM / 2; ++i) b.inv_freq[i] = pow(rope_theta, -(double)i / (SAS_GATE_DIM / 2));
    return hip_status(sas::launch_prefill_select(b, (hipStream_t)stream), "sas_prefill_select launch");
  }
  // longer sequences: the decode selection kernel once per (position, KV head)
  sas::GateParams p;
  p.q = (const uint16_t *)q;
  p.w_q = (const uint16_t *)w_q;
  p.w_qnorm = w_qnorm;
  p.gate_keys = (const uint16_t *)gate_keys;
  p.block_table = block_table_row;
  p.seq_lens = nullptr;  // entry t is position t: L = t + 1
  p.sel = sel;
  p.gates = gates;
  p.cnt = cnt;
  p.scores = scores;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.group = shape->n_q_heads / shape->n_kv_heads;
  p.max_blocks = shape->max_blocks;
  p.n_sel = budget_tokens / SAS_BLOCK;
  p.bt_row_stride = 0;
  p.aggregate = SAS_AGG_MEAN;
  for (int i = 0; i < SAS_GATE_DIM / 2; ++i) p.inv_freq[i] = pow(rope_theta, -(double)i / (SAS_GATE_DIM / 2));
  return hip_status(sas::launch_gate_topk(p, seq_len, (hipStream_t)stream), "sas_prefill_select launch");
}

sas_status sas_prefill_attend(const sas_shape *shape, const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *block_table_row, int32_t seq_len, const int32_t *sel,
                              const float *gates, const int32_t *cnt, int32_t max_sel, float sm_scale, void *out,
                              float *lse, void *stream) {
  sas_status st = check_prefill(shape, true, seq_len);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !block_table_row || !sel || !cnt || !out)
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (max_sel <= 0) return fail(SAS_ERR_INVALID_ARG, "max_sel must be positive");
  if (max_sel > 64) return fail(SAS_ERR_UNSUPPORTED, "max_sel %d exceeds 64 (budgets above 4,096 tokens)", max_sel);
  if (!(sm_scale > 0.f)) return fail(SAS_ERR_INVALID_ARG, "sm_scale must be positive");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(SAS_ERR_UNSUPPORTED, "q, k_pool, v_pool and out must be 16-byte aligned");
  sas::PrefillParams p;
  p.q = (const uint16_t *)q;
  p.k_pool = (const uint16_t *)k_pool;
  p.v_pool = (const uint16_t *)v_pool;
  p.block_table = block_table_row;
  p.sel = sel;
  p.gates = gates;
  p.cnt = cnt;
  p.out = (uint16_t *)out;
  p.lse = lse;
  p.page_stride = shape->page_stride;
  p.tok_stride = shape->tok_stride;
  p.head_stride = shape->head_stride;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.group = shape->n_q_heads / shape->n_kv_heads;
  p.head_groups = 0;  // set by the launcher for its wave layout
  p.max_sel = max_sel;
  p.seq_len = seq_len;
  p.n_qblocks = (seq_len + SAS_BLOCK - 1) / SAS_BLOCK;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  return hip_status(sas::launch_prefill_attend(p, (hipStream_t)stream), "sas_prefill_attend launch");
}

namespace {
struct DecodeWorkspace {
  size_t part_o, part_ml, total;  // byte offsets and size
};
DecodeWorkspace decode_workspace(const sas_shape *shape, int32_t max_sel) {
  sas::DecodeSplit sp = sas::decode_split(shape->batch, shape->n_kv_heads, max_sel, device_cus());
  const size_t slots = (size_t)shape->batch * shape->n_q_heads * sp.wg_per_unit;
  DecodeWorkspace w;
  w.part_o = 0;
  w.part_ml = w.part_o + align256(slots * SAS_HEAD_DIM * sizeof(float));
  w.total = w.part_ml + align256(slots * 2 * sizeof(float));
  return w;
}
}  // namespace

size_t sas_sparse_decode_workspace_bytes(const sas_shape *shape, int32_t max_sel) {
  if (!shape || shape->batch <= 0 || shape->n_kv_heads <= 0 || shape->n_q_heads <= 0 || max_sel <= 0) return 0;
  return decode_workspace(shape, max_sel).total;
}

namespace {
// Checks the attention arguments (not the workspace) and fills its
// parameter block for max_sel selection slots per (sequence, KV head).
sas_status decode_params(const sas_shape *shape, const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *block_table, const int32_t *seq_lens, const int32_t *sel, const float *gates,
                         int32_t gate_mode, const int32_t *cnt, int32_t max_sel, float sm_scale, void *out,
                         sas::DecodeParams &p) {
  sas_status st = check_shape(shape, true);
  if (st) return st;
  if (gate_mode != SAS_GATE_SCALE && gate_mode != SAS_GATE_LOGIT)
    return fail(SAS_ERR_INVALID_ARG, "unknown gate mode %d", gate_mode);
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !sel || !cnt || !out)
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (max_sel <= 0) return fail(SAS_ERR_INVALID_ARG, "max_sel must be positive");
  if (!(sm_scale > 0.f)) return fail(SAS_ERR_INVALID_ARG, "sm_scale must be positive");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(SAS_ERR_UNSUPPORTED, "q, k_pool and v_pool must be 16-byte aligned");
  const sas::DecodeSplit sp = sas::decode_split(shape->batch, shape->n_kv_heads, max_sel, device_cus());
  p.q = (const uint16_t *)q;
  p.k_pool = (const uint16_t *)k_pool;
  p.v_pool = (const uint16_t *)v_pool;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.sel = sel;
  p.cnt = cnt;
  p.gates = gates;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  p.out = (uint16_t *)out;
  p.page_stride = shape->page_stride;
  p.tok_stride = shape->tok_stride;
  p.head_stride = shape->head_stride;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.group = shape->n_q_heads / shape->n_kv_heads;
  p.max_blocks = shape->max_blocks;
  p.max_sel = max_sel;
  p.wg_per_unit = sp.wg_per_unit;
  p.blocks_per_wave = sp.blocks_per_wave;
  p.gate_mode = gate_mode;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  return SAS_OK;
}

// Carves the partial-result buffers of a split decode out of the workspace.
sas_status decode_workspace_bind(const sas_shape *shape, int32_t max_sel, void *workspace, size_t workspace_bytes,
                                 sas::DecodeParams &p) {
  if (!workspace) return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(workspace)) return fail(SAS_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  const DecodeWorkspace wl = decode_workspace(shape, max_sel);
  if (workspace_bytes < wl.total)
    return fail(SAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, wl.total);
  p.part_o = (float *)((char *)workspace + wl.part_o);
  p.part_ml = (float *)((char *)workspace + wl.part_ml);
  return SAS_OK;
}
}  // namespace

sas_status sas_sparse_decode_ex(const sas_shape *shape, const void *q, const void *k_pool, const void *v_pool,
                                const int32_t *block_table, const int32_t *seq_lens, const int32_t *sel,
                                const float *gates, int32_t gate_mode, const int32_t *cnt, int32_t max_sel,
                                float sm_scale, void *out, void *workspace, size_t workspace_bytes, void *stream) {
  sas::DecodeParams p;
  sas_status st = decode_params(shape, q, k_pool, v_pool, block_table, seq_lens, sel, gates, gate_mode, cnt, max_sel,
                                sm_scale, out, p);
  if (st) return st;
  st = decode_workspace_bind(shape, max_sel, workspace, workspace_bytes, p);
  if (st) return st;
  return hip_status(sas::launch_decode(p, shape->batch, (hipStream_t)stream), "sas_sparse_decode launch");
}

sas_status sas_sparse_decode(const sas_shape *shape, const void *q, const void *k_pool, const void *v_pool,
                             const int32_t *block_table, const int32_t *seq_lens, const int32_t *sel,
                             const float *gates, const int32_t *cnt, int32_t max_sel, float sm_scale, void *out,
                             void *workspace, size_t workspace_bytes, void *stream) {
  return sas_sparse_decode_ex(shape, q, k_pool, v_pool, block_table, seq_lens, sel, gates, SAS_GATE_SCALE, cnt,
                              max_sel, sm_scale, out, workspace, workspace_bytes, stream);
}

namespace {
// The path a decode step takes.  One fused launch when there are more
// (sequence, KV head) pairs than half the CUs.  With fewer pairs the
// attention splits each pair over several workgroups, and the selection
// either runs one workgroup per pair (sas_gate_topk's kernel) or, for block
// tables over 1,024 blocks (where one workgroup would score in several
// passes of 512 candidates), splits each pair's candidates over several
// workgroups (sliced selection: gate queries, slices, then one launch that
// merges the slices' lists and attends).
int step_path(const sas_shape *shape, int32_t budget_tokens, int32_t path) {
  if (path != SAS_STEP_AUTO) return path;
  const int n_sel = budget_tokens / SAS_BLOCK;
  const bool fits = sas::step_fits(shape->n_q_heads / shape->n_kv_heads, shape->max_blocks, n_sel);
  if (!fits) return SAS_STEP_TWO_LAUNCHES;
  if (sas::decode_split(shape->batch, shape->n_kv_heads, n_sel, device_cus()).wg_per_unit == 1) return SAS_STEP_FUSED;
  // few pairs: every workgroup of a split pair repeats the pair's selection,
  // which is cheap up to two score passes of 512 candidates
  return shape->max_blocks > 1024 ? SAS_STEP_SLICED : SAS_STEP_FUSED;
}

struct StepWorkspace {
  size_t part_o, part_ml, scores, gq, cand_key, cand_blk, cand_page, total;  // byte offsets and size
};
StepWorkspace step_workspace(const sas_shape *shape, int32_t budget_tokens, int path) {
  StepWorkspace w{};
  const int n_sel = budget_tokens / SAS_BLOCK;
  const DecodeWorkspace d = decode_workspace(shape, n_sel);
  if (path == SAS_STEP_FUSED) {  // the partials of pairs split over several workgroups
    if (sas::decode_split(shape->batch, shape->n_kv_heads, n_sel, device_cus()).wg_per_unit > 1) {
      w.part_o = d.part_o;
      w.part_ml = d.part_ml;
      w.total = d.total;
    }
    return w;
  }
  w.part_o = d.part_o;
  w.part_ml = d.part_ml;
  w.scores = d.total;  // room for the scores when the caller passes none
  w.total = w.scores + align256((size_t)shape->batch * shape->n_kv_heads * shape->max_blocks * sizeof(float));
  if (path == SAS_STEP_SLICED) {
    int slices, slice_len;
    sas::gate_slice_layout(shape->batch, shape->n_kv_heads, shape->max_blocks, device_cus(), &slices, &slice_len);
    const size_t entries = (size_t)shape->batch * shape->n_kv_heads * slices * n_sel;
    w.gq = w.total;
    w.cand_key = w.gq + align256((size_t)shape->batch * shape->n_q_heads * SAS_GATE_DIM * sizeof(float));
    w.cand_blk = w.cand_key + align256(entries * sizeof(uint32_t));
    w.cand_page = w.cand_blk + align256(entries * sizeof(int32_t));
    w.total = w.cand_page + align256(entries * sizeof(int32_t));
  }
  return w;
}
}  // namespace

size_t sas_decode_step_workspace_bytes(const sas_shape *shape, int32_t budget_tokens, int32_t path) {
  if (!shape || shape->batch <= 0 || shape->n_kv_heads <= 0 || shape->n_q_heads <= 0 || shape->max_blocks <= 0 ||
      budget_tokens < SAS_BLOCK || shape->n_q_heads % shape->n_kv_heads)
    return 0;
  if (path < SAS_STEP_AUTO || path > SAS_STEP_SLICED) return 0;
  return step_workspace(shape, budget_tokens, step_path(shape, budget_tokens, path)).total;
}

}  // extern "C"

namespace {
// The decode step on a given workspace.  ws_fixed: the workspace is the
// no-allocation entry point's scratch array (size ws_bytes), so a shortfall
// is reported as that array's limit.
sas_status decode_step_impl(const sas_shape *shape, const void *q, const void *w_q, const float *w_qnorm,
                            const void *gate_keys, const void *k_pool, const void *v_pool, const int32_t *block_table,
                            const int32_t *seq_lens, double rope_theta, int32_t budget_tokens, int32_t aggregate,
                            int32_t gated, int32_t gate_mode, float sm_scale, int32_t path, int32_t *sel,
                            float *gates, int32_t *cnt, float *scores, void *out, void *workspace,
                            size_t workspace_bytes, bool ws_fixed, void *stream) {
  if (path < SAS_STEP_AUTO || path > SAS_STEP_SLICED) return fail(SAS_ERR_INVALID_ARG, "unknown step path %d", path);
  if (gated != 0 && gated != 1) return fail(SAS_ERR_INVALID_ARG, "gated must be 0 or 1");
  if (gated && !gates) return fail(SAS_ERR_INVALID_ARG, "gated attention needs the gates output");
  sas::StepParams p;
  sas_status st = gate_params(shape, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, rope_theta, budget_tokens,
                              aggregate, sel, gates, cnt, scores, true, p.g);
  if (st) return st;
  const int32_t n_sel = budget_tokens / SAS_BLOCK;
  st = decode_params(shape, q, k_pool, v_pool, block_table, seq_lens, sel, gated ? gates : nullptr, gate_mode, cnt,
                     n_sel, sm_scale, out, p.d);
  if (st) return st;
  const hipStream_t hs = (hipStream_t)stream;
  const int how = step_path(shape, budget_tokens, path);
  if (how != SAS_STEP_TWO_LAUNCHES && !sas::step_fits(p.g.group, shape->max_blocks, n_sel))
    return fail(SAS_ERR_UNSUPPORTED, "shape outside the one-workgroup selection's limits");
  const StepWorkspace wl = step_workspace(shape, budget_tokens, how);
  if (how == SAS_STEP_FUSED && p.d.wg_per_unit == 1)  // one workgroup per (sequence, KV head), no workspace
    return hip_status(sas::launch_step(p, shape->batch, hs), "sas_decode_step launch");
  if (!workspace) return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(workspace)) return fail(SAS_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (workspace_bytes < wl.total) {
    if (ws_fixed)
      return fail(SAS_ERR_WORKSPACE,
                  "this step needs %zu bytes of scratch; sas_decode_step_noalloc holds at most %zu (use "
                  "sas_decode_step with a caller workspace)",
                  wl.total, workspace_bytes);
    return fail(SAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, wl.total);
  }
  char *ws = (char *)workspace;
  p.d.part_o = (float *)(ws + wl.part_o);
  p.d.part_ml = (float *)(ws + wl.part_ml);
  if (!p.g.scores && how != SAS_STEP_FUSED) p.g.scores = (float *)(ws + wl.scores);  // the fused kernel can skip them
  hipError_t e;
  if (how == SAS_STEP_FUSED) {
    e = sas::launch_step(p, shape->batch, hs);
  } else if (how == SAS_STEP_SLICED) {
    sas::gate_slice_layout(shape->batch, shape->n_kv_heads, shape->max_blocks, device_cus(), &p.g.slices, &p.g.slice_len);
    p.g.slot_len = ((p.g.slice_len > 512 ? p.g.slice_len : 512) + 7) / 8 * 8;
    p.g.batch = shape->batch;
    p.g.gq = (float *)(ws + wl.gq);
    p.g.cand_key = (uint32_t *)(ws + wl.cand_key);
    p.g.cand_blk = (int32_t *)(ws + wl.cand_blk);
    p.g.cand_page = (int32_t *)(ws + wl.cand_page);
    e = sas::launch_gate_query(p.g, hs);
    if (e == hipSuccess) e = sas::launch_gate_slices(p.g, shape->batch, hs);
    if (e == hipSuccess) e = sas::launch_select_decode(p, shape->batch, hs);
  } else {
    e = sas::launch_gate_topk(p.g, shape->batch, hs);
    if (e == hipSuccess) e = sas::launch_decode(p.d, shape->batch, hs);
  }
  return hip_status(e, "sas_decode_step launch");
}

// Scratch of sas_decode_step_noalloc: one copy per device, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns, taken once per device with that device current.
static __device__ __attribute__((aligned(256))) uint8_t scratch[SAS_NOALLOC_SCRATCH_BYTES];
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

sas_status scratch_of_current_device(void **out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SAS_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (es != hipSuccess || !p) return hip_status(es != hipSuccess ? es : hipErrorInvalidSymbol,
                                                    "hipGetSymbolAddress(scratch)");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SAS_OK;
}
}  // namespace

extern "C" {

sas_status sas_decode_step(const sas_shape *shape, const void *q, const void *w_q, const float *w_qnorm,
                           const void *gate_keys, const void *k_pool, const void *v_pool,
                           const int32_t *block_table, const int32_t *seq_lens, double rope_theta,
                           int32_t budget_tokens, int32_t aggregate, int32_t gated, int32_t gate_mode, float sm_scale,
                           int32_t path, int32_t *sel, float *gates, int32_t *cnt, float *scores, void *out,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return decode_step_impl(shape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, rope_theta,
                          budget_tokens, aggregate, gated, gate_mode, sm_scale, path, sel, gates, cnt, scores, out,
                          workspace, workspace_bytes, false, stream);
}

sas_status sas_decode_step_noalloc(const sas_shape *shape, const void *q, const void *w_q, const float *w_qnorm,
                                   const void *gate_keys, const void *k_pool, const void *v_pool,
                                   const int32_t *block_table, const int32_t *seq_lens, double rope_theta,
                                   int32_t budget_tokens, int32_t aggregate, int32_t gated, int32_t gate_mode,
                                   float sm_scale, int32_t path, int32_t *sel, float *gates, int32_t *cnt,
                                   float *scores, void *out, void *stream) {
  void *ws = nullptr;
  const sas_status st = scratch_of_current_device(&ws);
  if (st) return st;
  return decode_step_impl(shape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, rope_theta,
                          budget_tokens, aggregate, gated, gate_mode, sm_scale, path, sel, gates, cnt, scores, out,
                          ws, SAS_NOALLOC_SCRATCH_BYTES, true, stream);
}

namespace {
struct BackwardWorkspace {
  size_t du_q, dwqn, du_k, dwkn, pool, part, total;
};
BackwardWorkspace backward_workspace(const sas_shape *sh, int32_t max_sel) {
  const size_t q_rows = (size_t)sh->batch * sh->n_q_heads * SAS_GATE_DIM * sizeof(float);
  const size_t unit_rows = (size_t)sh->batch * sh->n_kv_heads * SAS_GATE_DIM * sizeof(float);
  const size_t k_slots = (size_t)sh->batch * sh->n_kv_heads * max_sel;
  BackwardWorkspace w;
  w.du_q = 0;
  w.dwqn = w.du_q + align256(q_rows);
  w.du_k = w.dwqn + align256(unit_rows);
  w.dwkn = w.du_k + align256(k_slots * SAS_GATE_DIM * sizeof(float));
  w.pool = w.dwkn + align256(unit_rows);
  w.part = w.pool + align256(k_slots * 3 * SAS_HEAD_DIM * sizeof(float));
  w.total = w.part + align256((size_t)sh->n_kv_heads * 12 * sas::kSplitK * 64 * 64 * sizeof(float));
  return w;
}
}  // namespace

size_t sas_gate_backward_workspace_bytes(const sas_shape *shape, int32_t max_sel) {
  if (!shape || shape->batch <= 0 || shape->n_kv_heads <= 0 || shape->n_q_heads <= 0 || max_sel <= 0) return 0;
  return backward_workspace(shape, max_sel).total;
}

sas_status sas_gate_backward(const sas_shape *shape, const void *q, const void *k_pool, const void *v_pool,
                             const int32_t *block_table, const int32_t *seq_lens, const int32_t *sel,
                             const float *gates, const int32_t *cnt, int32_t max_sel, float sm_scale,
                             const void *w_q, const float *w_qnorm, const void *w_k, const float *w_knorm,
                             const void *gate_keys, double rope_theta, const void *d_out, float *d_gates,
                             float *d_w_q, float *d_w_qnorm, float *d_w_k, float *d_w_knorm, void *workspace,
                             size_t workspace_bytes, void *stream) {
  sas_status st = check_shape(shape, true);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !sel || !gates || !cnt || !w_q || !w_qnorm || !w_k ||
      !w_knorm || !gate_keys || !d_out || !d_gates || !d_w_q || !d_w_qnorm || !d_w_k || !d_w_knorm || !workspace)
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (max_sel <= 0 || max_sel > sas::kMaxSelBackward) return fail(SAS_ERR_INVALID_ARG, "max_sel must be in 1..256");
  if (!(sm_scale > 0.f)) return fail(SAS_ERR_INVALID_ARG, "sm_scale must be positive");
  if (!(rope_theta > 1.0)) return fail(SAS_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(d_out) || !aligned16(w_q) ||
      !aligned16(w_k) || !aligned16(workspace))
    return fail(SAS_ERR_UNSUPPORTED, "q, k_pool, v_pool, d_out, w_q, w_k and workspace must be 16-byte aligned");
  const BackwardWorkspace wl = backward_workspace(shape, max_sel);
  if (workspace_bytes < wl.total)
    return fail(SAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, wl.total);
  sas::BackwardParams p;
  p.q = (const uint16_t *)q;
  p.k_pool = (const uint16_t *)k_pool;
  p.v_pool = (const uint16_t *)v_pool;
  p.d_out = (const uint16_t *)d_out;
  p.gate_keys = (const uint16_t *)gate_keys;
  p.w_q = (const uint16_t *)w_q;
  p.w_k = (const uint16_t *)w_k;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.sel = sel;
  p.cnt = cnt;
  p.gates = gates;
  p.w_qnorm = w_qnorm;
  p.w_knorm = w_knorm;
  p.d_gates = d_gates;
  p.d_w_q = d_w_q;
  p.d_w_qnorm = d_w_qnorm;
  p.d_w_k = d_w_k;
  p.d_w_knorm = d_w_knorm;
  char *ws = (char *)workspace;
  p.ws_du_q = (float *)(ws + wl.du_q);
  p.ws_dwqn = (float *)(ws + wl.dwqn);
  p.ws_du_k = (float *)(ws + wl.du_k);
  p.ws_dwkn = (float *)(ws + wl.dwkn);
  p.ws_pool = (float *)(ws + wl.pool);
  p.ws_part = (float *)(ws + wl.part);
  p.page_stride = shape->page_stride;
  p.tok_stride = shape->tok_stride;
  p.head_stride = shape->head_stride;
  p.batch = shape->batch;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.group = shape->n_q_heads / shape->n_kv_heads;
  p.max_blocks = shape->max_blocks;
  p.max_sel = max_sel;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  for (int i = 0; i < SAS_GATE_DIM / 2; ++i) p.inv_freq[i] = pow(rope_theta, -(double)i / (SAS_GATE_DIM / 2));
  return hip_status(sas::launch_gate_backward(p, (hipStream_t)stream), "sas_gate_backward launch");
}


namespace {
struct PrefillBackwardWorkspace {
  size_t dgp, ghat, a, du_q, dwqn, pool, dgk, du_k, dwkn, part, total;
  int n_hist, a_cols, key_chunks, head_groups, n_qblocks;
};
PrefillBackwardWorkspace prefill_backward_workspace(const sas_shape *sh, int32_t seq_len, int32_t max_sel) {
  PrefillBackwardWorkspace w;
  const size_t T = (size_t)seq_len, Hq = (size_t)sh->n_q_heads, Hkv = (size_t)sh->n_kv_heads, f = sizeof(float);
  w.n_qblocks = (seq_len + SAS_BLOCK - 1) / SAS_BLOCK;
  w.n_hist = (seq_len - 1) / SAS_BLOCK;
  w.a_cols = (w.n_hist + 63) / 64 * 64;
  w.key_chunks = (w.n_hist + sas::kChainBlocks - 1) / sas::kChainBlocks;
  const int hw = sas::prefill_heads_per_wave(sh->n_q_heads / sh->n_kv_heads);
  w.head_groups = (sh->n_q_heads / sh->n_kv_heads + hw - 1) / hw;
  const size_t tiles = Hq + Hkv * (size_t)((w.a_cols + 127) / 128);  // 128 x 128 partial tiles
  w.dgp = 0;
  w.ghat = w.dgp + align256((size_t)w.head_groups * T * Hkv * max_sel * f);
  w.a = w.ghat + align256(Hkv * T * SAS_GATE_DIM * f);
  w.du_q = w.a + align256(Hkv * T * (size_t)w.a_cols * f);
  w.dwqn = w.du_q + align256(T * Hq * SAS_GATE_DIM * f);
  w.pool = w.dwqn + align256((size_t)w.n_qblocks * Hkv * SAS_GATE_DIM * f);
  w.dgk = w.pool + align256(Hkv * (size_t)w.n_hist * 3 * SAS_HEAD_DIM * f);
  w.du_k = w.dgk + align256(Hkv * (size_t)w.a_cols * SAS_GATE_DIM * f);
  w.dwkn = w.du_k + align256(Hkv * (size_t)w.n_hist * SAS_GATE_DIM * f);
  w.part = w.dwkn + align256(Hkv * (size_t)w.key_chunks * SAS_GATE_DIM * f);
  w.total = w.part + align256(tiles * sas::kPrefillSplit * 128 * 128 * f);
  return w;
}
}  // namespace

size_t sas_prefill_gate_backward_workspace_bytes(const sas_shape *shape, int32_t seq_len, int32_t max_sel) {
  if (!shape || shape->n_kv_heads <= 0 || shape->n_q_heads <= 0 || shape->n_q_heads % shape->n_kv_heads ||
      seq_len < 1 || max_sel <= 0)
    return 0;
  return prefill_backward_workspace(shape, seq_len, max_sel).total;
}

sas_status sas_prefill_gate_backward(const sas_shape *shape, const void *q, const void *k_pool, const void *v_pool,
                                     const int32_t *block_table_row, int32_t seq_len, const int32_t *sel,
                                     const float *gates, const int32_t *cnt, int32_t max_sel, float sm_scale,
                                     const float *lse, const void *w_q, const float *w_qnorm, const void *w_k,
                                     const float *w_knorm, const void *gate_keys, double rope_theta,
                                     const void *d_out, float *d_gates, float *d_w_q, float *d_w_qnorm, float *d_w_k,
                                     float *d_w_knorm, void *workspace, size_t workspace_bytes, void *stream) {
  sas_status st = check_prefill(shape, true, seq_len);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !block_table_row || !sel || !gates || !cnt || !lse || !w_q || !w_qnorm || !w_k ||
      !w_knorm || !gate_keys || !d_out || !d_gates || !d_w_q || !d_w_qnorm || !d_w_k || !d_w_knorm || !workspace)
    return fail(SAS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (max_sel <= 0) return fail(SAS_ERR_INVALID_ARG, "max_sel must be positive");
  if (max_sel > 64) return fail(SAS_ERR_UNSUPPORTED, "max_sel %d exceeds 64 (budgets above 4,096 tokens)", max_sel);
  if (!(sm_scale > 0.f)) return fail(SAS_ERR_INVALID_ARG, "sm_scale must be positive");
  if (!(rope_theta > 1.0)) return fail(SAS_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(d_out) || !aligned16(w_q) ||
      !aligned16(w_k) || !aligned16(gate_keys) || !aligned16(workspace))
    return fail(SAS_ERR_UNSUPPORTED,
                "q, k_pool, v_pool, d_out, w_q, w_k, gate_keys and workspace must be 16-byte aligned");
  const PrefillBackwardWorkspace wl = prefill_backward_workspace(shape, seq_len, max_sel);
  if (workspace_bytes < wl.total)
    return fail(SAS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, wl.total);
  sas::PrefillBackwardParams p;
  p.q = (const uint16_t *)q;
  p.k_pool = (const uint16_t *)k_pool;
  p.v_pool = (const uint16_t *)v_pool;
  p.d_out = (const uint16_t *)d_out;
  p.gate_keys = (const uint16_t *)gate_keys;
  p.w_q = (const uint16_t *)w_q;
  p.w_k = (const uint16_t *)w_k;
  p.block_table = block_table_row;
  p.sel = sel;
  p.cnt = cnt;
  p.gates = gates;
  p.lse = lse;
  p.w_qnorm = w_qnorm;
  p.w_knorm = w_knorm;
  p.d_gates = d_gates;
  p.d_w_q = d_w_q;
  p.d_w_qnorm = d_w_qnorm;
  p.d_w_k = d_w_k;
  p.d_w_knorm = d_w_knorm;
  char *ws = (char *)workspace;
  p.ws_dgp = (float *)(ws + wl.dgp);
  p.ws_ghat = (float *)(ws + wl.ghat);
  p.ws_a = (float *)(ws + wl.a);
  p.ws_du_q = (float *)(ws + wl.du_q);
  p.ws_dwqn = (float *)(ws + wl.dwqn);
  p.ws_pool = (float *)(ws + wl.pool);
  p.ws_dgk = (float *)(ws + wl.dgk);
  p.ws_du_k = (float *)(ws + wl.du_k);
  p.ws_dwkn = (float *)(ws + wl.dwkn);
  p.ws_part = (float *)(ws + wl.part);
  p.page_stride = shape->page_stride;
  p.tok_stride = shape->tok_stride;
  p.head_stride = shape->head_stride;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.group = shape->n_q_heads / shape->n_kv_heads;
  p.head_groups = wl.head_groups;
  p.max_sel = max_sel;
  p.seq_len = seq_len;
  p.n_qblocks = wl.n_qblocks;
  p.n_hist = wl.n_hist;
  p.a_cols = wl.a_cols;
  p.key_chunks = wl.key_chunks;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  for (int i = 0; i < SAS_GATE_DIM / 2; ++i) p.inv_freq[i] = pow(rope_theta, -(double)i / (SAS_GATE_DIM / 2));
  return hip_status(sas::launch_prefill_gate_backward(p, (hipStream_t)stream), "sas_prefill_gate_backward launch");
}

}  // extern "C"
