/*
 * sas.h -- C ABI of libsas, the MI355X (gfx950) SAS sparse-decode library.
 *
 * Simple-Attention-Sparsification (SAS) decodes with attention over a learned
 * choice of 64-token KV blocks ("Tencent released Simple-Attention-
 * Sparsification ...", aigc.news, the paragraph listing the sparse-attention
 * setup; "Specifications and Configuration Table" of the localmodelwatch
 * model page): each key block is pooled (max + min + average) into a 128-wide
 * gate key with Q/K normalisation and gate RoPE; a query projection (Qproj)
 * of the decode query scores the blocks; a Top-K keeps 31 historical blocks
 * plus the local block for the default 2,048-token budget (1,024 / 4,096
 * tokens also, without retraining); attention then reads only those blocks,
 * optionally scaled by continuous gates on the selected blocks.
 *
 * Calls, in serving order:
 *   sas_pool_blocks    once per newly completed 64-token block   (pooling)
 *   sas_append_kv      once per decode step: the new token's K/V rows into
 *                      the cache, pooling each block this completes
 *                      (cache write fused with incremental pooling)
 *   sas_gate_topk      once per decode step                      (selection)
 *   sas_sparse_decode  once per decode step                      (attention)
 *   sas_decode_step    the two above as one call (one fused launch)
 * and, for the training-time forward of a whole sequence (every position a
 * query): sas_prefill_select, then sas_prefill_attend; for training the
 * gates: sas_gate_backward after a gated decode step, or
 * sas_prefill_gate_backward after the training-time forward.
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller (for
 *     example a torch tensor's data_ptr()), except `shape`, which is a host
 *     pointer read during the call.  The library never allocates, frees or
 *     copies between host and device, and never synchronises: each call only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns.
 *   - bf16 tensors hold IEEE bfloat16 bit patterns; all arithmetic inside is
 *     fp32 (MFMA bf16 x bf16 -> fp32 for the attention tiles); results
 *     rounded to bf16 use round-to-nearest-even.
 *   - head_dim = gate_dim = 128 and block = 64 tokens are fixed.
 *   - Arguments are checked on the host before anything is launched; a failed
 *     check launches nothing, leaves every output untouched and returns a
 *     non-zero sas_status.  Device-resident values (sequence lengths, block
 *     table entries, selections) are trusted: they must be in range.
 *   - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Calls are thread-safe; sas_last_error() is per host thread.
 */
#ifndef SAS_H
#define SAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAS_HEAD_DIM 128
#define SAS_GATE_DIM 128
#define SAS_BLOCK 64
#define SAS_MAX_GROUP 16       /* n_q_heads / n_kv_heads */
#define SAS_MAX_BLOCKS 16384   /* blocks per sequence (1,048,576 tokens) */

typedef int32_t sas_status;
enum {
  SAS_OK = 0,
  SAS_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad budget or stride */
  SAS_ERR_UNSUPPORTED = 2, /* outside the supported envelope (group > 16, misaligned, ...) */
  SAS_ERR_WORKSPACE = 3,   /* workspace too small */
  SAS_ERR_HIP = 4          /* a HIP launch failed; detail in sas_last_error() */
};

/*
 * Shape of one attention layer's decode batch and of its paged KV pools.
 * K/V element (page p, kv head h, token-in-block t, dim d) lives at
 *   pool[p * page_stride + h * head_stride + t * tok_stride + d]   (elements).
 *   head-major pages [P][Hkv][64][128]:  (Hkv*64*128, 128, 64*128)
 *   contiguous cache [B][L][Hkv][128] with block_table[s][c] = s*max_blocks+c:
 *                                       (64*Hkv*128, Hkv*128, 128)
 * Strides must be multiples of 8 elements and pools 16-byte aligned.
 */
typedef struct {
  int32_t batch;       /* B: sequences in the decode batch */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; Hq % Hkv == 0, Hq / Hkv <= 16 */
  int32_t max_blocks;  /* columns of block_table, <= SAS_MAX_BLOCKS */
  int64_t page_stride, tok_stride, head_stride;
} sas_shape;

/*
 * sas_pool_blocks -- key-block pooling into gate keys: pooling by max, min and
 * average, a 128-wide gate space, Q/K normalisation and gate RoPE (settings
 * table of the localmodelwatch model page; aigc.news release note).
 *
 * For each listed pair i (s = pool_seq[i], c = pool_blk[i]) and every KV head
 * h, over the 64 cached keys of block c (all 64 rows must be written):
 *   p  = [max_t k_t | min_t k_t | mean_t k_t]                     (384 values)
 *   u[j] = sum_i w_k[h][j][i] * p[i]      w_k: bf16 [Hkv][128][384], no bias
 *                                         (output-major, a Linear weight)
 *   n  = u / sqrt(mean(u^2) + 1e-6) * w_knorm                    (RMSNorm)
 *   gk = RoPE(n, position 64*c, rope_theta)   rotate-half pairs (i, i+64),
 *        angle position * rope_theta^(-i/64)
 *   gate_keys[block_table[s][c]][h][:] = bf16(gk)         bf16 [P][Hkv][128]
 * n == 0 is a no-op returning SAS_OK.  pool_seq / pool_blk: int32 [n].
 */
sas_status sas_pool_blocks(const sas_shape *shape, const void *k_pool, const int32_t *block_table,
                           const int32_t *pool_seq, const int32_t *pool_blk, int32_t n,
                           const void *w_k, const float *w_knorm, double rope_theta,
                           void *gate_keys, void *stream);

/*
 * sas_append_kv -- one decode step's cache write fused with incremental
 * pooling (the 64-token KV blocks and their max + min + average pooling of the
 * release note and settings table; when a block is pooled is not stated: here
 * it is pooled by the step that writes its last row).
 *
 * For every sequence s, with L = seq_lens[s] >= 1 its length counting the new
 * token (the token's position is L-1), and every KV head h:
 *   k_pool[row of token L-1, head h][:] = k_new[s][h][:]
 *   v_pool[row of token L-1, head h][:] = v_new[s][h][:]
 * and, when L % 64 == 0, the gate key of block L/64 - 1 (head h) is computed
 * and stored exactly as sas_pool_blocks computes it (bit-identical), with
 * the same w_k, w_knorm and rope_theta conventions.
 * k_new, v_new: bf16 [B][Hkv][128], 16-byte aligned.  Rows are written at
 * block_table[s][(L-1)/64]; distinct sequences must not share that page.
 * Everything else in the pools and in gate_keys is left as it is.
 */
sas_status sas_append_kv(const sas_shape *shape, const void *k_new, const void *v_new, void *k_pool,
                         void *v_pool, const int32_t *block_table, const int32_t *seq_lens,
                         const void *w_k, const float *w_knorm, double rope_theta, void *gate_keys,
                         void *stream);

/*
 * sas_gate_topk -- gate scores and per-KV-head Top-K block selection: the
 * Qproj query projection, a Top-K of 31 historical blocks at the default
 * 2,048-token budget (1,024 / 4,096 also), and a continuous gate per selected
 * block (aigc.news release note; localmodelwatch settings table).
 *
 * For sequence s with L = seq_lens[s] >= 1 cached tokens (the current token
 * included) the local block is l = (L-1)/64 and the candidates are c < l.
 *   gate query, per query head h: RoPE(RMSNorm(u) * w_qnorm, position L-1)
 *       with u[j] = sum_d w_q[h][j][d] * q[s][h][d]
 *                                 w_q: bf16 [Hq][128][128] output-major, no bias
 *   score of c for KV head k: mean over k's query heads of
 *       <gate query, gate_keys[block_table[s][c]][k]> / sqrt(128)
 *   Top-K: the min(budget/64 - 1, l) best candidates under (score descending,
 *       block index ascending; NaN ranks lowest, -0 == +0), then the local
 *       block.
 * Outputs ([B][Hkv][budget/64] unless noted; the selection ascending, the
 * local block last, padded with -1 / 0):
 *   sel    int32  selected block indices
 *   gates  fp32   sigmoid(score) per selected historical block (a NaN
 *                 score counts as -inf here too: gate 0), 1 for the local
 *                 block (nullable: not written)
 *   cnt    int32  [B][Hkv] number of selected blocks (>= 1)
 *   scores fp32   [B][Hkv][max_blocks] block scores (entries c >= l are -inf)
 * budget_tokens: a positive multiple of 64, at most 64 * 256.
 */
sas_status sas_gate_topk(const sas_shape *shape, const void *q, const void *w_q,
                         const float *w_qnorm, const void *gate_keys, const int32_t *block_table,
                         const int32_t *seq_lens, double rope_theta, int32_t budget_tokens,
                         int32_t *sel, float *gates, int32_t *cnt, float *scores, void *stream);

/*
 * sas_sparse_decode -- block-sparse flash-decode over the selected blocks
 * (the pages' block-sparse decoding within the token budget).
 *
 * For query head h of sequence s (KV head k = h / G) over the tokens j of the
 * cnt[s][k] blocks sel[s][k][:] with j <= L-1:
 *   z_j = sm_scale * <q[s][h], K_j>,   P = softmax(z) over those tokens
 *   plain mode (gates == NULL):  out = sum_j P_j V_j
 *   gated mode:                  out = sum_j gates[s][k][i(j)] * P_j V_j
 *       (each selected block's contribution scaled by its gate; P normalised
 *        over the whole selection)
 * q: bf16 [B][Hq][128]; out: bf16 [B][Hq][128]; sel / gates: [B][Hkv][max_sel]
 * as written by sas_gate_topk with max_sel = budget/64; cnt: [B][Hkv].
 * workspace: device scratch of at least
 * sas_sparse_decode_workspace_bytes(shape, max_sel) bytes (partial results
 * when a (sequence, KV head) is split across workgroups; no initial contents
 * needed).  Calls that overlap in time must not share a workspace.  The split,
 * and so the size, follows the compute-unit count of the device current at
 * the call (read once per device and cached; 256 when no device is visible).
 */
size_t sas_sparse_decode_workspace_bytes(const sas_shape *shape, int32_t max_sel);
sas_status sas_sparse_decode(const sas_shape *shape, const void *q, const void *k_pool,
                             const void *v_pool, const int32_t *block_table,
                             const int32_t *seq_lens, const int32_t *sel, const float *gates,
                             const int32_t *cnt, int32_t max_sel, float sm_scale, void *out,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Alternative readings, as options of the decode calls.  The pages say that
 * one selection serves a KV head (per-KV-head Top-K) and that continuous gates
 * sit on the selected blocks, but not how a group of query heads makes one
 * score nor how a gate enters attention.  The calls above use the mean of
 * the group's per-head scores and scale each selected block's share of the
 * output by its gate; these variants take the other plain readings:
 *   aggregate  SAS_AGG_MEAN  mean of the group's per-head scores (default)
 *              SAS_AGG_MAX   their maximum (group of at most 8 query heads)
 *   gate_mode  SAS_GATE_SCALE  out = sum_j g(j) P_j V_j, P the softmax over
 *                              the selection (default)
 *              SAS_GATE_LOGIT  out = sum_j P'_j V_j, P' the softmax over the
 *                              selection of z_j + log g(j) (a log-gate bias)
 * g(j) is the gate of token j's block.  Otherwise identical to sas_gate_topk
 * and sas_sparse_decode (gate_mode is ignored when gates is NULL).
 */
#define SAS_AGG_MEAN 0
#define SAS_AGG_MAX 1
#define SAS_GATE_SCALE 0
#define SAS_GATE_LOGIT 1
sas_status sas_gate_topk_ex(const sas_shape *shape, const void *q, const void *w_q,
                            const float *w_qnorm, const void *gate_keys, const int32_t *block_table,
                            const int32_t *seq_lens, double rope_theta, int32_t budget_tokens,
                            int32_t aggregate, int32_t *sel, float *gates, int32_t *cnt, float *scores,
                            void *stream);
sas_status sas_sparse_decode_ex(const sas_shape *shape, const void *q, const void *k_pool,
                                const void *v_pool, const int32_t *block_table,
                                const int32_t *seq_lens, const int32_t *sel, const float *gates,
                                int32_t gate_mode, const int32_t *cnt, int32_t max_sel,
                                float sm_scale, void *out, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * sas_decode_step -- the whole decode step, selection then attention: the
 * outputs of sas_gate_topk_ex followed by sas_sparse_decode_ex on the same
 * arguments (the pages' learned block selection and block-sparse decoding
 * within the token budget; aigc.news release note, "Tencent Hunyuan
 * open-sources SAS ...").
 *
 * Paths (all give the same selection; fused and two-launch outputs are the
 * same bits whenever the attention runs one workgroup per pair):
 *   SAS_STEP_FUSED  one kernel launch: each (sequence, KV head) is scored,
 *                   selected and attended by one workgroup, which keeps the
 *                   selection and the selected blocks' pages on chip; with
 *                   fewer pairs than the device's compute units, by several
 *                   workgroups that each make the pair's selection and attend
 *                   a share of its blocks, plus a launch that merges their
 *                   partial results;
 *   SAS_STEP_SLICED for few pairs: each pair's candidates are scored and
 *                   reduced to a Top-K list by several workgroups (slices),
 *                   then one launch merges the lists into the selection and
 *                   attends with each pair split over several workgroups;
 *   SAS_STEP_TWO_LAUNCHES  the kernels of the two calls above;
 *   SAS_STEP_AUTO   sliced for fewer pairs than the current device's
 *                   compute units and block tables over 1,024 blocks, else
 *                   fused (two launches where the fused kernel's limits
 *                   are exceeded).
 *
 * Arguments as for the two calls, with max_sel = budget_tokens / 64:
 *   aggregate  SAS_AGG_MEAN or SAS_AGG_MAX
 *   gated      0: plain Top-K attention; 1: gated attention (gate_mode
 *              SAS_GATE_SCALE or SAS_GATE_LOGIT), which needs `gates`
 *   gates      written when non-NULL (nullable when gated == 0)
 *   scores     written when non-NULL (nullable)
 *   sel, cnt, out  required
 * workspace: at least sas_decode_step_workspace_bytes(shape, budget_tokens,
 * path) bytes (0 on the fused path when every pair has one workgroup, where
 * workspace may be NULL; 0 also for an unknown path); no initial contents
 * needed; calls that overlap in time must not share one.
 */
#define SAS_STEP_AUTO 0
#define SAS_STEP_FUSED 1
#define SAS_STEP_TWO_LAUNCHES 2
#define SAS_STEP_SLICED 3
size_t sas_decode_step_workspace_bytes(const sas_shape *shape, int32_t budget_tokens, int32_t path);
sas_status sas_decode_step(const sas_shape *shape, const void *q, const void *w_q,
                           const float *w_qnorm, const void *gate_keys, const void *k_pool,
                           const void *v_pool, const int32_t *block_table,
                           const int32_t *seq_lens, double rope_theta, int32_t budget_tokens,
                           int32_t aggregate, int32_t gated, int32_t gate_mode, float sm_scale,
                           int32_t path, int32_t *sel, float *gates, int32_t *cnt, float *scores,
                           void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sas_decode_step_noalloc -- sas_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments, outputs and bits
 * without `workspace`.  The library's own scratch array stands in for it: a
 * file-scope device array of SAS_NOALLOC_SCRATCH_BYTES per device (held by
 * each device the library runs on until the process ends; its address is
 * taken once per device, on the first call with that device current).  The
 * call itself allocates nothing.  A step that would need a larger workspace
 * (sas_decode_step_workspace_bytes over the limit; the fused path needs
 * none) fails with SAS_ERR_WORKSPACE and launches nothing.  Every call on a
 * device shares that device's one array and leaves the last call's partial
 * results in it: calls that overlap in time on one device (two streams, two
 * host threads) race and must not be issued; sequential calls on one stream
 * are safe.  Nothing in the array needs initial contents.
 */
#define SAS_NOALLOC_SCRATCH_BYTES (16u << 20)
sas_status sas_decode_step_noalloc(const sas_shape *shape, const void *q, const void *w_q,
                                   const float *w_qnorm, const void *gate_keys, const void *k_pool,
                                   const void *v_pool, const int32_t *block_table,
                                   const int32_t *seq_lens, double rope_theta, int32_t budget_tokens,
                                   int32_t aggregate, int32_t gated, int32_t gate_mode, float sm_scale,
                                   int32_t path, int32_t *sel, float *gates, int32_t *cnt, float *scores,
                                   void *out, void *stream);

/*
 * Training-time forward of one sequence (every position is a query).  SAS
 * selects KV blocks for each query and trains with a Top-K of 31 historical
 * blocks on 32,768-token sequences (aigc.news release note; "Tencent Hunyuan
 * open-sources SAS ...": per-query block selection).  Position t (0-based,
 * T = seq_len positions) selects and attends exactly as a decode step whose
 * cache holds the first t+1 tokens: gate query at position t, candidates the
 * complete blocks c < t/64, its own block t/64 last, causal attention (keys
 * j <= t) over the selected blocks.
 *
 * shape->batch must be 1 (one sequence per call); T must fit in max_blocks
 * blocks.  q: bf16 [T][Hq][128]; block_table_row: int32 [max_blocks], the
 * sequence's pages (the K/V strides of shape address them as for decode).
 *
 * sas_prefill_select -- sas_gate_topk for every position: writes sel / gates /
 *   cnt ([T][Hkv][budget/64], [T][Hkv]) and, when scores is non-NULL, scores
 *   [T][Hkv][max_blocks], with the same definitions and conventions.
 * sas_prefill_attend -- the attention of every position over its selection:
 *   plain (gates NULL) or gated as in sas_sparse_decode, output bf16
 *   [T][Hq][128].  sel / gates / cnt as sas_prefill_select wrote them
 *   (max_sel = budget/64 <= 64, i.e. budgets up to 4,096 tokens).  lse
 *   (nullable): fp32 [T][Hq], the natural-log log-sum-exp of each query
 *   head's logits sm_scale * <q, k_j> over the tokens it attends (the plain
 *   softmax normaliser, gated or not), which sas_prefill_gate_backward
 *   takes.  Needs no workspace.
 */
sas_status sas_prefill_select(const sas_shape *shape, const void *q, const void *w_q,
                              const float *w_qnorm, const void *gate_keys,
                              const int32_t *block_table_row, int32_t seq_len, double rope_theta,
                              int32_t budget_tokens, int32_t *sel, float *gates, int32_t *cnt,
                              float *scores, void *stream);
sas_status sas_prefill_attend(const sas_shape *shape, const void *q, const void *k_pool,
                              const void *v_pool, const int32_t *block_table_row, int32_t seq_len,
                              const int32_t *sel, const float *gates, const int32_t *cnt,
                              int32_t max_sel, float sm_scale, void *out, float *lse, void *stream);

/*
 * sas_gate_backward -- gradients of the gate parameters through the
 * continuous gates of one gated decode step (default reading: each selected
 * block's share of the output scaled by its gate).  SAS's continuous gates on
 * the selected blocks give the language-model loss a differentiable path to
 * the block ranking (aigc.news release note; "Tencent Hunyuan open-sources
 * SAS ...").  The Top-K choice passes no gradient, the local block's gate is
 * the constant 1, and the bf16 gate keys pass the gradient straight through;
 * q, K and V (the frozen backbone's) get none.
 *
 * Inputs: the step's inputs and its forward outputs sel / gates / cnt (as
 * sas_gate_topk wrote them, max_sel = budget/64), the gate weights, the gate
 * keys, and d_out: bf16 [B][Hq][128], the gradient of the loss w.r.t. the
 * step's output.  Outputs (fp32, overwritten, summed over the batch):
 *   d_gates    [B][Hkv][max_sel]  dL/dg of every selected block (the local
 *              block's included, as if free), 0 in the padding
 *   d_w_q      [Hq][128][128]     d_w_qnorm [128]
 *   d_w_k      [Hkv][128][384]    d_w_knorm [128]
 * The sums over the batch run in a fixed order (deterministic).  workspace:
 * at least sas_gate_backward_workspace_bytes(shape, max_sel) bytes, no
 * initial contents needed.
 */
size_t sas_gate_backward_workspace_bytes(const sas_shape *shape, int32_t max_sel);
sas_status sas_gate_backward(const sas_shape *shape, const void *q, const void *k_pool,
                             const void *v_pool, const int32_t *block_table,
                             const int32_t *seq_lens, const int32_t *sel, const float *gates,
                             const int32_t *cnt, int32_t max_sel, float sm_scale, const void *w_q,
                             const float *w_qnorm, const void *w_k, const float *w_knorm,
                             const void *gate_keys, double rope_theta, const void *d_out,
                             float *d_gates, float *d_w_q, float *d_w_qnorm, float *d_w_k,
                             float *d_w_knorm, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * sas_prefill_gate_backward -- gradients of the gate parameters through the
 * continuous gates of the training-time forward of one sequence (the
 * backward of sas_prefill_select + gated sas_prefill_attend).  SAS trains its
 * gates with the language-model loss on 32,768-token sequences, each query
 * selecting its own blocks (aigc.news release note: training Top-K of 31
 * historical blocks; "Tencent Hunyuan open-sources SAS ...": per-query
 * selection, a differentiable path from the loss to the selector).  Position
 * t is the decode step whose cache holds its first t+1 tokens, so the loss
 * sum_t sum_h <d_out[t][h], out[t][h]> has the sum over positions of
 * sas_gate_backward's per-step gradients, under the same conventions: the
 * Top-K choice passes no gradient, each position's own block has the
 * constant gate 1, the bf16 gate keys pass the gradient straight through,
 * and q, K and V get none.  A block's key collects the gradient of every
 * position that selected it.
 *
 * shape->batch must be 1.  Inputs: q, d_out bf16 [T][Hq][128]; the pools,
 * block_table_row and seq_len as for sas_prefill_attend; sel / gates / cnt
 * as sas_prefill_select wrote them (max_sel = budget/64 <= 64); lse
 * [T][Hq] as sas_prefill_attend wrote it for these inputs; the gate weights
 * and keys as for sas_prefill_select.  Outputs (fp32, overwritten):
 *   d_gates   [T][Hkv][max_sel]  dL/dg of every selected block (the own
 *             block's included, as if free), 0 in the padding
 *   d_w_q     [Hq][128][128]     d_w_qnorm [128]
 *   d_w_k     [Hkv][128][384]    d_w_knorm [128]
 * Sums run in a fixed order (deterministic).  workspace: at least
 * sas_prefill_gate_backward_workspace_bytes(shape, seq_len, max_sel) bytes,
 * no initial contents needed; it grows as Hkv * T * T / 16 bytes (a dense
 * position x block matrix: 512 MiB at T = 32,768 with 8 KV heads) besides
 * terms linear in T.  Errors as for sas_prefill_attend, plus
 * SAS_ERR_WORKSPACE.
 */
size_t sas_prefill_gate_backward_workspace_bytes(const sas_shape *shape, int32_t seq_len, int32_t max_sel);
sas_status sas_prefill_gate_backward(const sas_shape *shape, const void *q, const void *k_pool,
                                     const void *v_pool, const int32_t *block_table_row, int32_t seq_len,
                                     const int32_t *sel, const float *gates, const int32_t *cnt,
                                     int32_t max_sel, float sm_scale, const float *lse, const void *w_q,
                                     const float *w_qnorm, const void *w_k, const float *w_knorm,
                                     const void *gate_keys, double rope_theta, const void *d_out,
                                     float *d_gates, float *d_w_q, float *d_w_qnorm, float *d_w_k,
                                     float *d_w_knorm, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * sas_probe_read -- measurement utility, not a step of the method: reads
 * n_chunks 16 KiB chunks with nothing else to do, so that the attention's
 * gather rate can be compared with a gather ceiling measured on the same
 * chunks (the attention reads each selected block of K and of V as one
 * 16 KiB chunk of a paged head-major pool).
 *   chunk_addr     device array [n_chunks] of device addresses, each
 *                  16-byte aligned, of 16,384 readable bytes (trusted, like
 *                  block tables: not checked on the host)
 *   chunks_per_wg  chunks each 256-thread workgroup reads, 1..64
 *   sink           device buffer of ceil(n_chunks / chunks_per_wg) 16-byte
 *                  words, 16-byte aligned: word w = XOR of every 16-byte
 *                  word of chunks [w * chunks_per_wg, ...) (so the reads
 *                  cannot be skipped, and a test can check them)
 * n_chunks = 0 is a no-op.  Errors: SAS_ERR_INVALID_ARG for a NULL pointer,
 * a negative count, chunks_per_wg outside 1..64, sink_bytes too small or a
 * misaligned sink.
 */
sas_status sas_probe_read(const uint64_t *chunk_addr, int32_t n_chunks, int32_t chunks_per_wg, void *sink,
                          size_t sink_bytes, void *stream);

/* Text of a status code (static storage). */
const char *sas_status_str(sas_status status);
/* Detail of the last failed call on this host thread ("" if none). */
const char *sas_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t sas_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAS_H */
