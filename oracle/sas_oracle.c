/*
 * SAS decode-path ORACLE -- test infrastructure, not product code.
 *
 * A plain, slow CPU implementation of what the SAS sparse-decode path computes,
 * written from the pages that describe Simple-Attention-Sparsification (SAS):
 *   "Tencent released Simple-Attention-Sparsification, a method for efficient
 *    sparse attention in Qwen3 models" (aigc.news, body paragraph that lists the
 *    sparse-attention setup) and the "Specifications and Configuration Table" of
 *   "Simple-Attention-Sparsification Text Generation Model: 12GB+ VRAM"
 *   (localmodelwatch, EN) and its Japanese twin.
 * Those passages fix: 64-token KV blocks, Top-K of 31 historical blocks, gate
 * hidden size 128, a query projection named Qproj, key-block pooling by
 * max + min + average, Q/K normalisation, gate RoPE, and a 2,048-token decode
 * budget (1,024 / 4,096 also usable without retraining).  Everything else is a
 * reading of those passages; each reading is named where it is used.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code with the HIP path.
 *
 * Arithmetic: every floating-point step runs in fp64 on the exact fp64 values
 * of the bf16 / fp32 inputs.  Rounded outputs are named as such.
 *
 * Parity pins (tests/test_oracle_*.py): pooling vs numpy max/min/mean, RMSNorm
 * vs torch.rms_norm, RoPE vs complex multiplication, scores/selection vs brute
 * force subset search and numpy lexsort, attention vs torch scaled-dot-product
 * attention with an explicit boolean mask, gate-parameter count vs the pages'
 * 33.0M / 42.0M.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HEAD_DIM 128   /* Qwen3 attention head dimension */
#define GATE_DIM 128   /* gate hidden size (settings table) */
#define BLOCK 64       /* KV block size in tokens (settings table) */
#define HALF_GATE (GATE_DIM / 2)
#define POOLED (3 * HEAD_DIM) /* [max | min | mean] */
#define NORM_EPS 1e-6

/* ------------------------------------------------------------------ */
/* bf16 <-> fp64 (bf16 = upper 16 bits of an IEEE binary32)            */
/* ------------------------------------------------------------------ */
static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round an fp64 value to the nearest bf16, ties to even, in one step. */
uint16_t sas_oracle_round_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  int e;
  frexp(fabs(x), &e);                 /* |x| = m * 2^e, m in [0.5, 1) */
  int ulp_exp = e - 8;                /* 8 significant bits */
  if (ulp_exp < -133) ulp_exp = -133; /* bf16 subnormal spacing */
  double r = ldexp(nearbyint(ldexp(x, -ulp_exp)), ulp_exp); /* RNE */
  const double bf16_max = 3.3895313892515355e38;            /* (2 - 2^-7) * 2^127 */
  if (fabs(r) > bf16_max) return x > 0 ? 0x7F80 : 0xFF80;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Q/K normalisation and gate RoPE                                     */
/* ------------------------------------------------------------------ */
/* READING (the pages only say that Q/K normalisation is on): RMSNorm with a
 * learned weight vector, eps 1e-6, applied after the projection. */
void sas_oracle_rms_norm(double *v, const float *w) {
  double ss = 0.0;
  for (int i = 0; i < GATE_DIM; ++i) ss += v[i] * v[i];
  double inv = 1.0 / sqrt(ss / GATE_DIM + NORM_EPS);
  for (int i = 0; i < GATE_DIM; ++i) v[i] = v[i] * inv * (double)w[i];
}

/* READING (the pages only say that a gate RoPE is on): rotate-half rotary embedding
 * over the 128-wide gate vector; pair (i, i+64) turns by pos * theta^(-i/64). */
void sas_oracle_rope(double *v, double pos, double theta) {
  for (int i = 0; i < HALF_GATE; ++i) {
    double ang = pos * pow(theta, -(double)i / HALF_GATE);
    double c = cos(ang), s = sin(ang);
    double a = v[i], b = v[i + HALF_GATE];
    v[i] = a * c - b * s;
    v[i + HALF_GATE] = b * c + a * s;
  }
}

/* ------------------------------------------------------------------ */
/* Paged KV addressing                                                 */
/* ------------------------------------------------------------------ */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, max_blocks;
  int64_t page_stride, tok_stride, head_stride; /* elements; dim stride 1 */
} oracle_shape;

static const uint16_t *kv_row(const oracle_shape *sh, const uint16_t *pool,
                              const int32_t *block_table, int s, int kvh, int tok) {
  int32_t page = block_table[(int64_t)s * sh->max_blocks + tok / BLOCK];
  return pool + (int64_t)page * sh->page_stride + (int64_t)kvh * sh->head_stride +
         (int64_t)(tok % BLOCK) * sh->tok_stride;
}

/* ------------------------------------------------------------------ */
/* Stage 1: key-block pooling -> gate key                              */
/* ------------------------------------------------------------------ */
/* Pooled statistics of one 64-token key block of one KV head: per dimension
 * the max, the min and the average over the block's 64 cached keys (the
 * pooling the settings table lists).  READING: the cached keys as
 * stored are pooled, and the three statistics are concatenated in the order
 * the pages list them. */
void sas_oracle_pool_stats(const oracle_shape *sh, const uint16_t *k_pool,
                           const int32_t *block_table, int s, int c, int kvh,
                           double *pooled /* [384] */) {
  for (int d = 0; d < HEAD_DIM; ++d) {
    double mx = -INFINITY, mn = INFINITY, sum = 0.0;
    for (int t = 0; t < BLOCK; ++t) {
      double x = bf16_value(kv_row(sh, k_pool, block_table, s, kvh, c * BLOCK + t)[d]);
      if (x > mx) mx = x;
      if (x < mn) mn = x;
      sum += x;
    }
    pooled[d] = mx;
    pooled[HEAD_DIM + d] = mn;
    pooled[2 * HEAD_DIM + d] = sum / BLOCK;
  }
}

/* Gate key of block c, KV head kvh.  READING: a bias-free linear map of the
 * 384 pooled values to the 128-wide gate space (one weight matrix per KV head,
 * stored output-major like a torch Linear weight, w_k[kvh][j][i]; the shape
 * the pages' gate-parameter counts imply), then
 * RMSNorm with weight w_knorm, then RoPE at the block's first position 64*c.
 * Output: fp64 before rounding (gk_f64, nullable) and bf16 RNE (gk_bf16). */
void sas_oracle_gate_key(const oracle_shape *sh, const uint16_t *k_pool,
                         const int32_t *block_table, int s, int c, int kvh,
                         const uint16_t *w_k, const float *w_knorm, double theta,
                         double *gk_f64, uint16_t *gk_bf16) {
  double pooled[POOLED], u[GATE_DIM];
  sas_oracle_pool_stats(sh, k_pool, block_table, s, c, kvh, pooled);
  const uint16_t *w = w_k + (int64_t)kvh * GATE_DIM * POOLED;
  for (int j = 0; j < GATE_DIM; ++j) {
    double acc = 0.0;
    for (int i = 0; i < POOLED; ++i) acc += pooled[i] * bf16_value(w[j * POOLED + i]);
    u[j] = acc;
  }
  sas_oracle_rms_norm(u, w_knorm);
  sas_oracle_rope(u, (double)c * BLOCK, theta);
  for (int j = 0; j < GATE_DIM; ++j) {
    if (gk_f64) gk_f64[j] = u[j];
    if (gk_bf16) gk_bf16[j] = sas_oracle_round_bf16(u[j]);
  }
}

/* Pool the listed (sequence, block) pairs for every KV head; writes the bf16
 * gate keys at gate_keys[page][kvh][128], page = block_table[s][c]. */
void sas_oracle_pool_blocks(const oracle_shape *sh, const uint16_t *k_pool,
                            const int32_t *block_table, const int32_t *pool_seq,
                            const int32_t *pool_blk, int32_t n, const uint16_t *w_k,
                            const float *w_knorm, double theta, uint16_t *gate_keys,
                            double *gate_keys_f64 /* nullable, [n][Hkv][128] */) {
  int64_t units = (int64_t)n * sh->n_kv_heads;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t u = 0; u < units; ++u) {
    int i = (int)(u / sh->n_kv_heads), kvh = (int)(u % sh->n_kv_heads);
    int s = pool_seq[i], c = pool_blk[i];
    int32_t page = block_table[(int64_t)s * sh->max_blocks + c];
    uint16_t *dst = gate_keys + ((int64_t)page * sh->n_kv_heads + kvh) * GATE_DIM;
    double *dst64 = gate_keys_f64 ? gate_keys_f64 + u * GATE_DIM : NULL;
    sas_oracle_gate_key(sh, k_pool, block_table, s, c, kvh, w_k, w_knorm, theta, dst64, dst);
  }
}

/* One decode step's cache write followed by incremental pooling.  Each
 * sequence's current token sits at position L-1, L = seq_lens[s] >= 1 the
 * length with that token counted; its key and value rows (k_new / v_new,
 * [B][Hkv][128]) are written there for every KV head.  A sequence whose length
 * reaches a multiple of 64 has just completed block L/64 - 1, and that block
 * is pooled into its gate key exactly as sas_oracle_pool_blocks does.
 * READING: the pages pool each full 64-token key block (release note and
 * settings table); they say nothing of when, so a block is pooled once, at the
 * step that writes its last row.  Returns the number of blocks pooled; their
 * (sequence, block) pairs go to done_seq / done_blk ([B] each). */
int32_t sas_oracle_append_kv(const oracle_shape *sh, uint16_t *k_pool, uint16_t *v_pool,
                             const int32_t *block_table, const int32_t *seq_lens,
                             const uint16_t *k_new, const uint16_t *v_new,
                             const uint16_t *w_k, const float *w_knorm, double theta,
                             uint16_t *gate_keys, int32_t *done_seq, int32_t *done_blk) {
  int32_t n_done = 0;
  for (int s = 0; s < sh->batch; ++s) {
    const int pos = seq_lens[s] - 1;
    for (int kvh = 0; kvh < sh->n_kv_heads; ++kvh) {
      const int64_t off = kv_row(sh, k_pool, block_table, s, kvh, pos) - k_pool;
      const int64_t src = ((int64_t)s * sh->n_kv_heads + kvh) * HEAD_DIM;
      for (int d = 0; d < HEAD_DIM; ++d) {
        k_pool[off + d] = k_new[src + d];
        v_pool[off + d] = v_new[src + d];
      }
    }
    if (seq_lens[s] % BLOCK == 0) {
      done_seq[n_done] = s;
      done_blk[n_done] = seq_lens[s] / BLOCK - 1;
      ++n_done;
    }
  }
  sas_oracle_pool_blocks(sh, k_pool, block_table, done_seq, done_blk, n_done, w_k, w_knorm,
                         theta, gate_keys, NULL);
  return n_done;
}

/* ------------------------------------------------------------------ */
/* Stage 2: gate query, block scores, Top-K, gates                     */
/* ------------------------------------------------------------------ */
/* Gate query of query head h of sequence s (the Qproj query projection).
 * READING: a bias-free 128x128 linear map per query head, stored
 * output-major like a torch Linear weight, w_q[h][j][d], then RMSNorm with
 * w_qnorm, then RoPE at the current token's position L-1. */
void sas_oracle_gate_query(const uint16_t *q /* [B][Hq][128] */, int n_q_heads, int s,
                           int h, const uint16_t *w_q, const float *w_qnorm,
                           double theta, int32_t seq_len, double *gq /* [128] */) {
  const uint16_t *qh = q + ((int64_t)s * n_q_heads + h) * HEAD_DIM;
  const uint16_t *w = w_q + (int64_t)h * HEAD_DIM * GATE_DIM;
  for (int j = 0; j < GATE_DIM; ++j) {
    double acc = 0.0;
    for (int d = 0; d < HEAD_DIM; ++d) acc += bf16_value(qh[d]) * bf16_value(w[j * HEAD_DIM + d]);
    gq[j] = acc;
  }
  sas_oracle_rms_norm(gq, w_qnorm);
  sas_oracle_rope(gq, (double)(seq_len - 1), theta);
}

/* Block scores of (s, kvh) for the candidates c < l, l = (L-1)/64 the local
 * block.  Per query head the score is <gate query, gate key> / sqrt(128);
 * READING: one selection per KV head, scored by the mean of its G query
 * heads' scores.  The result is rounded to fp32 (the precision in which the
 * GPU takes the same ranking decision).  scores[c] for c >= l is left as is. */
/* Block scores of one (sequence, KV head).  aggregate 0: the mean of the
 * group's per-head scores (the default reading); 1: their maximum (the
 * alternative reading of how one selection per KV head comes from a group of
 * query heads). */
void sas_oracle_block_scores_ex(const oracle_shape *sh, const uint16_t *q, const uint16_t *w_q,
                                const float *w_qnorm, const uint16_t *gate_keys,
                                const int32_t *block_table, const int32_t *seq_lens,
                                double theta, int s, int kvh, int aggregate, float *scores) {
  int G = sh->n_q_heads / sh->n_kv_heads;
  int32_t L = seq_lens[s];
  int local = (L - 1) / BLOCK;
  double *gq = (double *)malloc(sizeof(double) * GATE_DIM * G);
  for (int g = 0; g < G; ++g)
    sas_oracle_gate_query(q, sh->n_q_heads, s, kvh * G + g, w_q, w_qnorm, theta, L, gq + g * GATE_DIM);
  for (int c = 0; c < local; ++c) {
    int32_t page = block_table[(int64_t)s * sh->max_blocks + c];
    const uint16_t *gk = gate_keys + ((int64_t)page * sh->n_kv_heads + kvh) * GATE_DIM;
    double mean = 0.0, mx = -INFINITY;
    for (int g = 0; g < G; ++g) {
      double dot = 0.0;
      for (int j = 0; j < GATE_DIM; ++j) dot += gq[g * GATE_DIM + j] * bf16_value(gk[j]);
      mean += dot / sqrt((double)GATE_DIM);
      if (dot / sqrt((double)GATE_DIM) > mx) mx = dot / sqrt((double)GATE_DIM);
    }
    scores[c] = (float)(aggregate == 1 ? mx : mean / G);
  }
  free(gq);
}

void sas_oracle_block_scores(const oracle_shape *sh, const uint16_t *q, const uint16_t *w_q,
                             const float *w_qnorm, const uint16_t *gate_keys,
                             const int32_t *block_table, const int32_t *seq_lens,
                             double theta, int s, int kvh, float *scores) {
  sas_oracle_block_scores_ex(sh, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, theta, s, kvh, 0,
                             scores);
}

typedef struct {
  float score;
  int32_t block;
} ranked;

/* Total order of candidates: higher score first, lower block index on equal
 * scores (READING: the pages give no tie rule; this one makes the Top-K set
 * unique).  NaN ranks as -inf; -0 equals +0 under float comparison. */
static int rank_cmp(const void *pa, const void *pb) {
  const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
  float sa = isnan(a->score) ? -INFINITY : a->score;
  float sb = isnan(b->score) ? -INFINITY : b->score;
  if (sa > sb) return -1;
  if (sa < sb) return 1;
  return (a->block > b->block) - (a->block < b->block);
}

static int int_cmp(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

/* Continuous gates of a selection of cnt blocks (the last one local):
 * g = sigmoid(score) for the historical blocks, 1 for the local block, 0 for
 * the padding up to n_sel.  A NaN score counts as -inf here as in the
 * ranking (READING), so its gate is sigmoid(-inf) = 0. */
void sas_oracle_block_gates(const float *scores, const int32_t *sel, int32_t cnt, int32_t n_sel,
                            float *gates) {
  for (int i = 0; i < n_sel; ++i) {
    if (i < cnt - 1) {
      double sc = isnan(scores[sel[i]]) ? -INFINITY : (double)scores[sel[i]];
      gates[i] = (float)(1.0 / (1.0 + exp(-sc)));
    } else
      gates[i] = i == cnt - 1 ? 1.0f : 0.0f;
  }
}

/* Top-K of one (s, kvh).  The budget of B tokens is B/64 blocks: the local
 * block (always attended, never a candidate) plus K_hist = B/64 - 1 historical
 * blocks (31 at the default 2,048 tokens).  K_eff = min(K_hist, l).  Output:
 * selected blocks ascending (the local block, the largest index, last),
 * padded with -1 to B/64 entries; gates g = sigmoid(score) for historical
 * blocks and 1 for the local block (READING of "continuous gates on selected
 * blocks").  Returns the count K_eff + 1. */
int32_t sas_oracle_select(const float *scores, int32_t seq_len, int32_t budget_tokens,
                          int32_t *sel, float *gates) {
  int n_sel = budget_tokens / BLOCK;
  int k_hist = n_sel - 1;
  int local = (seq_len - 1) / BLOCK;
  int k_eff = k_hist < local ? k_hist : local;
  ranked *r = (ranked *)malloc(sizeof(ranked) * (local > 0 ? local : 1));
  for (int c = 0; c < local; ++c) {
    r[c].score = scores[c];
    r[c].block = c;
  }
  qsort(r, (size_t)local, sizeof(ranked), rank_cmp);
  int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (k_eff + 1));
  for (int i = 0; i < k_eff; ++i) chosen[i] = r[i].block;
  qsort(chosen, (size_t)k_eff, sizeof(int32_t), int_cmp);
  chosen[k_eff] = local;
  for (int i = 0; i < n_sel; ++i) sel[i] = i <= k_eff ? chosen[i] : -1;
  if (gates) sas_oracle_block_gates(scores, sel, k_eff + 1, n_sel, gates);
  free(chosen);
  free(r);
  return k_eff + 1;
}

/* Gate stage for the whole batch: scores_out [B][Hkv][max_blocks] (nullable;
 * entries c >= l are set to -inf), sel/gates [B][Hkv][budget/64], cnt [B][Hkv]. */
void sas_oracle_gate_topk_ex(const oracle_shape *sh, const uint16_t *q, const uint16_t *w_q,
                             const float *w_qnorm, const uint16_t *gate_keys,
                             const int32_t *block_table, const int32_t *seq_lens, double theta,
                             int32_t budget_tokens, int aggregate, int32_t *sel, float *gates,
                             int32_t *cnt, float *scores_out) {
  int n_sel = budget_tokens / BLOCK;
  int64_t units = (int64_t)sh->batch * sh->n_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int s = (int)(u / sh->n_kv_heads), kvh = (int)(u % sh->n_kv_heads);
    float *scores = (float *)malloc(sizeof(float) * (sh->max_blocks > 0 ? sh->max_blocks : 1));
    for (int c = 0; c < sh->max_blocks; ++c) scores[c] = -INFINITY;
    sas_oracle_block_scores_ex(sh, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, theta, s, kvh,
                               aggregate, scores);
    cnt[u] = sas_oracle_select(scores, seq_lens[s], budget_tokens, sel + u * n_sel,
                               gates ? gates + u * n_sel : NULL);
    if (scores_out) memcpy(scores_out + u * sh->max_blocks, scores, sizeof(float) * sh->max_blocks);
    free(scores);
  }
}

void sas_oracle_gate_topk(const oracle_shape *sh, const uint16_t *q, const uint16_t *w_q,
                          const float *w_qnorm, const uint16_t *gate_keys,
                          const int32_t *block_table, const int32_t *seq_lens, double theta,
                          int32_t budget_tokens, int32_t *sel, float *gates, int32_t *cnt,
                          float *scores_out) {
  sas_oracle_gate_topk_ex(sh, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, theta, budget_tokens, 0,
                          sel, gates, cnt, scores_out);
}

/* ------------------------------------------------------------------ */
/* Stage 3: attention over the selected blocks, as dense masked softmax */
/* ------------------------------------------------------------------ */
/* Decode attention of query head h of sequence s over all L cached tokens with
 * an explicit token mask: token j is kept iff its block j/64 is in the
 * selection (and j <= L-1).  z_j = sm_scale * <q, k_j>; P = softmax(z) over
 * the kept tokens.  Plain mode: o = sum_j P_j v_j.  Gated mode (gates given):
 * READING of the continuous gates on selected blocks -- each selected block's
 * contribution is scaled by its gate, o = sum_j g_{block(j)} P_j v_j, with P
 * normalised over the whole selection.  GQA: head h reads KV head h / G. */
void sas_oracle_attend_head(const oracle_shape *sh, const uint16_t *q, const uint16_t *k_pool,
                            const uint16_t *v_pool, const int32_t *block_table,
                            const int32_t *seq_lens, const int32_t *sel, const float *gates,
                            const int32_t *cnt, int32_t n_sel, double sm_scale, int gate_mode,
                            int s, int h, double *out /* [128] */) {
  int G = sh->n_q_heads / sh->n_kv_heads;
  int kvh = h / G;
  int32_t L = seq_lens[s];
  int nblk = (L + BLOCK - 1) / BLOCK;
  const int32_t *my_sel = sel + ((int64_t)s * sh->n_kv_heads + kvh) * n_sel;
  const float *my_gate = gates ? gates + ((int64_t)s * sh->n_kv_heads + kvh) * n_sel : NULL;
  int32_t my_cnt = cnt[(int64_t)s * sh->n_kv_heads + kvh];
  /* explicit per-token mask and per-token gate */
  char *keep = (char *)calloc((size_t)L, 1);
  double *gate_tok = (double *)malloc(sizeof(double) * (size_t)L);
  double *blk_gate = (double *)malloc(sizeof(double) * (size_t)nblk);
  char *blk_keep = (char *)calloc((size_t)nblk, 1);
  for (int i = 0; i < my_cnt; ++i) {
    int b = my_sel[i];
    if (b >= 0 && b < nblk) {
      blk_keep[b] = 1;
      blk_gate[b] = my_gate ? (double)my_gate[i] : 1.0;
    }
  }
  for (int j = 0; j < L; ++j) {
    keep[j] = blk_keep[j / BLOCK];
    gate_tok[j] = keep[j] ? blk_gate[j / BLOCK] : 0.0;
  }
  const uint16_t *qh = q + ((int64_t)s * sh->n_q_heads + h) * HEAD_DIM;
  double *z = (double *)malloc(sizeof(double) * (size_t)L);
  double zmax = -INFINITY;
  for (int j = 0; j < L; ++j) {
    const uint16_t *kr = kv_row(sh, k_pool, block_table, s, kvh, j);
    double dot = 0.0;
    for (int d = 0; d < HEAD_DIM; ++d) dot += bf16_value(qh[d]) * bf16_value(kr[d]);
    z[j] = keep[j] ? dot * sm_scale : -INFINITY;
    if (z[j] > zmax) zmax = z[j];
  }
  /* gate_mode 0: softmax over the selected tokens, then each token's weight
   * scaled by its block's gate (the default reading).  gate_mode 1: the gate
   * as a factor on exp(logit) before normalising (a log-gate bias on the
   * logits, the alternative reading). */
  double denom = 0.0;
  for (int j = 0; j < L; ++j) {
    z[j] = keep[j] ? exp(z[j] - zmax) : 0.0;
    if (gate_mode == 1) z[j] *= gate_tok[j];
    denom += z[j];
  }
  for (int d = 0; d < HEAD_DIM; ++d) out[d] = 0.0;
  for (int j = 0; j < L; ++j) {
    double p = denom > 0 ? z[j] / denom : 0.0; /* 0 for masked tokens */
    double w = gate_mode == 1 ? p : p * gate_tok[j];
    const uint16_t *vr = kv_row(sh, v_pool, block_table, s, kvh, j);
    for (int d = 0; d < HEAD_DIM; ++d) out[d] += w * bf16_value(vr[d]);
  }
  free(z);
  free(blk_keep);
  free(blk_gate);
  free(gate_tok);
  free(keep);
}

/* Attention for a list of (sequence, query head) pairs (all pairs when
 * pairs == NULL, n_pairs = B*Hq); out is [n_pairs][128] fp64. */
void sas_oracle_attend(const oracle_shape *sh, const uint16_t *q, const uint16_t *k_pool,
                       const uint16_t *v_pool, const int32_t *block_table,
                       const int32_t *seq_lens, const int32_t *sel, const float *gates,
                       const int32_t *cnt, int32_t n_sel, double sm_scale, int gate_mode,
                       const int32_t *pairs /* [n][2] or NULL */, int64_t n_pairs, double *out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_pairs; ++i) {
    int s, h;
    if (pairs) {
      s = pairs[2 * i];
      h = pairs[2 * i + 1];
    } else {
      s = (int)(i / sh->n_q_heads);
      h = (int)(i % sh->n_q_heads);
    }
    sas_oracle_attend_head(sh, q, k_pool, v_pool, block_table, seq_lens, sel, gates, cnt, n_sel,
                           sm_scale, gate_mode, s, h, out + i * HEAD_DIM);
  }
}

int sas_oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
