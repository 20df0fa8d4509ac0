"""SAS decode-path oracle -- test infrastructure, not product code.

Python face of ``sas_oracle.c``: a plain, slow, fp64 CPU implementation of the
three SAS stages (key-block pooling -> gate scores + per-KV-head Top-K ->
attention over the selected 64-token blocks, written as dense softmax
attention over an explicit token mask).  The passages each step follows are
cited in the C source.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path:
its inputs are plain numpy arrays (bf16 values travel as their uint16 bit
patterns) and it never calls into the GPU library.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sas_oracle.c")
_LIB = os.path.join(_HERE, "_sas_oracle.so")

BLOCK = 64
HEAD_DIM = 128
GATE_DIM = 128
# alternative readings: how a group's per-head scores make one score, and how
# a gate enters attention ("scale" its block's share / "logit" a log bias)
AGGREGATE = {"mean": 0, "max": 1}
GATE_MODE = {"scale": 0, "logit": 1}
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, IEEE arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("page_stride", ctypes.c_int64), ("tok_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _lib.sas_oracle_round_bf16.restype = ctypes.c_uint16
        _lib.sas_oracle_round_bf16.argtypes = [ctypes.c_double]
        _lib.sas_oracle_select.restype = ctypes.c_int32
        _lib.sas_oracle_num_threads.restype = ctypes.c_int
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _shape(batch, n_q_heads, n_kv_heads, max_blocks, strides):
    ps, ts, hs = strides
    return _Shape(batch, n_q_heads, n_kv_heads, max_blocks, ps, ts, hs)


def num_threads() -> int:
    return int(_load().sas_oracle_num_threads())


def round_bf16(x: float) -> int:
    """fp64 -> bf16 bit pattern, round to nearest even in one step."""
    return int(_load().sas_oracle_round_bf16(float(x)))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rms_norm(v: np.ndarray, w: np.ndarray) -> np.ndarray:
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    w = np.ascontiguousarray(w, dtype=np.float32)
    _load().sas_oracle_rms_norm(_p(out), _p(w))
    return out


def rope(v: np.ndarray, pos: float, theta: float) -> np.ndarray:
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    _load().sas_oracle_rope(_p(out), ctypes.c_double(pos), ctypes.c_double(theta))
    return out


def pool_stats(k_pool, block_table, strides, max_blocks, n_kv_heads, s, c, kvh) -> np.ndarray:
    sh = _shape(block_table.shape[0], n_kv_heads, n_kv_heads, max_blocks, strides)
    out = np.zeros(3 * HEAD_DIM, np.float64)
    _load().sas_oracle_pool_stats(ctypes.byref(sh), _p(k_pool), _p(block_table), s, c, kvh, _p(out))
    return out


def pool_blocks(k_pool, block_table, strides, n_kv_heads, pool_seq, pool_blk, w_k, w_knorm,
                theta, gate_keys, want_f64=False):
    """Fill gate_keys (uint16 [P][Hkv][128], modified in place) for the listed
    (sequence, block) pairs.  Returns the fp64 keys before rounding
    ([n][Hkv][128]) when want_f64."""
    B, max_blocks = block_table.shape
    sh = _shape(B, n_kv_heads, n_kv_heads, max_blocks, strides)
    pool_seq = np.ascontiguousarray(pool_seq, np.int32)
    pool_blk = np.ascontiguousarray(pool_blk, np.int32)
    n = len(pool_seq)
    f64 = np.zeros((n, n_kv_heads, GATE_DIM), np.float64) if want_f64 else None
    _load().sas_oracle_pool_blocks(ctypes.byref(sh), _p(k_pool), _p(block_table), _p(pool_seq),
                                   _p(pool_blk), ctypes.c_int32(n), _p(w_k), _p(w_knorm),
                                   ctypes.c_double(theta), _p(gate_keys), _p(f64))
    return f64


def append_kv(k_pool, v_pool, block_table, strides, n_kv_heads, seq_lens, k_new, v_new, w_k, w_knorm,
              theta, gate_keys):
    """One decode step's cache write + incremental pooling, in place: rows
    k_new / v_new ([B][Hkv][128]) go to position seq_lens[s]-1 of each
    sequence; blocks that this completes are pooled into gate_keys.  Returns
    the (sequence, block) pairs pooled, as two int32 arrays."""
    B, max_blocks = block_table.shape
    sh = _shape(B, n_kv_heads, n_kv_heads, max_blocks, strides)
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    done_seq = np.zeros(B, np.int32)
    done_blk = np.zeros(B, np.int32)
    n = _load().sas_oracle_append_kv(ctypes.byref(sh), _p(k_pool), _p(v_pool), _p(block_table), _p(seq_lens),
                                     _p(np.ascontiguousarray(k_new)), _p(np.ascontiguousarray(v_new)), _p(w_k),
                                     _p(w_knorm), ctypes.c_double(theta), _p(gate_keys), _p(done_seq),
                                     _p(done_blk))
    return done_seq[:n].copy(), done_blk[:n].copy()


def gate_query(q, w_q, w_qnorm, theta, seq_len, s, h) -> np.ndarray:
    out = np.zeros(GATE_DIM, np.float64)
    _load().sas_oracle_gate_query(_p(q), ctypes.c_int(q.shape[1]), ctypes.c_int(s), ctypes.c_int(h),
                                  _p(w_q), _p(w_qnorm), ctypes.c_double(theta),
                                  ctypes.c_int32(seq_len), _p(out))
    return out


def gate_topk(q, w_q, w_qnorm, gate_keys, block_table, seq_lens, theta, budget_tokens,
              n_kv_heads, aggregate="mean"):
    """Gate stage for the batch.  Returns (sel, gates, cnt, scores):
    sel int32 [B][Hkv][budget/64] (ascending, local block last, -1 padded),
    gates f32 (same shape; sigmoid(score), 1 for the local block, 0 padding),
    cnt int32 [B][Hkv], scores f32 [B][Hkv][max_blocks] (-inf for c >= l)."""
    B, Hq, _ = q.shape
    max_blocks = block_table.shape[1]
    sh = _shape(B, Hq, n_kv_heads, max_blocks, (0, 0, 0))
    n_sel = budget_tokens // BLOCK
    sel = np.zeros((B, n_kv_heads, n_sel), np.int32)
    gates = np.zeros((B, n_kv_heads, n_sel), np.float32)
    cnt = np.zeros((B, n_kv_heads), np.int32)
    scores = np.zeros((B, n_kv_heads, max_blocks), np.float32)
    _load().sas_oracle_gate_topk_ex(ctypes.byref(sh), _p(q), _p(w_q), _p(w_qnorm), _p(gate_keys),
                                    _p(block_table), _p(np.ascontiguousarray(seq_lens, np.int32)),
                                    ctypes.c_double(theta), ctypes.c_int32(budget_tokens),
                                    ctypes.c_int(AGGREGATE[aggregate]), _p(sel), _p(gates), _p(cnt), _p(scores))
    return sel, gates, cnt, scores


def select(scores: np.ndarray, seq_len: int, budget_tokens: int):
    """Top-K of one (sequence, KV head) from its fp32 block scores."""
    n_sel = budget_tokens // BLOCK
    sel = np.zeros(n_sel, np.int32)
    gates = np.zeros(n_sel, np.float32)
    sc = np.ascontiguousarray(scores, np.float32)
    cnt = _load().sas_oracle_select(_p(sc), ctypes.c_int32(seq_len), ctypes.c_int32(budget_tokens),
                                    _p(sel), _p(gates))
    return sel, gates, int(cnt)


def block_gates(scores: np.ndarray, sel: np.ndarray, cnt: int) -> np.ndarray:
    """Gates of a given selection of one (sequence, KV head): sigmoid of the
    block scores, 1 for the last (local) block, 0 padding."""
    sc = np.ascontiguousarray(scores, np.float32)
    sel = np.ascontiguousarray(sel, np.int32)
    out = np.zeros(len(sel), np.float32)
    _load().sas_oracle_block_gates(_p(sc), _p(sel), ctypes.c_int32(cnt), ctypes.c_int32(len(sel)), _p(out))
    return out


def attend(q, k_pool, v_pool, block_table, strides, n_kv_heads, seq_lens, sel, gates, cnt,
           sm_scale, pairs=None, gate_mode="scale"):
    """Dense masked softmax attention.  gates=None is plain Top-K mode.
    pairs: optional int32 [n][2] list of (sequence, query head); default all.
    Returns fp64 [n][128] (or [B][Hq][128] when pairs is None)."""
    B, Hq, _ = q.shape
    max_blocks = block_table.shape[1]
    sh = _shape(B, Hq, n_kv_heads, max_blocks, strides)
    n_sel = sel.shape[-1]
    if pairs is not None:
        pairs = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
        n = pairs.shape[0]
    else:
        n = B * Hq
    out = np.zeros((n, HEAD_DIM), np.float64)
    g = None if gates is None else np.ascontiguousarray(gates, np.float32)
    _load().sas_oracle_attend(ctypes.byref(sh), _p(q), _p(k_pool), _p(v_pool), _p(block_table),
                              _p(np.ascontiguousarray(seq_lens, np.int32)),
                              _p(np.ascontiguousarray(sel, np.int32)), _p(g),
                              _p(np.ascontiguousarray(cnt, np.int32)), ctypes.c_int32(n_sel),
                              ctypes.c_double(sm_scale), ctypes.c_int(GATE_MODE[gate_mode]), _p(pairs),
                              ctypes.c_int64(n), _p(out))
    return out if pairs is not None else out.reshape(B, Hq, HEAD_DIM)


def prefill(q, k_pool, v_pool, block_table_row, strides, n_kv_heads, gate_keys, w_q, w_qnorm, theta,
            budget_tokens, gated, sm_scale, positions=None):
    """Training-time forward of one sequence with per-query block selection.

    The pages say SAS selects KV blocks for each query and trains with a
    Top-K of 31 historical blocks on 32,768-token sequences (aigc.news release
    note; "Tencent Hunyuan open-sources SAS ...": per-query block selection).
    READING: query position t (0-based, q[t], T = len(q) positions) selects and
    attends exactly as a decode step whose cache holds the first t+1 tokens:
    gate query at position t, candidates the complete blocks c < t/64, the
    Top-K plus its own block t/64, then causal attention over the selected
    blocks' tokens j <= t.  So the forward is gate_topk + attend over the batch
    of positions, all sharing the one block-table row.

    positions: optional int array of the positions to compute (default all).
    Returns (sel, gates, cnt, scores, out) for those positions, shaped as
    gate_topk / attend return them with the positions as the batch."""
    T = q.shape[0]
    pos = np.arange(T, dtype=np.int32) if positions is None else np.asarray(positions, np.int32)
    qp = np.ascontiguousarray(q[pos])
    lens = (pos + 1).astype(np.int32)
    bt = np.ascontiguousarray(np.broadcast_to(np.asarray(block_table_row, np.int32),
                                              (len(pos), len(block_table_row))))
    sel, gates, cnt, scores = gate_topk(qp, w_q, w_qnorm, gate_keys, bt, lens, theta, budget_tokens, n_kv_heads)
    out = attend(qp, k_pool, v_pool, bt, strides, n_kv_heads, lens, sel, gates if gated else None, cnt, sm_scale)
    return sel, gates, cnt, scores, out


def _block_rows(pool, block_table, strides, s, c, kvh, nvalid):
    """The first nvalid rows of block c of sequence s, KV head kvh, fp64 [n][128]."""
    ps, ts, hs = strides
    page = int(block_table[s, c])
    base = page * ps + kvh * hs
    idx = base + np.arange(nvalid)[:, None] * ts + np.arange(HEAD_DIM)[None, :]
    return bf16_to_f64(pool.reshape(-1)[idx])


def gate_backward(q, k_pool, v_pool, block_table, strides, n_kv_heads, seq_lens, sel, gates, cnt, sm_scale,
                  w_q, w_qnorm, w_k, w_knorm, gate_keys, theta, d_out, round_keys=True):
    """Gradients of the gate parameters through the continuous gates of one
    gated decode step (the default reading: each selected block's share of
    the output scaled by its gate g = sigmoid(score)).

    SAS puts continuous gates on the selected blocks so that the language-model
    loss reaches the ranking (aigc.news release note; "Tencent Hunyuan
    open-sources SAS ...": a differentiable path from the LM loss to the
    selector).  READING: the Top-K choice itself passes no gradient; the local
    block's gate is the constant 1; the gate keys' bf16 storage passes the
    gradient unchanged (straight through); the backbone's q, K, V are inputs.

    d_out: bf16 bits [B][Hq][128], the gradient of the loss w.r.t. the step's
    output.  With o_h = sum_i g_i sum_{j in block c_i} P_hj v_j:
      dg_i  = sum_{h in group} sum_{j in c_i} P_hj <d_out_h, v_j>
      dS_i  = dg_i g_i (1 - g_i)                  (historical blocks only)
      dghat = sum_i dS_i gk_{c_i} / sqrt(128),   d gk_{c_i} = dS_i ghat / sqrt(128)
    then through the group mean, RoPE (a rotation: its transpose rotates
    back), RMSNorm and the bias-free projections.  round_keys: use the stored
    bf16 gate keys in dghat (as the forward's scores do); False uses the
    unrounded fp64 keys (the smooth function finite differences can see).
    Returns dict(d_gates [B][Hkv][n_sel], d_w_q [Hq][128][128],
    d_w_qnorm [128], d_w_k [Hkv][128][384], d_w_knorm [128]), fp64, summed
    over the batch; d_gates covers every selected block (local included)."""
    B, Hq, _ = q.shape
    Hkv = n_kv_heads
    G = Hq // Hkv
    max_blocks = block_table.shape[1]
    qf, dO = bf16_to_f64(q), bf16_to_f64(d_out)
    wq, wk = bf16_to_f64(w_q), bf16_to_f64(w_k)
    wqn, wkn = np.asarray(w_qnorm, np.float64), np.asarray(w_knorm, np.float64)
    rs = math.sqrt(GATE_DIM)
    out = dict(d_gates=np.zeros(sel.shape), d_w_q=np.zeros((Hq, GATE_DIM, HEAD_DIM)), d_w_qnorm=np.zeros(GATE_DIM),
               d_w_k=np.zeros((Hkv, GATE_DIM, 3 * HEAD_DIM)), d_w_knorm=np.zeros(GATE_DIM))

    def rms_parts(u):
        r = math.sqrt(float(np.mean(u * u)) + 1e-6)
        return u / r, r

    def rms_back(dn, nrm, r, w):
        """d(u) from d(n), n = (u / r) * w; also d(w)."""
        a = dn * w
        return (a - nrm * float(np.mean(a * nrm))) / r, dn * nrm

    for s in range(B):
        L = int(seq_lens[s])
        for kvh in range(Hkv):
            c_sel = sel[s, kvh, :cnt[s, kvh]]
            g_sel = np.asarray(gates[s, kvh, :cnt[s, kvh]], np.float64)
            K = [_block_rows(k_pool, block_table, strides, s, int(c), kvh, min(64, L - 64 * int(c))) for c in c_sel]
            V = [_block_rows(v_pool, block_table, strides, s, int(c), kvh, min(64, L - 64 * int(c))) for c in c_sel]
            Kall, Vall = np.concatenate(K), np.concatenate(V)
            edges = np.cumsum([0] + [len(k) for k in K])
            dg = np.zeros(len(c_sel))
            for h in range(kvh * G, (kvh + 1) * G):
                z = Kall @ qf[s, h] * sm_scale
                P = np.exp(z - z.max())
                P /= P.sum()
                dv = Vall @ dO[s, h]
                for i in range(len(c_sel)):
                    dg[i] += float(P[edges[i]:edges[i + 1]] @ dv[edges[i]:edges[i + 1]])
            out["d_gates"][s, kvh, :len(c_sel)] = dg
            n_hist = len(c_sel) - 1
            dS = dg[:n_hist] * g_sel[:n_hist] * (1.0 - g_sel[:n_hist])
            # gate queries of the group and their mean
            parts = []
            for h in range(kvh * G, (kvh + 1) * G):
                u = wq[h] @ qf[s, h]
                nrm, r = rms_parts(u)
                parts.append((h, nrm, r, rope(nrm * wqn, L - 1, theta)))
            ghat = np.mean([p[3] for p in parts], axis=0)
            # keys of the historical selection: stored bf16, and the fp64 chain
            keys = []
            for i in range(n_hist):
                c = int(c_sel[i])
                p_c = pool_stats(k_pool, block_table, strides, max_blocks, Hkv, s, c, kvh)
                u = wk[kvh] @ p_c
                nrm, r = rms_parts(u)
                gk64 = rope(nrm * wkn, 64.0 * c, theta)
                gk_b = bf16_to_f64(gate_keys[int(block_table[s, c]), kvh]) if round_keys else gk64
                keys.append((c, p_c, nrm, r, gk_b))
            dghat = np.zeros(GATE_DIM)
            for i, (c, p_c, nrm, r, gk_b) in enumerate(keys):
                dghat += dS[i] * gk_b / rs
                dm = rope(dS[i] * ghat / rs, -64.0 * c, theta)
                du, dw = rms_back(dm, nrm, r, wkn)
                out["d_w_knorm"] += dw
                out["d_w_k"][kvh] += np.outer(du, p_c)
            for h, nrm, r, _ in parts:
                dn = rope(dghat / G, -(L - 1.0), theta)
                du, dw = rms_back(dn, nrm, r, wqn)
                out["d_w_qnorm"] += dw
                out["d_w_q"][h] += np.outer(du, qf[s, h])
    return out


def prefill_gate_backward(q, k_pool, v_pool, block_table_row, strides, n_kv_heads, sel, gates, cnt, sm_scale,
                          w_q, w_qnorm, w_k, w_knorm, gate_keys, theta, d_out, round_keys=True, positions=None):
    """Gradients of the gate parameters through the continuous gates of the
    training-time forward of one sequence (prefill above: every position a
    query), for the loss sum_t sum_h <d_out[t][h], out[t][h]>.

    SAS trains its gates with the language-model loss on 32,768-token
    sequences, each query selecting its own blocks (aigc.news release note:
    training Top-K of 31 historical blocks, the LM loss ranking the context
    end to end; "Tencent Hunyuan open-sources SAS ...": per-query selection,
    a differentiable path to the selector).  READING: with the forward's
    reading (position t is the decode step whose cache holds its first t+1
    tokens) the loss is a sum over positions, so its gradient is the sum of
    gate_backward's per-step gradients over the batch of positions sharing
    the one block-table row; each block's key receives the gradient of every
    position that selected it.

    sel / gates / cnt: [T][Hkv][n_sel], [T][Hkv] as prefill returns them;
    d_out: bf16 bits [T][Hq][128].  positions: optional subset of positions
    whose terms are summed (the gradient of the loss with d_out zero at every
    other position); d_gates then covers those positions only.
    Returns gate_backward's dict."""
    T = q.shape[0]
    pos = np.arange(T, dtype=np.int32) if positions is None else np.asarray(positions, np.int32)
    lens = (pos + 1).astype(np.int32)
    bt = np.ascontiguousarray(np.broadcast_to(np.asarray(block_table_row, np.int32),
                                              (len(pos), len(block_table_row))))
    return gate_backward(np.ascontiguousarray(q[pos]), k_pool, v_pool, bt, strides, n_kv_heads, lens,
                         np.ascontiguousarray(sel[pos]), np.ascontiguousarray(gates[pos]),
                         np.ascontiguousarray(cnt[pos]), sm_scale, w_q, w_qnorm, w_k, w_knorm, gate_keys, theta,
                         np.ascontiguousarray(d_out[pos]), round_keys=round_keys)
