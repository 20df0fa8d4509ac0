"""Test-side glue: hand a workload's arrays to the oracle as numpy arrays."""
from __future__ import annotations

import math

import numpy as np

import oracle
from learned_block_sparse_tok_amd import workloads as wl

SM_SCALE = 1.0 / math.sqrt(wl.HEAD_DIM)


class Host:
    """Host (numpy) copies of a workload's arrays, bf16 as uint16 bits."""

    def __init__(self, w: wl.Workload):
        self.w = w
        self.q = wl.host(w.q)
        self.k = wl.host(w.k_pool)
        self.v = wl.host(w.v_pool)
        self.bt = wl.host(w.block_table)
        self.lens = wl.host(w.seq_lens).astype(np.int32)
        self.w_q = wl.host(w.w_q)
        self.w_k = wl.host(w.w_k)
        self.wqn = wl.host(w.w_qnorm).astype(np.float32)
        self.wkn = wl.host(w.w_knorm).astype(np.float32)


def complete_blocks(lens: np.ndarray):
    """(sequence, block) pairs of every full 64-token block."""
    seq, blk = [], []
    for s, L in enumerate(lens):
        for c in range(int(L) // wl.BLOCK):
            seq.append(s)
            blk.append(c)
    return np.asarray(seq, np.int32), np.asarray(blk, np.int32)


def oracle_gate_keys(h: Host, want_f64=False):
    w = h.w
    gk = np.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), np.uint16)
    seq, blk = complete_blocks(h.lens)
    f64 = oracle.pool_blocks(h.k, h.bt, w.strides, w.n_kv_heads, seq, blk, h.w_k, h.wkn, w.theta,
                             gk, want_f64=want_f64)
    return (gk, f64, seq, blk) if want_f64 else gk


def oracle_step(h: Host, gated: bool, budget: int | None = None, gate_keys=None):
    """The whole step on the oracle: pool -> gate/Top-K -> dense masked attention."""
    w = h.w
    budget = budget or w.budget
    gk = oracle_gate_keys(h) if gate_keys is None else gate_keys
    sel, gates, cnt, scores = oracle.gate_topk(h.q, h.w_q, h.wqn, gk, h.bt, h.lens, w.theta, budget,
                                               w.n_kv_heads)
    out = oracle.attend(h.q, h.k, h.v, h.bt, w.strides, w.n_kv_heads, h.lens, sel,
                        gates if gated else None, cnt, SM_SCALE)
    return dict(gate_keys=gk, sel=sel, gates=gates, cnt=cnt, scores=scores, out=out)
