"""Planted-block recipe for the recall workloads (test side; uses the oracle).

A planted block c of (sequence s, KV head kvh) gets the same offset vector
added to all 64 of its cached keys.  Adding one vector to every row shifts the
block's max, min and mean by exactly that vector, so the pooled statistics --
and through them the gate key -- move along a known direction.  READING of the
"+delta offset along the query direction" of the recall workloads: the offset
points along the direction that raises block c's gate score fastest, i.e. the
gate query mapped back into key space,

    u = unit( (Wk_max + Wk_min + Wk_mean)^T @ (w_knorm * R(-64c) gq_mean) ),

where Wk_* are the three 128-column slices of the pooled-key projection
(output-major, [128 out][384 in]), R the
gate RoPE rotation and gq_mean the mean gate query of the KV head's group.
Its per-component RMS is delta (norm delta * sqrt(128)), matching the
N(0, 1) scale of the keys.  K stays bf16: the offset is added in fp32 and
rounded to nearest even.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from learned_block_sparse_tok_amd import workloads as wl


def plant(w: wl.Workload) -> None:
    """Apply the planted offsets of ``w`` to ``w.k_pool`` in place."""
    if w.planted is None:
        return
    q = wl.host(w.q)
    w_q = wl.host(w.w_q)
    w_k = oracle.bf16_to_f64(wl.host(w.w_k)).reshape(w.n_kv_heads, wl.GATE_DIM, 3, wl.HEAD_DIM)
    wqn = wl.host(w.w_qnorm)
    wkn = wl.host(w.w_knorm).astype(np.float64)
    lens = wl.host(w.seq_lens)
    bt = wl.host(w.block_table)
    G = w.group
    ps, ts, hs = w.strides
    flat = w.k_pool.view(-1)
    rows = torch.arange(wl.BLOCK, device=flat.device, dtype=torch.int64)
    dims = torch.arange(wl.HEAD_DIM, device=flat.device, dtype=torch.int64)
    for s in range(w.batch):
        for kvh in range(w.n_kv_heads):
            gq = np.mean([oracle.gate_query(q, w_q, wqn, w.theta, int(lens[s]), s, kvh * G + g)
                          for g in range(G)], axis=0)
            wsum = w_k[kvh].sum(axis=1)  # [128 gate][128 key dim]
            for c in w.planted[s, kvh]:
                t = wkn * oracle.rope(gq, -float(c) * wl.BLOCK, w.theta)
                u = wsum.T @ t
                u = u / np.linalg.norm(u) * (w.plant_delta * np.sqrt(wl.HEAD_DIM))
                page = int(bt[s, c])
                idx = page * ps + kvh * hs + rows[:, None] * ts + dims[None, :]
                off = torch.as_tensor(u, dtype=torch.float32, device=flat.device)
                flat[idx] = (flat[idx].float() + off[None, :]).to(torch.bfloat16)
