"""GPU-side test glue: run the libsas path on a workload (the comparison with
the oracle and its tie accounting are in compare.py)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from compare import (OUT_MAX_ABS, OUT_MEAN_ABS, TIE_REL, assert_out_close, compare_selection,  # noqa: F401
                     compare_step, topk_band)
from harness import complete_blocks
from learned_block_sparse_tok_amd import ops
from learned_block_sparse_tok_amd import workloads as wl


def shape_of(w: wl.Workload) -> ops.SasShape:
    return ops.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)


def gpu_pool(w: wl.Workload, seq=None, blk=None) -> torch.Tensor:
    """Gate keys of every complete block (or of the listed pairs), on the GPU."""
    gk = torch.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), dtype=torch.bfloat16, device=w.q.device)
    if seq is None:
        seq, blk = complete_blocks(wl.host(w.seq_lens))
    ops.pool_blocks(shape_of(w), w.k_pool, w.block_table, torch.as_tensor(seq, device=w.q.device),
                    torch.as_tensor(blk, device=w.q.device), w.w_k, w.w_knorm, w.theta, gk)
    return gk


def gpu_step(w: wl.Workload, gate_keys: torch.Tensor, gated: bool, budget: int | None = None, path="auto"):
    budget = budget or w.budget
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, budget, w.theta,
                            gated, device=w.q.device, path=path)
    dec.step(w.q, w.w_q, w.w_qnorm, gate_keys, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
    torch.cuda.synchronize()
    return dict(sel=wl.host(dec.sel), gates=wl.host(dec.gates), cnt=wl.host(dec.cnt),
                scores=wl.host(dec.scores), out=bf16_out(dec.out), gate_keys=wl.host(gate_keys))


def prefill_gate_keys(w: wl.Workload) -> torch.Tensor:
    """Gate keys of a prefill workload's complete blocks, pooled on the GPU."""
    dev = w.q.device
    nb = w.batch // 64
    gk = torch.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), dtype=torch.bfloat16, device=dev)
    shape1 = ops.make_shape(1, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
    if nb:
        ops.pool_blocks(shape1, w.k_pool, w.block_table[:1].contiguous(),
                        torch.zeros(nb, dtype=torch.int32, device=dev), torch.arange(nb, dtype=torch.int32, device=dev),
                        w.w_k, w.w_knorm, w.theta, gk)
    return gk


def gpu_prefill(w: wl.Workload, gk: torch.Tensor, gated: bool, budget: int, positions=None):
    """sas_prefill_select + sas_prefill_attend over the whole sequence; the
    results of `positions` (default all) copied to the host."""
    dev = w.q.device
    pf = ops.Prefill(w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, w.batch, budget, w.theta, gated,
                     device=dev, keep_scores=True)
    pf.forward(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table[0])
    torch.cuda.synchronize()
    idx = slice(None) if positions is None else torch.as_tensor(np.asarray(positions), device=dev)
    return dict(sel=wl.host(pf.sel[idx]), gates=wl.host(pf.gates[idx]), cnt=wl.host(pf.cnt[idx]),
                scores=wl.host(pf.scores[idx]), out=bf16_out(pf.out[idx]), gate_keys=wl.host(gk))


def bf16_out(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(wl.host(t))
