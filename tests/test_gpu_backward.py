"""Parity of sas_gate_backward (continuous-gate backward of a gated decode step)
with the oracle's fp64 backward.

Each side runs its own forward (pooling, gate scores, Top-K, gates); the
selections must agree without boundary ties (the seeds are chosen so), then
the GPU backward on the GPU's forward is compared with the oracle backward on
the oracle's forward, output by output.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import compare_selection, gpu_pool, shape_of
from harness import SM_SCALE, Host, oracle_gate_keys
from learned_block_sparse_tok_amd import ops
from learned_block_sparse_tok_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


BWD_CASES = [
    dict(name="paged_g4_ragged", lens=[3000, 700, 64, 1, 1500], Hq=8, Hkv=2, budget=512, layout="paged", mb=50,
         seed=61),
    dict(name="contig_g5", lens=[5000, 1500], Hq=10, Hkv=2, budget=1024, layout="contiguous", mb=None, seed=62),
    dict(name="paged_g4_b2048", lens=[12000, 9000, 4096], Hq=16, Hkv=4, budget=2048, layout="paged", mb=200,
         seed=63),
]


def close(got, want, rel, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    scale = max(float(np.abs(want).max()), 1e-30)
    err = np.abs(got - want)
    say(f"  {what}: max |err| / max |want| = {err.max() / scale:.2e}, mean {err.mean() / scale:.2e}")
    assert np.all(np.isfinite(got)), what
    assert err.max() <= rel * scale, (what, float(err.max() / scale))
    assert err.mean() <= 0.1 * rel * scale, (what, float(err.mean() / scale))


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: c["name"])
def test_gate_backward_parity(case):
    say("gate backward", case["name"])
    w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], case["budget"], case["layout"],
                case["seed"], DEV, max_blocks=case["mb"], random_norms=True, extra_pages=2)
    h = Host(w)
    budget, n_sel = case["budget"], case["budget"] // 64
    # forward, each side on its own
    gk_o = oracle_gate_keys(h)
    sel_o, gates_o, cnt_o, scores_o = oracle.gate_topk(h.q, h.w_q, h.wqn, gk_o, h.bt, h.lens, w.theta, budget,
                                                       w.n_kv_heads)
    gk_g = gpu_pool(w)
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, budget, w.theta, True,
                            device=DEV)
    dec.select(w.q, w.w_q, w.w_qnorm, gk_g, w.block_table, w.seq_lens)
    torch.cuda.synchronize()
    g = dict(sel=wl.host(dec.sel), gates=wl.host(dec.gates), cnt=wl.host(dec.cnt))
    o = dict(sel=sel_o, gates=gates_o, cnt=cnt_o, scores=scores_o)
    assert compare_selection(g, o, h.lens, budget) == []
    # backward
    gen = torch.Generator(device=DEV).manual_seed(case["seed"])
    d_out = torch.randn((w.batch, w.n_q_heads, 128), generator=gen, device=DEV).to(torch.bfloat16)
    bg = ops.gate_backward(shape_of(w), w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, dec.sel, dec.gates,
                           dec.cnt, n_sel, SM_SCALE, w.w_q, w.w_qnorm, w.w_k, w.w_knorm, gk_g, w.theta, d_out)
    torch.cuda.synchronize()
    bo = oracle.gate_backward(h.q, h.k, h.v, h.bt, w.strides, w.n_kv_heads, h.lens, sel_o, gates_o, cnt_o, SM_SCALE,
                              h.w_q, h.wqn, h.w_k, h.wkn, gk_o, w.theta, wl.host(d_out))
    # fp32 sums against fp64, and the two sides' bf16 gate keys may differ by
    # one rounding step (moving a score by ~1e-4 relative): 1e-3 of the
    # largest entry, 1e-4 on average
    for name in ("d_gates", "d_w_q", "d_w_qnorm", "d_w_k", "d_w_knorm"):
        close(wl.host(bg[name]), bo[name], 1e-3, name)
    # padding slots carry no gradient
    dgh = wl.host(bg["d_gates"])
    for s in range(w.batch):
        for k in range(w.n_kv_heads):
            assert np.all(dgh[s, k, g["cnt"][s, k]:] == 0)
    # a fixed summation order: the same inputs give the same bits
    bg2 = ops.gate_backward(shape_of(w), w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, dec.sel, dec.gates,
                            dec.cnt, n_sel, SM_SCALE, w.w_q, w.w_qnorm, w.w_k, w.w_knorm, gk_g, w.theta, d_out)
    torch.cuda.synchronize()
    for name in bg:
        assert torch.equal(bg[name], bg2[name]), name
