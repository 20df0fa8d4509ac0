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


# ------------------------------------------------------------------ backward of the training-time forward
PREFILL_BWD_CASES = [
    dict(name="paged_g4_t1000", T=1000, Hq=8, Hkv=2, budget=256, layout="paged", seed=71),
    dict(name="contig_g5_t700", T=700, Hq=10, Hkv=2, budget=512, layout="contiguous", seed=72),
    dict(name="paged_g1_t577", T=577, Hq=2, Hkv=2, budget=128, layout="paged", seed=73),
    dict(name="paged_g8_t900_b1024", T=900, Hq=16, Hkv=2, budget=1024, layout="paged", seed=74),
    dict(name="paged_g16_t300", T=300, Hq=16, Hkv=1, budget=192, layout="paged", seed=75),
    dict(name="one_block_t50", T=50, Hq=4, Hkv=1, budget=128, layout="paged", seed=76),
    dict(name="g2_full_budget_t1100_b4096", T=1100, Hq=4, Hkv=2, budget=4096, layout="contiguous", seed=77),
    # unions over two 64-block pairing chunks (66 blocks, ragged last one)
    dict(name="two_chunks_t4200", T=4200, Hq=4, Hkv=1, budget=512, layout="paged", seed=78),
]


def prefill_oracle_gates(o: dict, sel_g: np.ndarray, cnt: np.ndarray) -> np.ndarray:
    """The oracle's gates (sigmoid of its own scores) of the GPU's selection:
    the oracle's where the two selections agree, else recomputed per unit."""
    gates = o["gates"].copy()
    T, Hkv, _ = sel_g.shape
    for t in range(T):
        for k in range(Hkv):
            if not np.array_equal(sel_g[t, k], o["sel"][t, k]):
                gates[t, k] = oracle.block_gates(o["scores"][t, k], sel_g[t, k], int(cnt[t, k]))
    return gates


def gpu_prefill_backward(w, gk, budget, d_out, pf=None):
    """sas_prefill_select + gated sas_prefill_attend (with lse) +
    sas_prefill_gate_backward; returns (Prefill, dict of device gradients)."""
    if pf is None:
        pf = ops.Prefill(w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, w.batch, budget, w.theta, True,
                         device=DEV, keep_scores=True)
        pf.forward(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table[0])
    shape = ops.make_shape(1, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
    bg = ops.prefill_gate_backward(shape, w.q, w.k_pool, w.v_pool, w.block_table[0], w.batch, pf.sel, pf.gates,
                                   pf.cnt, budget // 64, SM_SCALE, pf.lse, w.w_q, w.w_qnorm, w.w_k, w.w_knorm, gk,
                                   w.theta, d_out)
    return pf, bg


@pytest.mark.parametrize("case", PREFILL_BWD_CASES, ids=lambda c: c["name"])
def test_prefill_gate_backward_parity(case):
    """sas_prefill_gate_backward against oracle.prefill_gate_backward at every
    position (several 64-position tiles, ragged last tile, groups of 1, 2, 4,
    5, 8 and 16 query heads, budgets 128 to 4,096 (the largest selecting every
    candidate), paged and contiguous, a sequence with no historical block).  Each side runs its own forward; the
    GPU's selection is validated against the oracle's (ties resolved inside
    the band are allowed) and the oracle's backward runs on it, with the
    oracle's own gates of those blocks."""
    from gpu_harness import prefill_gate_keys
    say("prefill gate backward", case["name"])
    w = wl.make_prefill(case["T"], case["Hq"], case["Hkv"], case["budget"], case["layout"], case["seed"], DEV,
                        random_norms=True, extra_pages=2)
    h = Host(w)
    budget = case["budget"]
    nb = w.batch // 64
    gk_o = np.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), np.uint16)
    oracle.pool_blocks(h.k, h.bt[:1], w.strides, w.n_kv_heads, np.zeros(nb, np.int32), np.arange(nb, dtype=np.int32),
                       h.w_k, h.wkn, w.theta, gk_o)
    sel_o, gates_o, cnt_o, scores_o, _ = oracle.prefill(h.q, h.k, h.v, h.bt[0], w.strides, w.n_kv_heads, gk_o,
                                                        h.w_q, h.wqn, w.theta, budget, True, SM_SCALE)
    gk_g = prefill_gate_keys(w)
    gen = torch.Generator(device=DEV).manual_seed(case["seed"])
    d_out = torch.randn((w.batch, w.n_q_heads, 128), generator=gen, device=DEV).to(torch.bfloat16)
    pf, bg = gpu_prefill_backward(w, gk_g, budget, d_out)
    torch.cuda.synchronize()
    sel_g, cnt_g = wl.host(pf.sel), wl.host(pf.cnt)
    o = dict(sel=sel_o, gates=gates_o, cnt=cnt_o, scores=scores_o)
    ties = compare_selection(dict(sel=sel_g, gates=wl.host(pf.gates), cnt=cnt_g), o, h.lens, budget)
    say(f"  boundary ties {len(ties)}")
    gates_for = prefill_oracle_gates(o, sel_g, cnt_g)
    bo = oracle.prefill_gate_backward(h.q, h.k, h.v, h.bt[0], w.strides, w.n_kv_heads, sel_g, gates_for, cnt_g,
                                      SM_SCALE, h.w_q, h.wqn, h.w_k, h.wkn, gk_o, w.theta, wl.host(d_out))
    for name in ("d_gates", "d_w_q", "d_w_qnorm", "d_w_k", "d_w_knorm"):
        if name in ("d_w_k", "d_w_knorm") and w.batch <= 64:
            # no position has a historical block: the key side is exactly zero
            assert not np.any(wl.host(bg[name])), name
            continue
        close(wl.host(bg[name]), bo[name], 1e-3, name)
    dgh = wl.host(bg["d_gates"])
    for t in range(w.batch):
        for k in range(w.n_kv_heads):
            assert np.all(dgh[t, k, cnt_g[t, k]:] == 0)
    # a fixed summation order: the same inputs give the same bits
    _, bg2 = gpu_prefill_backward(w, gk_g, budget, d_out, pf=pf)
    torch.cuda.synchronize()
    for name in bg:
        assert torch.equal(bg[name], bg2[name]), name
