"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Stage tests feed both sides the same seeded inputs for one stage; whole-step
tests run pool -> select -> attend on each side from the same workload and
compare with tie accounting (selection bit-exact outside the 1e-3 boundary
band; outputs within max-abs 2e-2 / mean-abs 2e-3 of the fp64 oracle).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import (assert_out_close, bf16_out, compare_selection, compare_step, gpu_pool, gpu_prefill,
                         gpu_step, prefill_gate_keys, shape_of)
from harness import SM_SCALE, Host, complete_blocks, oracle_gate_keys, oracle_step
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


# ------------------------------------------------------------------ pooling
POOL_CASES = [
    dict(name="paged_ragged", lens=[300, 64, 1, 4097, 200], Hq=8, Hkv=2, layout="paged", mb=70),
    dict(name="contig_g4", lens=[4096, 777], Hq=4, Hkv=1, layout="contiguous", mb=None),
    dict(name="paged_8kv", lens=[2048, 1000, 130], Hq=32, Hkv=8, layout="paged", mb=40),
]


@pytest.mark.parametrize("case", POOL_CASES, ids=lambda c: c["name"])
def test_pool_blocks_parity(case):
    say("pool", case["name"])
    w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], 1024, case["layout"], 31, DEV,
                max_blocks=case["mb"], random_norms=True, extra_pages=3)
    h = Host(w)
    gk_o, f64, seq, blk = oracle_gate_keys(h, want_f64=True)
    gk_g = wl.host(gpu_pool(w))
    # pages outside the list stay untouched (zero)
    listed = np.zeros(w.n_pages, bool)
    listed[h.bt[seq, blk]] = True
    assert np.all(gk_g[~listed] == 0)
    # each key within one bf16 ulp of the oracle's unrounded fp64 key, plus the
    # fp32 error of the 384-term projection and the norm (keys have RMS ~1,
    # so an absolute 2e-5 bounds it): near-zero elements have ulps far below
    # that error and may round either way
    pages = h.bt[seq, blk]
    got = oracle.bf16_to_f64(gk_g[pages])
    ulp = 2.0 ** (np.floor(np.log2(np.abs(f64) + 1e-30)) - 7)
    excess = np.abs(got - f64) - ulp
    assert np.all(excess <= 2e-5), float(excess.max())
    flips = int(np.count_nonzero(gk_g[pages] != gk_o[pages]))
    say(f"  gate-key bf16 values differing from the oracle's rounding: {flips} of {gk_o[pages].size}")
    assert flips <= 0.01 * gk_o[pages].size


def test_pool_blocks_empty_list_is_noop():
    w = wl.make(1, 4, 1, 300, 1024, "paged", 32, DEV, max_blocks=5)
    gk = torch.full((w.n_pages, 1, 128), 7, dtype=torch.bfloat16, device=DEV)
    e = torch.zeros(0, dtype=torch.int32, device=DEV)
    ops.pool_blocks(shape_of(w), w.k_pool, w.block_table, e, e, w.w_k, w.w_knorm, w.theta, gk)
    torch.cuda.synchronize()
    assert torch.all(gk == 7)


# ------------------------------------------------------------------ cache write + incremental pooling
APPEND_CASES = [
    dict(name="paged", lens=[60, 1, 127, 4095, 200], Hq=8, Hkv=2, layout="paged", mb=70),
    dict(name="contig", lens=[63, 4000], Hq=4, Hkv=1, layout="contiguous", mb=66),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=lambda c: c["name"])
def test_append_kv_parity(case):
    """70 decode steps of sas_append_kv against the oracle's append: pools
    bit-exact, gate keys of the completed blocks within the pooling bar, and
    bit-identical to sas_pool_blocks over the same blocks."""
    steps = 70
    say("append", case["name"])
    w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], 1024, case["layout"], 33, DEV,
                max_blocks=case["mb"], random_norms=True, extra_pages=3)
    h = Host(w)
    Hkv = w.n_kv_heads
    _, k_new, v_new = wl.append_rows(w, steps, seed=34)
    kn_h, vn_h = wl.host(k_new), wl.host(v_new)
    shape = shape_of(w)
    gk = torch.zeros((w.n_pages, Hkv, wl.GATE_DIM), dtype=torch.bfloat16, device=DEV)
    gk_o = np.zeros((w.n_pages, Hkv, wl.GATE_DIM), np.uint16)
    k_o, v_o = h.k.copy(), h.v.copy()
    lens = h.lens.copy()
    seq_all, blk_all = [], []
    for step in range(steps):
        lens += 1
        w.seq_lens.copy_(torch.as_tensor(lens, device=DEV))
        ops.append_kv(shape, k_new[step], v_new[step], w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.w_k,
                      w.w_knorm, w.theta, gk)
        seq, blk = oracle.append_kv(k_o, v_o, h.bt, w.strides, Hkv, lens, kn_h[step], vn_h[step], h.w_k, h.wkn,
                                    w.theta, gk_o)
        seq_all += seq.tolist()
        blk_all += blk.tolist()
    torch.cuda.synchronize()
    say(f"  blocks completed and pooled: {list(zip(seq_all, blk_all))}")
    assert len(seq_all) >= 3
    np.testing.assert_array_equal(wl.host(w.k_pool), k_o)
    np.testing.assert_array_equal(wl.host(w.v_pool), v_o)
    gk_g = wl.host(gk)
    pages = h.bt[seq_all, blk_all]
    untouched = np.ones(w.n_pages, bool)
    untouched[pages] = False
    assert np.all(gk_g[untouched] == 0)
    f64 = oracle.pool_blocks(k_o, h.bt, w.strides, Hkv, np.array(seq_all, np.int32), np.array(blk_all, np.int32),
                             h.w_k, h.wkn, w.theta, np.zeros_like(gk_o), want_f64=True)
    got = oracle.bf16_to_f64(gk_g[pages])
    ulp = 2.0 ** (np.floor(np.log2(np.abs(f64) + 1e-30)) - 7)
    excess = np.abs(got - f64) - ulp
    assert np.all(excess <= 2e-5), float(excess.max())
    # the fused pooling is the same arithmetic as sas_pool_blocks
    gk2 = wl.host(gpu_pool(w, np.array(seq_all, np.int32), np.array(blk_all, np.int32)))
    np.testing.assert_array_equal(gk2[pages], gk_g[pages])


# ------------------------------------------------------------------ training-time forward (every position a query)
PREFILL_CASES = [
    dict(name="paged_g4_ragged", T=1000, Hq=8, Hkv=2, budget=256, layout="paged"),
    dict(name="contig_g1", T=700, Hq=2, Hkv=2, budget=192, layout="contiguous"),
    dict(name="paged_g5", T=640, Hq=10, Hkv=2, budget=128, layout="paged"),
    dict(name="paged_g16_tail1", T=577, Hq=16, Hkv=1, budget=320, layout="paged"),
    dict(name="full_budget", T=300, Hq=4, Hkv=1, budget=320, layout="paged"),
    dict(name="b4096_g2", T=1500, Hq=4, Hkv=2, budget=4096, layout="paged"),
    # 66 blocks, a ragged last one: the later query blocks' unions span two
    # 64-block pairing chunks, the second with one or two blocks (a pair
    # without its second block)
    dict(name="two_chunks_t4200", T=4200, Hq=4, Hkv=1, budget=512, layout="paged"),
]


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: c["name"])
def test_prefill_parity(case, gated):
    """sas_prefill_select + sas_prefill_attend against the oracle's forward at
    every position (several query blocks, a ragged last block, group sizes 1,
    2, 4, 5 and 16, budgets up to 4,096), with the decode path's tie
    accounting."""
    say("prefill", case["name"], "gated" if gated else "plain")
    w = wl.make_prefill(case["T"], case["Hq"], case["Hkv"], case["budget"], case["layout"], 41, DEV,
                        random_norms=True, extra_pages=2)
    h = Host(w)
    nb = w.batch // 64
    gk_o = np.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), np.uint16)
    oracle.pool_blocks(h.k, h.bt[:1], w.strides, w.n_kv_heads, np.zeros(nb, np.int32), np.arange(nb, dtype=np.int32),
                       h.w_k, h.wkn, w.theta, gk_o)
    sel, gates, cnt, scores, out = oracle.prefill(h.q, h.k, h.v, h.bt[0], w.strides, w.n_kv_heads, gk_o, h.w_q,
                                                  h.wqn, w.theta, case["budget"], gated, SM_SCALE)
    o = dict(gate_keys=gk_o, sel=sel, gates=gates, cnt=cnt, scores=scores, out=out)
    g = gpu_prefill(w, prefill_gate_keys(w), gated, case["budget"])
    ties = compare_step(h, g, o, gated, case["budget"])
    say(f"  boundary ties {ties}")


# ------------------------------------------------------------------ gate / Top-K
GATE_CASES = [
    dict(name="tiny_1024", lens=[4096], Hq=4, Hkv=1, budget=1024, mb=64),
    dict(name="b64_k0", lens=[1000, 5000], Hq=8, Hkv=2, budget=64, mb=80),
    dict(name="mixed_2048", lens=[32768, 1, 64, 65, 2048, 2049, 3000], Hq=16, Hkv=4, budget=2048, mb=512),
    dict(name="long_2047", lens=[131072, 70000], Hq=40, Hkv=8, budget=2048, mb=2048),
    dict(name="ragged_4096", lens=[4096, 65536, 12345, 40000], Hq=32, Hkv=8, budget=4096, mb=1026),
    dict(name="g16", lens=[9000, 600], Hq=16, Hkv=1, budget=1024, mb=150),
]


def _gate_inputs(case, seed):
    w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], case["budget"], "paged", seed, DEV,
                max_blocks=case["mb"], random_norms=True)
    gk = wl.random_gate_keys(w.n_pages, w.n_kv_heads, seed, DEV)
    return w, gk


def _gpu_gate(w, gk, budget):
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, budget, w.theta, True,
                            device=DEV)
    dec.select(w.q, w.w_q, w.w_qnorm, gk, w.block_table, w.seq_lens)
    torch.cuda.synchronize()
    return dict(sel=wl.host(dec.sel), gates=wl.host(dec.gates), cnt=wl.host(dec.cnt), scores=wl.host(dec.scores))


@pytest.mark.parametrize("case", GATE_CASES, ids=lambda c: c["name"])
def test_gate_topk_parity(case):
    say("gate", case["name"])
    w, gk = _gate_inputs(case, 41)
    h = Host(w)
    sel, gates, cnt, scores = oracle.gate_topk(h.q, h.w_q, h.wqn, wl.host(gk), h.bt, h.lens, w.theta,
                                               case["budget"], w.n_kv_heads)
    o = dict(sel=sel, gates=gates, cnt=cnt, scores=scores)
    g = _gpu_gate(w, gk, case["budget"])
    for s in range(w.batch):
        n = (int(h.lens[s]) - 1) // 64
        np.testing.assert_allclose(g["scores"][:, :, :][s, :, :n], scores[s, :, :n], rtol=1e-5, atol=1e-5)
        assert np.all(np.isneginf(g["scores"][s, :, n:]))
    ties = compare_selection(g, o, h.lens, case["budget"])
    say(f"  boundary ties: {len(ties)} of {w.batch * w.n_kv_heads}")
    tie_set = set(ties)
    for s in range(w.batch):
        for k in range(w.n_kv_heads):
            if (s, k) not in tie_set:
                c = cnt[s, k]
                np.testing.assert_allclose(g["gates"][s, k, :c], gates[s, k, :c], rtol=1e-5, atol=1e-6)
                assert np.all(g["gates"][s, k, c:] == 0)


def test_gate_topk_exact_ties_break_by_index():
    # many candidate blocks share one physical page: identical scores on both
    # sides, so the lower block index must win every tie, bit-exactly
    w = wl.make(3, 8, 2, [5000, 3000, 20000], 2048, "paged", 43, DEV, max_blocks=320)
    n_pages = w.n_pages
    bt = wl.host(w.block_table).copy()
    rng = np.random.default_rng(0)
    bt = rng.integers(0, 12, size=bt.shape).astype(np.int32)  # only 12 distinct pages
    w.block_table = torch.as_tensor(bt, device=DEV)
    gk = wl.random_gate_keys(n_pages, 2, 43, DEV)
    h = Host(w)
    sel, gates, cnt, scores = oracle.gate_topk(h.q, h.w_q, h.wqn, wl.host(gk), h.bt, h.lens, w.theta, 2048, 2)
    g = _gpu_gate(w, gk, 2048)
    for s in range(w.batch):
        for k in range(2):
            # the GPU's scores of equal pages are equal, so ties are exact on both sides
            n = (int(h.lens[s]) - 1) // 64
            gs = g["scores"][s, k, :n]
            for page in range(12):
                vals = gs[bt[s, :n] == page]
                assert len(set(vals.tolist())) <= 1
    ties = compare_selection(g, dict(sel=sel, gates=gates, cnt=cnt, scores=scores), h.lens, 2048)
    # equal-score groups straddle the threshold: the lower indices must win on both sides
    assert ties == []


# ------------------------------------------------------------------ attention
DEC_CASES = [
    dict(name="tiny_contig", lens=[4096], Hq=4, Hkv=1, budget=1024, layout="contiguous", mb=None),
    dict(name="ragged_paged", lens=[300, 64, 1, 4097, 200, 129], Hq=8, Hkv=2, budget=512, layout="paged", mb=70),
    dict(name="g5", lens=[9000, 20000], Hq=40, Hkv=8, budget=2048, layout="paged", mb=320),
    dict(name="g1", lens=[3000, 70], Hq=4, Hkv=4, budget=1024, layout="paged", mb=50),
    dict(name="g16", lens=[5000], Hq=16, Hkv=1, budget=4096, layout="contiguous", mb=None),
    dict(name="b32_h8", lens=[2500] * 32, Hq=32, Hkv=8, budget=2048, layout="paged", mb=40),
    dict(name="budget_ge_ctx", lens=[1500, 2000], Hq=8, Hkv=2, budget=4096, layout="paged", mb=32),
]


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: c["name"])
def test_sparse_decode_parity(case, gated):
    say("decode", case["name"], gated)
    w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], case["budget"], case["layout"], 51, DEV,
                max_blocks=case["mb"])
    h = Host(w)
    sel, gates, cnt = wl.random_selection(h.lens, w.n_kv_heads, case["budget"], seed=52)
    want = oracle.attend(h.q, h.k, h.v, h.bt, w.strides, w.n_kv_heads, h.lens, sel, gates if gated else None,
                         cnt, SM_SCALE)
    shape = shape_of(w)
    n_sel = case["budget"] // 64
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(ops.sparse_decode_workspace_bytes(shape, n_sel), dtype=torch.uint8, device=DEV)
    t_sel = torch.as_tensor(sel, device=DEV)
    t_gates = torch.as_tensor(gates, device=DEV) if gated else None
    ops.sparse_decode(shape, w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, t_sel, t_gates,
                      torch.as_tensor(cnt, device=DEV), n_sel, SM_SCALE, out, ws)
    torch.cuda.synchronize()
    mx, mean = assert_out_close(bf16_out(out), want)
    say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_sparse_decode_dense_equivalence_and_nan_rows():
    # budget >= context: every block is selected and the output equals dense
    # attention; NaN in the unused rows of the local page must not leak in
    w = wl.make(2, 8, 2, [1000, 63], 2048, "paged", 53, DEV, max_blocks=16)
    bt = wl.host(w.block_table)
    ps, ts, hs = w.strides
    for pool in (w.k_pool, w.v_pool):
        flat = pool.view(-1)
        for s, L in enumerate([1000, 63]):
            page = int(bt[s, (L - 1) // 64])
            for kvh in range(2):
                for r in range(L % 64, 64):
                    base = page * ps + kvh * hs + r * ts
                    flat[base:base + 128] = float("nan")
    h = Host(w)
    sel, gates, cnt = wl.random_selection(h.lens, 2, 2048, seed=1, full=True)
    want = oracle.attend(h.q, h.k, h.v, h.bt, w.strides, 2, h.lens, sel, None, cnt, SM_SCALE)
    shape = shape_of(w)
    out = torch.empty((2, 8, 128), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(ops.sparse_decode_workspace_bytes(shape, 32), dtype=torch.uint8, device=DEV)
    ops.sparse_decode(shape, w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, torch.as_tensor(sel, device=DEV),
                      None, torch.as_tensor(cnt, device=DEV), 32, SM_SCALE, out, ws)
    torch.cuda.synchronize()
    assert_out_close(bf16_out(out), want)


# ------------------------------------------------------------------ whole step
STEP_CASES = [
    dict(name="tiny_planted", named="tiny", budget=1024),
    dict(name="tiny_dense", named="tiny", budget=4096),
    dict(name="small_8b_like", lens=[8192] * 4, Hq=32, Hkv=8, budget=2048, layout="paged", mb=128),
    dict(name="small_4b_like", lens=[6000, 8192], Hq=32, Hkv=8, budget=2048, layout="contiguous", mb=None),
    dict(name="small_ragged", lens=[4096, 9000, 6543, 5000], Hq=32, Hkv=8, budget=4096, layout="paged", mb=150),
    dict(name="small_14b_like", lens=[20000], Hq=40, Hkv=8, budget=2048, layout="paged", mb=320, planted=8),
]


def _step_workload(case):
    if "named" in case:
        w = wl.named(case["named"], device=DEV, budget=case["budget"])
    else:
        w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], case["budget"], case["layout"], 61,
                    DEV, max_blocks=case["mb"], n_planted=case.get("planted", 0), plant_delta=3.0)
    from planting import plant
    plant(w)
    return w


# These few (sequence, KV head) pairs split over several workgroups each:
# "fused" (also what "auto" takes here) repeats the selection in every
# workgroup of a pair, "sliced" divides it among them, "two_launches"
# selects with one workgroup per pair.
@pytest.mark.parametrize("path", ["two_launches", "fused", "sliced"])
@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: c["name"])
def test_step_parity(case, gated, path):
    say("step", case["name"], gated, path)
    w = _step_workload(case)
    h = Host(w)
    o = oracle_step(h, gated, case["budget"])
    g = gpu_step(w, gpu_pool(w), gated, case["budget"], path=path)
    ties = compare_step(h, g, o, gated, case["budget"])
    say(f"  boundary ties {ties}")
    if w.planted is not None:
        for s in range(w.batch):
            for k in range(w.n_kv_heads):
                got = set(g["sel"][s, k, :g["cnt"][s, k]].tolist())
                assert set(w.planted[s, k].tolist()) <= got


# ------------------------------------------------------------------ fused step = two launches
# More (sequence, KV head) pairs than half the CUs: both paths attend with
# one workgroup per pair, so the fused launch must give the two launches'
# bits exactly (its selection and attention run the same arithmetic in the
# same order).  Ragged lengths cover an empty history (L <= 64), a selection
# shorter than the budget, several 512-candidate score passes and the
# largest budget.
FUSED_CASES = [
    dict(name="b17_ragged", lens=[1, 64, 65, 4097, 2048, 2049, 40000, 777, 12345, 3000, 130, 63, 8191, 8192, 33000,
                                  5000, 600], Hq=32, Hkv=8, budget=2048, mb=630),
    dict(name="b17_g5_b4096", lens=[70000, 1, 4096, 9000, 65, 30000, 2500, 128, 129, 60000, 7000, 500, 64, 20000,
                                    3333, 1234, 16384], Hq=40, Hkv=8, budget=4096, mb=1100),
    dict(name="b130_g1_b16384", lens=[100 + 811 * i for i in range(130)], Hq=1, Hkv=1, budget=16384, mb=1700),
    dict(name="b129_g16", lens=[1 + 97 * i for i in range(129)], Hq=16, Hkv=1, budget=1024, mb=200),
]
FUSED_OPTS = [("mean", False, "scale"), ("mean", True, "scale"), ("mean", True, "logit"), ("max", True, "scale"),
              ("max", False, "scale")]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: c["name"])
def test_fused_step_equals_two_launches(case):
    w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], case["budget"], "paged", 91, DEV,
                max_blocks=case["mb"])
    assert w.batch * w.n_kv_heads > 128
    gk = gpu_pool(w)
    args = (w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
    for aggregate, gated, gate_mode in FUSED_OPTS:
        if aggregate == "max" and w.n_q_heads // w.n_kv_heads > 8:
            continue
        say("fused", case["name"], aggregate, gated, gate_mode)
        res = {}
        for path in ("two_launches", "fused"):
            dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, case["budget"],
                                    w.theta, gated, device=DEV, aggregate=aggregate, gate_mode=gate_mode, path=path)
            dec.sel.fill_(-7)
            dec.gates.fill_(3.0)
            dec.out.zero_()
            dec.step(*args)
            torch.cuda.synchronize()
            res[path] = [t.clone() for t in (dec.sel, dec.gates, dec.cnt, dec.scores, dec.out)]
        for name, a, b in zip(("sel", "gates", "cnt", "scores", "out"), res["two_launches"], res["fused"]):
            assert torch.equal(a, b), name
        cnt = wl.host(res["fused"][2])
        assert cnt.min() >= 1 and cnt.max() <= case["budget"] // 64


# Fewer pairs than CUs: the sliced selection (several workgroups per pair,
# each keeping its slice's Top-K, then one merge) and the split fused step
# (each of a pair's workgroups repeating its selection) must give the two
# launches' bits exactly, since all three then attend with the same split.
SLICED_CASES = [
    dict(name="ragged_g4", lens=[1, 64, 65, 4097, 9000, 33000], Hq=8, Hkv=2, budget=1024, mb=520, layout="paged"),
    dict(name="b8_g4_32k", lens=[32768] * 8, Hq=32, Hkv=8, budget=2048, mb=512, layout="contiguous"),
    dict(name="b4_g5_131k", lens=[131072, 100000, 77777, 131000], Hq=40, Hkv=8, budget=2048, mb=2048,
         layout="paged"),
    dict(name="g16_b4096", lens=[20000, 700], Hq=16, Hkv=1, budget=4096, mb=320, layout="paged"),
    dict(name="b2_b16384", lens=[100000, 50000], Hq=4, Hkv=1, budget=16384, mb=1600, layout="paged"),
]


@pytest.mark.parametrize("case", SLICED_CASES, ids=lambda c: c["name"])
def test_sliced_step_equals_two_launches(case):
    w = wl.make(len(case["lens"]), case["Hq"], case["Hkv"], case["lens"], case["budget"], case["layout"], 93, DEV,
                max_blocks=case["mb"])
    assert w.batch * w.n_kv_heads <= 128
    gk = gpu_pool(w)
    args = (w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
    for aggregate, gated, gate_mode in FUSED_OPTS:
        if aggregate == "max" and w.n_q_heads // w.n_kv_heads > 8:
            continue
        say("sliced", case["name"], aggregate, gated, gate_mode)
        res = {}
        for path in ("two_launches", "sliced", "fused"):
            dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, case["budget"],
                                    w.theta, gated, device=DEV, aggregate=aggregate, gate_mode=gate_mode, path=path)
            dec.sel.fill_(-7)
            dec.gates.fill_(3.0)
            dec.scores.fill_(5.0)
            dec.out.zero_()
            dec.step(*args)
            torch.cuda.synchronize()
            res[path] = [t.clone() for t in (dec.sel, dec.gates, dec.cnt, dec.scores, dec.out)]
        for path in ("sliced", "fused"):
            for name, a, b in zip(("sel", "gates", "cnt", "scores", "out"), res["two_launches"], res[path]):
                assert torch.equal(a, b), (path, name)


@pytest.mark.parametrize("path", ["two_launches", "fused", "sliced"])
def test_step_short_sequence_with_nan_scores(path):
    """A NaN gate key gives a NaN score, which ranks as -inf and gets gate 0.
    Sequence 0 has 5 candidates (all selected, two of them NaN); in the
    sliced merge its 5 non-zero keys sit among zero padding with the NaN
    keys' top digit 0, the case where the select takes every non-zero key.
    Against the oracle on every path; sliced and two launches bit-equal."""
    w = wl.make(3, 8, 2, [321, 50000, 20000], 2048, "paged", 95, DEV, max_blocks=800)
    nan_blocks = [(0, 1), (0, 3), (2, 7), (1, 400)]
    bt = wl.host(w.block_table)
    gk = gpu_pool(w)
    h = Host(w)
    gk_o = oracle_gate_keys(h)
    for s, c in nan_blocks:
        gk[int(bt[s, c])] = float("nan")
        gk_o[int(bt[s, c])] = 0x7FC0
    for gated in (False, True):
        say("nan scores", path, gated)
        o = oracle_step(h, gated, 2048, gate_keys=gk_o)
        g = gpu_step(w, gk, gated, 2048, path=path)
        assert compare_step(h, g, o, gated, 2048) == 0
        assert list(g["sel"][0, 0, :6]) == [0, 1, 2, 3, 4, 5]
        assert g["gates"][0, 0, 1] == 0.0 and g["gates"][0, 0, 3] == 0.0
        if path == "sliced":
            ref = gpu_step(w, gk, gated, 2048, path="two_launches")
            for name in ("sel", "gates", "cnt", "out"):
                np.testing.assert_array_equal(g[name], ref[name])


def test_fused_step_without_scores_or_gates():
    # scores and (in plain mode) gates are optional outputs of the step
    w = wl.make(17, 32, 8, [3000 + 500 * i for i in range(17)], 2048, "paged", 92, DEV, max_blocks=180)
    gk = gpu_pool(w)
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, 2048, w.theta, False,
                            device=DEV, path="fused")
    dec.step(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dec.sel, dec.cnt, dec.out)]
    sel, cnt, out = torch.full_like(dec.sel, -7), torch.zeros_like(dec.cnt), torch.zeros_like(dec.out)
    ops.decode_step(dec.shape, w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.theta,
                    2048, sel, None, cnt, None, out, None, dec.sm_scale, False, path="fused")
    torch.cuda.synchronize()
    for a, b in zip(ref, (sel, cnt, out)):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ errors
VARIANTS = [("max", "scale"), ("mean", "logit"), ("max", "logit")]


@pytest.mark.parametrize("path", ["auto", "fused"])
@pytest.mark.parametrize("aggregate,gate_mode", VARIANTS, ids=[f"{a}-{m}" for a, m in VARIANTS])
@pytest.mark.parametrize("case", [STEP_CASES[0], STEP_CASES[4], STEP_CASES[5]], ids=lambda c: c["name"])
def test_step_parity_alternative_readings(case, aggregate, gate_mode, path):
    """The max-over-heads scores and the gate as a log-bias on the logits
    (sas_decode_step's options, as in sas_gate_topk_ex / sas_sparse_decode_ex)
    against the oracle run with the same options."""
    say("variant", case["name"], aggregate, gate_mode, path)
    w = _step_workload(case)
    h = Host(w)
    gk_o = oracle_gate_keys(h)
    sel, gates, cnt, scores = oracle.gate_topk(h.q, h.w_q, h.wqn, gk_o, h.bt, h.lens, w.theta, case["budget"],
                                               w.n_kv_heads, aggregate=aggregate)
    out = oracle.attend(h.q, h.k, h.v, h.bt, w.strides, w.n_kv_heads, h.lens, sel, gates, cnt, SM_SCALE,
                        gate_mode=gate_mode)
    o = dict(gate_keys=gk_o, sel=sel, gates=gates, cnt=cnt, scores=scores, out=out)
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, case["budget"], w.theta,
                            True, device=DEV, aggregate=aggregate, gate_mode=gate_mode, path=path)
    gk = gpu_pool(w)
    dec.step(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
    torch.cuda.synchronize()
    g = dict(sel=wl.host(dec.sel), gates=wl.host(dec.gates), cnt=wl.host(dec.cnt), scores=wl.host(dec.scores),
             out=bf16_out(dec.out), gate_keys=wl.host(gk))
    ties = compare_step(h, g, o, True, case["budget"], gate_mode=gate_mode)
    say(f"  boundary ties {ties}")


def test_invalid_arguments_raise():
    w = wl.make(1, 4, 1, 300, 1024, "paged", 71, DEV, max_blocks=5)
    shape = shape_of(w)
    dec = ops.SparseDecoder(1, 4, 1, 5, w.strides, 1024, w.theta, True, device=DEV)
    gk = torch.zeros((w.n_pages, 1, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.SasError) as ei:
        ops.gate_topk(shape, w.q, w.w_q, w.w_qnorm, gk, w.block_table, w.seq_lens, w.theta, 1000, dec.sel,
                      dec.gates, dec.cnt, dec.scores)
    assert ei.value.status == ops.SAS_ERR_INVALID_ARG
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ops.SasError) as ei:
        ops.sparse_decode(shape, w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, dec.sel, None, dec.cnt, 16,
                          SM_SCALE, dec.out, small)
    assert ei.value.status == ops.SAS_ERR_WORKSPACE
    with pytest.raises(TypeError):
        ops.sparse_decode(shape, w.q.float(), w.k_pool, w.v_pool, w.block_table, w.seq_lens, dec.sel, None,
                          dec.cnt, 16, SM_SCALE, dec.out, dec.ws_dec)


# ------------------------------------------------------------------ graphs, determinism
@pytest.mark.parametrize("path", ["two_launches", "fused", "sliced"])
def test_graph_replay_matches_eager(path):
    # the step captured into one HIP graph: every replay, with eager work and
    # synchronisations in between, reproduces the eager result bit for bit
    w = wl.make(4, 32, 8, [8192, 5000, 3000, 8192], 2048, "paged", 81, DEV, max_blocks=128)
    gk = gpu_pool(w)
    for gated in (False, True):
        dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, 2048, w.theta, gated,
                                device=DEV, path=path)
        args = (w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
        dec.step(*args)
        torch.cuda.synchronize()
        ref = [t.clone() for t in (dec.sel, dec.gates, dec.cnt, dec.out, dec.scores)]
        dec.step(*args)  # a second eager call: deterministic
        torch.cuda.synchronize()
        for a, b in zip(ref, (dec.sel, dec.gates, dec.cnt, dec.out, dec.scores)):
            assert torch.equal(a, b)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dec.step(*args)
        for r in range(4):
            dec.out.zero_()
            dec.sel.fill_(-7)
            dec.gates.fill_(3.0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for a, b in zip(ref, (dec.sel, dec.gates, dec.cnt, dec.out, dec.scores)):
                assert torch.equal(a, b), f"replay {r}"


@pytest.mark.parametrize("path", ["auto", "two_launches"])
def test_prepared_step_matches_step(path):
    # the step with its arguments marshalled once (as bench.py times it):
    # the same outputs as step(), eagerly and captured into a graph
    w = wl.make(4, 32, 8, [8192, 5000, 3000, 8192], 2048, "paged", 83, DEV, max_blocks=128)
    gk = gpu_pool(w)
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, 2048, w.theta, True,
                            device=DEV, path=path)
    args = (w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
    dec.step(*args)
    torch.cuda.synchronize()
    outs = (dec.sel, dec.gates, dec.cnt, dec.out, dec.scores)
    ref = [t.clone() for t in outs]
    call = dec.prepare_step(*args)
    for t in outs:
        t.zero_()
    call()
    torch.cuda.synchronize()
    for a, b in zip(ref, outs):
        assert torch.equal(a, b)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), f"replay {r}"
