"""The parity comparator's tie path, on the CPU.

The GPU side is stood in for by the oracle run on a chosen selection, so that
the comparison logic itself is exercised: a selection that differs from the
oracle's only inside the boundary band (here an exact tie, made by giving two
blocks the same gate key) must pass and be counted as a tie, with its output
compared against the oracle's output for that resolution; a swap with a
candidate outside the band, a different number of band members, or an output
that belongs to another selection must fail.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from compare import compare_selection, compare_step, topk_band
from harness import SM_SCALE, Host, oracle_gate_keys, oracle_step
from learned_block_sparse_tok_amd import workloads as wl

BUDGET = 512  # 7 historical blocks + the local block


def _tied_workload(n_tied=2, above=0, boost_v=8.0):
    """A small paged workload whose unit (0, 0) has n_tied candidates with
    identical gate keys straddling the K-th place: the key of the oracle's
    K-th block copied to the `above` blocks ranked just before it and to the
    n_tied - 1 - above ranked just after it.  Their V rows are scaled by
    boost_v, so that taking one or another changes the output far beyond
    the tolerance."""
    w = wl.make(2, 8, 2, [1500, 900], BUDGET, "paged", 31, "cpu", max_blocks=24, random_norms=True,
                extra_pages=3)
    h = Host(w)
    gk = oracle_gate_keys(h)
    sel, _, cnt, scores = oracle.gate_topk(h.q, h.w_q, h.wqn, gk, h.bt, h.lens, w.theta, BUDGET, w.n_kv_heads)
    n = (int(h.lens[0]) - 1) // 64
    k = BUDGET // 64 - 1
    sc = scores[0, 0, :n].astype(np.float64)
    order = np.lexsort((np.arange(n), -sc))
    kth = int(order[k - 1])
    others = [int(c) for c in order[k - 1 - above:k - 1]] + [int(c) for c in order[k:k + n_tied - 1 - above]]
    for c in [kth] + others:
        page = int(h.bt[0, c])
        boosted = torch.as_tensor(oracle.bf16_to_f64(h.v[page, 0]) * boost_v).float()
        h.v[page, 0] = wl.bf16_bits(boosted.to(torch.bfloat16))
    for c in others:
        gk[int(h.bt[0, c]), 0] = gk[int(h.bt[0, kth]), 0]
    return w, h, gk, [kth] + others


def _as_gpu(h: Host, o: dict, sel: np.ndarray, gated: bool) -> dict:
    """A stand-in GPU result for selection sel: the oracle's gates of those
    blocks and the oracle's attention over them, output rounded to bf16."""
    w = h.w
    cnt = o["cnt"].copy()
    gates = np.zeros_like(sel, dtype=np.float32)
    for s in range(w.batch):
        n = (int(h.lens[s]) - 1) // 64
        for kvh in range(w.n_kv_heads):
            gates[s, kvh] = oracle.block_gates(o["scores"][s, kvh, :n], sel[s, kvh], int(cnt[s, kvh]))
    out = oracle.attend(h.q, h.k, h.v, h.bt, w.strides, w.n_kv_heads, h.lens, sel, gates if gated else None, cnt,
                        SM_SCALE)
    bits = np.vectorize(oracle.round_bf16, otypes=[np.uint16])(out)
    return dict(sel=sel, gates=gates, cnt=cnt, scores=o["scores"], out=oracle.bf16_to_f64(bits))


def _swap(sel_row: np.ndarray, k: int, drop: int, add: int) -> np.ndarray:
    row = sel_row.copy()
    hist = sorted((set(row[:k].tolist()) - {drop}) | {add})
    row[:k] = hist
    return row


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
def test_swap_inside_the_band_passes_and_is_counted(gated):
    w, h, gk, tied = _tied_workload()
    o = oracle_step(h, gated, BUDGET, gate_keys=gk)
    k = BUDGET // 64 - 1
    winner, loser = min(tied), max(tied)  # equal scores: the lower index wins
    assert winner in o["sel"][0, 0, :k] and loser not in o["sel"][0, 0, :k]
    _, band = topk_band(o["scores"][0, 0, :(int(h.lens[0]) - 1) // 64], k)
    assert set(tied) <= band
    sel = o["sel"].copy()
    sel[0, 0] = _swap(sel[0, 0], k, winner, loser)
    g = _as_gpu(h, o, sel, gated)
    assert np.abs(g["out"][0, :w.group] - o["out"][0, :w.group]).max() > 0.1  # the swap matters
    assert compare_step(h, g, o, gated, BUDGET) == 1
    assert compare_selection(g, o, h.lens, BUDGET) == [(0, 0)]


def test_swap_with_a_candidate_outside_the_band_fails():
    w, h, gk, tied = _tied_workload()
    o = oracle_step(h, True, BUDGET, gate_keys=gk)
    n = (int(h.lens[0]) - 1) // 64
    k = BUDGET // 64 - 1
    _, band = topk_band(o["scores"][0, 0, :n], k)
    outside = [c for c in range(n) if c not in band and c not in o["sel"][0, 0, :k]]
    sel = o["sel"].copy()
    sel[0, 0] = _swap(sel[0, 0], k, min(tied), outside[0])
    g = _as_gpu(h, o, sel, True)
    with pytest.raises(AssertionError):
        compare_selection(g, o, h.lens, BUDGET)
    with pytest.raises(AssertionError):
        compare_step(h, g, o, True, BUDGET)


def test_a_fixed_block_traded_for_a_band_member_fails():
    # the GPU keeps both tied blocks and drops a block the oracle holds
    # outside the band: the same count, but not a valid resolution
    w, h, gk, tied = _tied_workload()
    o = oracle_step(h, True, BUDGET, gate_keys=gk)
    n = (int(h.lens[0]) - 1) // 64
    k = BUDGET // 64 - 1
    _, band = topk_band(o["scores"][0, 0, :n], k)
    fixed = [c for c in o["sel"][0, 0, :k].tolist() if c not in band]
    sel = o["sel"].copy()
    sel[0, 0] = _swap(sel[0, 0], k, fixed[0], max(tied))
    g = _as_gpu(h, o, sel, True)
    with pytest.raises(AssertionError):
        compare_step(h, g, o, True, BUDGET)


def test_output_of_another_resolution_fails():
    # the GPU reports the swapped selection but the output of the oracle's own
    w, h, gk, tied = _tied_workload()
    o = oracle_step(h, True, BUDGET, gate_keys=gk)
    k = BUDGET // 64 - 1
    sel = o["sel"].copy()
    sel[0, 0] = _swap(sel[0, 0], k, min(tied), max(tied))
    g = _as_gpu(h, o, sel, True)
    g["out"] = _as_gpu(h, o, o["sel"], True)["out"]
    with pytest.raises(AssertionError):
        compare_step(h, g, o, True, BUDGET)


def test_a_wide_band_is_compared_not_skipped():
    # 12 candidates with one gate key around the K-th place, 4 of them within
    # the Top-K: C(12, 4) = 495 valid resolutions, more than one would
    # enumerate; the GPU stand-in takes the highest-index ones and its output
    # is still compared
    w, h, gk, tied = _tied_workload(n_tied=12, above=3, boost_v=1.0)
    o = oracle_step(h, True, BUDGET, gate_keys=gk)
    n = (int(h.lens[0]) - 1) // 64
    k = BUDGET // 64 - 1
    _, band = topk_band(o["scores"][0, 0, :n], k)
    assert len(band) >= 12
    fixed = set(o["sel"][0, 0, :k].tolist()) - band
    need = k - len(fixed)
    assert need >= 4
    take = sorted(band)[-need:]
    sel = o["sel"].copy()
    sel[0, 0, :k] = sorted(fixed | set(take))
    assert not np.array_equal(sel[0, 0], o["sel"][0, 0])
    g = _as_gpu(h, o, sel, True)
    assert compare_step(h, g, o, True, BUDGET) == 1
    g["out"][0, 0, 5] += 0.05  # a wrong output in the tied unit is caught
    with pytest.raises(AssertionError):
        compare_step(h, g, o, True, BUDGET)
