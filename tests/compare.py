"""Parity comparison of a GPU result with the oracle's, with the tie
accounting of the Top-K (CPU only: numpy and the oracle).

Selection: bit-exact outside the boundary band of each (sequence, KV head);
inside it either side may take any of the tied candidates, but both take the
same number.  A unit whose set differs inside the band (a boundary tie) is
counted, and its outputs are compared with the oracle's output for the valid
resolution of the band that the GPU took: the oracle's own fixed part of the
selection (its Top-K minus the band) plus the band members the GPU took,
which compare_selection has checked to be a valid resolution.  Every unit's
output is compared; none is skipped.
"""
from __future__ import annotations

import numpy as np

import oracle
from harness import SM_SCALE, Host

TIE_REL = 1e-3       # boundary band: |S_c - S_K| <= 1e-3 * max(|S_K|, 1)
OUT_MAX_ABS = 2e-2   # attention outputs vs the fp64 oracle, bf16 inputs
OUT_MEAN_ABS = 2e-3


def topk_band(scores: np.ndarray, k: int):
    """K-th best oracle score under (score desc, index asc) and the tie band."""
    n = len(scores)
    order = np.lexsort((np.arange(n), -np.where(np.isnan(scores), -np.inf, scores).astype(np.float64)))
    sk = float(scores[order[k - 1]])
    tol = TIE_REL * max(abs(sk), 1.0)
    band = set(np.nonzero(np.abs(scores.astype(np.float64) - sk) <= tol)[0].tolist())
    return sk, band


def compare_selection(g: dict, o: dict, lens: np.ndarray, budget: int):
    """Selection parity: bit-exact outside the boundary band of each
    (sequence, KV head); inside it both sides must take the same number of
    candidates.  Returns the (s, kvh) pairs whose sets differ (ties)."""
    B, Hkv = o["cnt"].shape
    ties = []
    for s in range(B):
        n = (int(lens[s]) - 1) // 64
        k = min(budget // 64 - 1, n)
        for h in range(Hkv):
            assert g["cnt"][s, h] == o["cnt"][s, h] == k + 1, (s, h)
            gs, os_ = g["sel"][s, h], o["sel"][s, h]
            assert gs[k] == os_[k] == n and np.all(gs[k + 1:] == -1), (s, h)
            assert np.all(np.diff(gs[:k + 1]) > 0), (s, h)
            if np.array_equal(gs, os_):
                continue
            assert 0 < k < n, (s, h, gs, os_)
            _, band = topk_band(o["scores"][s, h, :n], k)
            gset, oset = set(gs[:k].tolist()), set(os_[:k].tolist())
            assert gset - band == oset - band, (s, h, sorted(gset ^ oset))
            assert len(gset & band) == len(oset & band), (s, h)
            ties.append((s, h))
    return ties


def band_resolution(o: dict, s: int, kvh: int, n: int, k: int, gsel: np.ndarray) -> list:
    """The valid resolution of (s, kvh)'s tie band that the GPU took, built on
    the oracle's side: its selection outside the band plus the band members
    in gsel.  Raises if gsel is not such a resolution."""
    _, band = topk_band(o["scores"][s, kvh, :n], k)
    fixed = set(o["sel"][s, kvh, :k].tolist()) - band
    taken = band & set(gsel[:k].tolist())
    chosen = sorted(fixed | taken)
    if len(chosen) != k or chosen != sorted(gsel[:k].tolist()):
        raise AssertionError(f"GPU selection of ({s}, {kvh}) is not a valid resolution of the tie band")
    return chosen


def resolved_outputs(h: Host, o: dict, s: int, kvh: int, gsel: np.ndarray, gated: bool, budget: int,
                     gate_mode: str = "scale"):
    """Oracle outputs of the G query heads of (s, kvh) under the resolution
    of its tie band that the GPU took (band_resolution), with the oracle's
    gates of those blocks."""
    w = h.w
    n = (int(h.lens[s]) - 1) // 64
    k = min(budget // 64 - 1, n)
    chosen = band_resolution(o, s, kvh, n, k, gsel)
    n_sel = budget // 64
    sel = np.full((w.batch, w.n_kv_heads, n_sel), -1, np.int32)
    cnt = np.ones((w.batch, w.n_kv_heads), np.int32)
    sel[:, :, 0] = 0
    sel[s, kvh, :k] = chosen
    sel[s, kvh, k] = n
    cnt[s, kvh] = k + 1
    gates = np.zeros_like(sel, dtype=np.float32)
    gates[s, kvh] = oracle.block_gates(o["scores"][s, kvh, :n], sel[s, kvh], k + 1)
    pairs = np.array([[s, kvh * w.group + g] for g in range(w.group)], np.int32)
    out = oracle.attend(h.q, h.k, h.v, h.bt, w.strides, w.n_kv_heads, h.lens, sel, gates if gated else None, cnt,
                        SM_SCALE, pairs=pairs, gate_mode=gate_mode)
    return out, gates[s, kvh, :k + 1]


SCORE_ATOL = 2e-5  # fp32 gate query and score arithmetic on identical gate keys (the stage bar is 1e-5)


def gate_tolerance(gk_gpu: np.ndarray, gk_oracle: np.ndarray, pages: np.ndarray, kvh: int, wqn) -> np.ndarray:
    """Largest gate difference the two sides' own gate keys allow, per block.

    Each side pools its own gate keys; they may differ by bf16 rounding flips
    (the pooling bar).  With d = the difference of one block's two keys, the
    score moves by |<g, d>| / sqrt(128) <= ||g|| ||d|| / sqrt(128), and the
    gate query g (a mean or one of the group's rotated, RMS-normalised,
    w_qnorm-scaled queries) has ||g|| <= sqrt(128) max|w_qnorm|; the sigmoid's
    slope is at most 1/4.  So |dg| <= (max|w_qnorm| ||d|| + SCORE_ATOL) / 4,
    plus the fp32 sigmoid's own error."""
    a, b = gk_gpu[pages, kvh], gk_oracle[pages, kvh]
    d = np.where(a == b, 0.0, oracle.bf16_to_f64(a) - oracle.bf16_to_f64(b))  # equal bits (NaN too): 0
    delta = np.linalg.norm(d.reshape(len(pages), -1), axis=1)
    return 0.25 * (float(np.max(np.abs(wqn))) * delta + SCORE_ATOL) + 1e-6


def check_gates(got: np.ndarray, want: np.ndarray, sel_row: np.ndarray, cnt: int, bt_row: np.ndarray, kvh: int,
                wqn, gk_gpu=None, gk_oracle=None, gate_atol: float = 2e-4, what=""):
    """Gates of one unit's cnt selected blocks (the last local, gate 1)."""
    if gk_gpu is None:
        np.testing.assert_allclose(got[:cnt], want[:cnt], rtol=0, atol=gate_atol, err_msg=what)
        return
    tol = np.full(cnt, 1e-6)
    if cnt > 1:
        tol[:cnt - 1] = gate_tolerance(gk_gpu, gk_oracle, bt_row[sel_row[:cnt - 1]], kvh, wqn)
    err = np.abs(got[:cnt].astype(np.float64) - want[:cnt].astype(np.float64))
    assert np.all(err <= tol), (what, err.max(), tol[np.argmax(err - tol)])


def assert_out_close(got: np.ndarray, want: np.ndarray, what=""):
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), what
    assert err.max() <= OUT_MAX_ABS, (what, float(err.max()))
    assert err.mean() <= OUT_MEAN_ABS, (what, float(err.mean()))
    return float(err.max()), float(err.mean())


def compare_step(h: Host, g: dict, o: dict, gated: bool, budget: int, gate_atol: float = 2e-4,
                 gate_mode: str = "scale") -> int:
    """Whole-step parity with tie accounting; returns the number of boundary
    ties.  Gates: when g carries the GPU's own gate keys (g["gate_keys"],
    host uint16 [P][Hkv][128]) and o the oracle's, each block's gate within
    the bound its two keys allow (gate_tolerance); otherwise within
    gate_atol."""
    w = h.w
    ties = compare_selection(g, o, h.lens, budget)
    tie_set = set(ties)
    mask = np.ones((w.batch, w.n_q_heads), bool)
    compared = 0
    gk_g, gk_o = g.get("gate_keys"), o.get("gate_keys")
    if gk_o is None:
        gk_g = None
    for (s, kvh) in ties:
        heads = slice(kvh * w.group, (kvh + 1) * w.group)
        mask[s, heads] = False
        alt, alt_gates = resolved_outputs(h, o, s, kvh, g["sel"][s, kvh], gated, budget, gate_mode=gate_mode)
        assert_out_close(g["out"][s, heads], alt, f"tie-resolved output s={s} kvh={kvh}")
        check_gates(g["gates"][s, kvh], alt_gates, g["sel"][s, kvh], len(alt_gates), h.bt[s], kvh, h.wqn, gk_g, gk_o,
                    gate_atol, f"gates s={s} kvh={kvh}")
        compared += w.group
    if mask.any():
        assert_out_close(g["out"][mask], o["out"][mask], "output")
        compared += int(mask.sum())
    assert compared == w.batch * w.n_q_heads  # every (sequence, query head) compared
    # gates of the blocks both sides selected
    for s in range(w.batch):
        for kvh in range(w.n_kv_heads):
            if (s, kvh) in tie_set:
                continue
            c = int(o["cnt"][s, kvh])
            check_gates(g["gates"][s, kvh], o["gates"][s, kvh], o["sel"][s, kvh], c, h.bt[s], kvh, h.wqn, gk_g,
                        gk_o, gate_atol, f"gates s={s} kvh={kvh}")
    return len(ties)
