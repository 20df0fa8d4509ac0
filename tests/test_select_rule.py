"""CPU replay of the wave radix select's threshold rule (select.h).

The kernel's Top-K finds a threshold key T digit by digit (8-bit digits,
most significant first) from histograms of the non-zero keys, then takes
every key above T and the lowest-index keys equal to T.  Key 0 is padding
(the sliced merge pads each slice's list with it; real keys are > 0).  This
replays that rule on the host, with 32-bit unsigned arithmetic, and checks it
against a brute-force Top-K on lists that include padding, keys below 2^24
(scores of -inf, NaN or below -2^127 map there) and ties.
"""
from __future__ import annotations

import numpy as np
import pytest

M32 = 0xFFFFFFFF


def replay(keys, k_eff, guarded=True):
    """Indices chosen by the kernel's rule, ascending."""
    n = len(keys)
    T, krem = 0, 0
    if 0 < k_eff < n:
        prefix = mask = 0
        krem = k_eff
        for shift in (24, 16, 8, 0):
            hist = [0] * 256
            for k in keys:
                if k != 0 and (k & mask) == prefix:
                    hist[(k >> shift) & 255] += 1
            run = 0
            found = None
            for d in range(255, -1, -1):  # digits in descending order
                if run < krem <= run + hist[d]:
                    found = d
                    break
                run += hist[d]
            assert found is not None, "no digit reaches the remaining count"
            krem -= run
            bin_cnt = hist[found]
            prefix |= found << shift
            mask |= 0xFF << shift
            if bin_cnt == krem:
                T = (prefix - 1 if prefix else 0) if guarded else (prefix - 1) & M32
                krem = 0
                break
            T = prefix
    if k_eff <= 0:
        return []
    chosen, eq_rank = [], 0
    for c, k in enumerate(keys):
        take = k > T
        if krem > 0 and k == T:
            take = eq_rank < krem
            eq_rank += 1
        if take:
            chosen.append(c)
    return chosen


def brute(keys, k_eff):
    nz = [(-int(k), c) for c, k in enumerate(keys) if k != 0]
    return sorted(c for _, c in sorted(nz)[:k_eff])


def key_of(score: float) -> int:
    """The kernel's order-preserving map of an fp32 score (NaN as -inf)."""
    s = np.float32(score)
    if np.isnan(s):
        s = np.float32(-np.inf)
    if s == 0:
        s = np.float32(0.0)
    u = int(s.view(np.uint32))
    return (~u) & M32 if u & 0x80000000 else u | 0x80000000


def test_key_map_orders_scores():
    vals = [-np.inf, -3e38, -2.0 ** 127, -1.0, -1e-40, -0.0, 0.0, 1e-40, 0.5, 1.0, 3e38, np.inf]
    keys = [key_of(v) for v in vals]
    assert all(a < b for a, b in zip(keys[:5], keys[1:6]))
    assert keys[5] == keys[6] and all(a < b for a, b in zip(keys[6:], keys[7:]))
    assert key_of(float("nan")) == key_of(-np.inf) < 1 << 24
    assert all(k > 0 for k in keys)


def test_padded_list_with_a_minus_inf_key():
    # three real keys (one from a -inf score) padded with zeros, all three taken
    keys = [key_of(0.5), key_of(-np.inf), key_of(1.0)] + [0] * 125
    assert replay(keys, 3) == brute(keys, 3) == [0, 1, 2]
    assert replay(keys, 3, guarded=False) == []  # the unguarded rule wraps T and takes nothing


@pytest.mark.parametrize("seed", range(40))
def test_random_lists_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    n_real = int(rng.integers(1, 300))
    scores = rng.normal(size=n_real).astype(np.float32)
    # special scores: -inf / NaN (keys below 2^24), huge negatives, ties
    n_spec = int(rng.integers(0, 6))
    for i in rng.choice(n_real, size=min(n_spec, n_real), replace=False):
        scores[i] = rng.choice([-np.inf, np.nan, -3e38, scores[0]])
    if n_real > 3 and rng.random() < 0.5:
        scores[: n_real // 3] = scores[0]  # a wide tie
    keys = [key_of(float(s)) for s in scores]
    pad = int(rng.integers(0, 200))
    is_pad = np.zeros(n_real + pad, bool)
    is_pad[rng.choice(n_real + pad, size=pad, replace=False)] = True
    it = iter(keys)
    full = [0 if p else next(it) for p in is_pad]
    for k_eff in sorted({1, 2, min(31, n_real), n_real, max(1, n_real // 2)}):
        if k_eff > n_real:
            continue
        assert replay(full, k_eff) == brute(full, k_eff), (seed, k_eff)


def test_nonzero_count_equal_to_k_with_padding_in_every_digit():
    # every real key below 2^24 (all digits of the first pass 0)
    keys = [key_of(-np.inf)] * 3 + [0] * 61 + [key_of(float("nan"))] + [0] * 63
    assert replay(keys, 4) == brute(keys, 4) == [0, 1, 2, 64]
