"""Parity at the benchmark workloads' full sizes, on sampled sequences.

The GPU runs the whole path over the full batch in the launch configuration
the benchmark times (sas_pool_blocks over every complete block, then
sas_gate_topk + sas_sparse_decode through SparseDecoder).  The oracle then
recomputes sampled sequences one by one from host copies of their pages --
pooling, gate scores, full sort, dense masked attention -- and the two are
compared with the same tie accounting as the small-size tests.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import dataclasses

from compare import check_gates
from gpu_harness import (assert_out_close, bf16_out, compare_selection, compare_step, gpu_pool, gpu_prefill,
                         prefill_gate_keys)
from harness import SM_SCALE, Host, complete_blocks, oracle_step
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


def sub_workload(w: wl.Workload, seqs) -> wl.Workload:
    """The sampled sequences as a workload of their own: their pages gathered
    into a compact pool with an identity block table (host-side input
    marshalling for the oracle; no arithmetic)."""
    seqs = list(seqs)
    bt = w.block_table[seqs]  # [n][max_blocks]
    pages = bt.reshape(-1).long()
    per_page = w.k_pool.numel() // w.n_pages
    k = w.k_pool.view(w.n_pages, per_page).index_select(0, pages)
    v = w.v_pool.view(w.n_pages, per_page).index_select(0, pages)
    n = len(seqs)
    if w.layout == "contiguous":
        shape = (n, w.max_blocks * wl.BLOCK, w.n_kv_heads, wl.HEAD_DIM)
    else:
        shape = (n * w.max_blocks, w.n_kv_heads, wl.BLOCK, wl.HEAD_DIM)
    return wl.Workload(name=w.name + "_sample", batch=n, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                       max_blocks=w.max_blocks, layout=w.layout, budget=w.budget, theta=w.theta,
                       seq_lens=w.seq_lens[seqs].clone(), q=w.q[seqs].clone(), k_pool=k.reshape(shape),
                       v_pool=v.reshape(shape),
                       block_table=torch.arange(n * w.max_blocks, dtype=torch.int32, device=w.q.device).reshape(
                           n, w.max_blocks),
                       w_q=w.w_q, w_k=w.w_k, w_qnorm=w.w_qnorm, w_knorm=w.w_knorm, strides=w.strides)


def gpu_full_step(w, gk, gated, budget):
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, budget, w.theta, gated,
                            device=DEV)
    dec.step(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
    torch.cuda.synchronize()
    return dec


def gpu_sample(dec, seqs):
    seqs = list(seqs)
    return dict(sel=wl.host(dec.sel)[seqs], gates=wl.host(dec.gates)[seqs], cnt=wl.host(dec.cnt)[seqs],
                scores=wl.host(dec.scores)[seqs], out=bf16_out(dec.out)[seqs])


def check_sampled(w, dec, seqs, gated, budget, gk):
    """The sampled sequences' whole step against the oracle's (its own
    pooling of their blocks); the GPU's gate keys of those blocks, in the
    sub-workload's page order, bound the gate differences."""
    sub = sub_workload(w, seqs)
    h = Host(sub)
    o = oracle_step(h, gated, budget)
    g = gpu_sample(dec, seqs)
    g["gate_keys"] = wl.host(gk)[wl.host(w.block_table)[list(seqs)].reshape(-1)]
    return compare_step(h, g, o, gated, budget)


def check_every_unit(w, dec, budget, gk):
    """Selection of every (sequence, KV head) of the full batch against the
    oracle's gate stage: the oracle pools every complete block from a host
    copy of K and runs its gate scores and full sort; sel and cnt must match
    bit for bit outside the boundary band (compare_selection), and the gates
    of every selected block within the stage tolerance (for a tie unit, the
    oracle's gates of the band resolution the GPU took).  Returns the ties."""
    lens = wl.host(w.seq_lens).astype(np.int32)
    k_host = wl.host(w.k_pool)
    bt = wl.host(w.block_table)
    gk_o = np.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), np.uint16)
    seq, blk = complete_blocks(lens)
    oracle.pool_blocks(k_host, bt, w.strides, w.n_kv_heads, seq, blk, wl.host(w.w_k), wl.host(w.w_knorm), w.theta,
                       gk_o)
    del k_host
    gk_g = wl.host(gk)
    wqn = wl.host(w.w_qnorm)
    sel, gates, cnt, scores = oracle.gate_topk(wl.host(w.q), wl.host(w.w_q), wl.host(w.w_qnorm), gk_o, bt, lens,
                                               w.theta, budget, w.n_kv_heads)
    o = dict(sel=sel, gates=gates, cnt=cnt, scores=scores)
    g = dict(sel=wl.host(dec.sel), gates=wl.host(dec.gates), cnt=wl.host(dec.cnt))
    ties = compare_selection(g, o, lens, budget)
    tie_set = set(ties)
    for s in range(w.batch):
        n = (int(lens[s]) - 1) // 64
        for kvh in range(w.n_kv_heads):
            c = int(cnt[s, kvh])
            want = gates[s, kvh]
            if (s, kvh) in tie_set:
                want = oracle.block_gates(scores[s, kvh, :n], g["sel"][s, kvh], c)
            check_gates(g["gates"][s, kvh], want, g["sel"][s, kvh], c, bt[s], kvh, wqn, gk_g, gk_o,
                        what=f"gates s={s} kvh={kvh}")
    say(f"  every unit's selection: {w.batch * w.n_kv_heads} units, boundary ties {len(ties)}")
    return ties


FULL = [
    ("qwen3_4b", 2048, [0, 5]),
    ("qwen3_8b", 1024, [0, 17, 31]),
    ("qwen3_8b", 2048, [3, 30]),
    ("qwen3_8b", 4096, [11, 26]),
]


@pytest.mark.parametrize("name,budget,seqs", FULL, ids=[f"{n}-{b}" for n, b, _ in FULL])
def test_full_size_sampled_parity(name, budget, seqs):
    w = wl.named(name, device=DEV, budget=budget)
    gk = gpu_pool(w)
    for gated in (False, True):
        say(f"{name} budget {budget} {'gated' if gated else 'plain'}: sequences {seqs}")
        dec = gpu_full_step(w, gk, gated, budget)
        ties = check_sampled(w, dec, seqs, gated, budget, gk)
        say(f"  boundary ties {ties}")
        # every unit of the full batch selected exactly budget/64 blocks
        assert np.all(wl.host(dec.cnt) == budget // 64)
        assert np.all(np.isfinite(bf16_out(dec.out)))
        if gated:  # the selection is the same in both modes: check every unit once
            check_every_unit(w, dec, budget, gk)


def test_full_size_qwen3_14b_planted_recall():
    from planting import plant
    w = wl.named("qwen3_14b", device=DEV)
    plant(w)
    gk = gpu_pool(w)
    dec = gpu_full_step(w, gk, True, 2048)
    sel, cnt = wl.host(dec.sel), wl.host(dec.cnt)
    hit = tot = 0
    for s in range(w.batch):
        for k in range(w.n_kv_heads):
            chosen = set(sel[s, k, :cnt[s, k]].tolist())
            hit += len(chosen & set(w.planted[s, k].tolist()))
            tot += w.planted.shape[2]
    say(f"qwen3_14b planted recall {hit}/{tot}")
    assert hit == tot
    check_every_unit(w, dec, 2048, gk)
    ties = check_sampled(w, dec, [1], True, 2048, gk)
    say(f"  boundary ties {ties}")


@pytest.mark.parametrize("fused", [False, True], ids=["scatter_then_pool", "append_kv"])
def test_ragged_incremental_serving(fused):
    """64 ragged sequences, 128 decode steps: append one token per sequence,
    pool every block the new token completes, select, attend -- the append
    either as a tensor scatter followed by sas_pool_blocks over the completed
    blocks, or as the fused sas_append_kv.  Sampled sequences are checked
    against the oracle at the first, a middle and the last step; the
    incrementally pooled gate keys against the oracle's pooling of the same
    blocks."""
    steps = 128
    w = wl.named("ragged", device=DEV, steps=steps)
    shape = ops.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
    gk = gpu_pool(w)
    q_new, k_new, v_new = wl.append_rows(w, steps, seed=55)
    lens = wl.host(w.seq_lens).astype(np.int64)
    bt = wl.host(w.block_table)
    ps, ts, hs = w.strides
    dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, w.budget, w.theta, True,
                            device=DEV)
    kflat, vflat = w.k_pool.view(-1), w.v_pool.view(-1)
    dims = torch.arange(wl.HEAD_DIM, device=DEV)
    heads = torch.arange(w.n_kv_heads, device=DEV)
    pooled_seq, pooled_blk = [], []
    check_at = {0, steps // 2, steps - 1}
    for step in range(steps):
        # the new token goes to position L (its K/V rows), then L += 1
        pos = lens.copy()
        lens += 1
        w.seq_lens.copy_(torch.as_tensor(lens.astype(np.int32)))
        w.q.copy_(q_new[step])
        done = np.nonzero(lens % 64 == 0)[0].astype(np.int32)
        blk = (lens[done] // 64 - 1).astype(np.int32)
        if fused:
            ops.append_kv(shape, k_new[step], v_new[step], w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.w_k,
                          w.w_knorm, w.theta, gk)
        else:
            page = bt[np.arange(w.batch), pos // 64].astype(np.int64)
            base = torch.as_tensor(page * ps + (pos % 64) * ts, device=DEV)
            idx = base[:, None, None] + heads[None, :, None] * hs + dims[None, None, :]
            kflat[idx] = k_new[step]
            vflat[idx] = v_new[step]
            if len(done):
                ops.pool_blocks(shape, w.k_pool, w.block_table, torch.as_tensor(done, device=DEV),
                                torch.as_tensor(blk, device=DEV), w.w_k, w.w_knorm, w.theta, gk)
        pooled_seq += done.tolist()
        pooled_blk += blk.tolist()
        dec.step(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
        if step in check_at:
            torch.cuda.synchronize()
            seqs = [step % 64, (step * 7 + 3) % 64]
            say(f"ragged step {step}: sequences {seqs} lengths {lens[seqs].tolist()}")
            ties = check_sampled(w, dec, seqs, True, w.budget, gk)
            say(f"  boundary ties {ties}")
            check_every_unit(w, dec, w.budget, gk)
    # incrementally pooled keys vs the oracle's pooling of the same blocks
    # (their pages gathered into a compact pool; block indices kept, since
    # they set the gate-key RoPE position)
    assert len(pooled_seq) > 0
    torch.cuda.synchronize()
    n = len(pooled_seq)
    pages = bt[pooled_seq, pooled_blk].astype(np.int64)
    per_page = w.k_pool.numel() // w.n_pages
    k_sub = wl.host(w.k_pool.view(w.n_pages, per_page).index_select(0, torch.as_tensor(pages, device=DEV)))
    bt_sub = np.zeros((n, w.max_blocks), np.int32)
    bt_sub[np.arange(n), pooled_blk] = np.arange(n)
    gk_o = np.zeros((n, w.n_kv_heads, 128), np.uint16)
    oracle.pool_blocks(k_sub, bt_sub, w.strides, w.n_kv_heads, np.arange(n, dtype=np.int32),
                       np.array(pooled_blk, np.int32), wl.host(w.w_k), wl.host(w.w_knorm), w.theta, gk_o)
    got = oracle.bf16_to_f64(wl.host(gk)[pages])
    want = oracle.bf16_to_f64(gk_o)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(want) + 1e-30)) - 7)
    assert np.all(np.abs(got - want) <= ulp + 2e-5)
    say(f"ragged: {n} blocks pooled incrementally")


def test_prefill_full_size_sampled_parity():
    """Training-time forward of one 32,768-token sequence with Qwen3-8B heads
    (32/8) at the 2,048 budget, in the launch configuration the benchmark
    times; sampled positions (first and last of blocks, the first complete
    candidate, the end) checked against the oracle's forward at those
    positions, both modes."""
    w = wl.named("prefill_8b", device=DEV)
    T = w.batch
    gk = prefill_gate_keys(w)
    pos = np.array([0, 63, 64, 127, 128, 1000, 4095, 4096, 20000, 32766, 32767])
    # the oracle sees the sampled positions as a batch sharing the one cache
    sub = dataclasses.replace(w, batch=len(pos), q=w.q[torch.as_tensor(pos, device=DEV)],
                              seq_lens=torch.as_tensor(pos + 1, dtype=torch.int32, device=DEV),
                              block_table=w.block_table[:len(pos)])
    h = Host(sub)
    nb = T // 64
    gk_o = np.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), np.uint16)
    oracle.pool_blocks(h.k, h.bt[:1], w.strides, w.n_kv_heads, np.zeros(nb, np.int32), np.arange(nb, dtype=np.int32),
                       h.w_k, h.wkn, w.theta, gk_o)
    for gated in (False, True):
        say(f"prefill_8b T={T} {'gated' if gated else 'plain'}: positions {pos.tolist()}")
        g = gpu_prefill(w, gk, gated, w.budget, positions=pos)
        sel, gates, cnt, scores, out = oracle.prefill(wl.host(w.q), h.k, h.v, h.bt[0], w.strides, w.n_kv_heads, gk_o,
                                                      h.w_q, h.wqn, w.theta, w.budget, gated, SM_SCALE, positions=pos)
        o = dict(gate_keys=gk_o, sel=sel, gates=gates, cnt=cnt, scores=scores, out=out)
        ties = compare_step(h, g, o, gated, w.budget)
        say(f"  boundary ties {ties}")
    # the selection of every 8th position (4,096 positions x 8 KV heads)
    # against the oracle's gate stage
    every = np.arange(3, T, 8)
    g = gpu_prefill(w, gk, True, w.budget, positions=every)
    bt_all = np.ascontiguousarray(np.broadcast_to(h.bt[0], (len(every), h.bt.shape[1])))
    lens = (every + 1).astype(np.int32)
    sel, gates, cnt, scores = oracle.gate_topk(wl.host(w.q)[every], h.w_q, h.wqn, gk_o, bt_all, lens, w.theta,
                                               w.budget, w.n_kv_heads)
    ties = compare_selection(g, dict(sel=sel, gates=gates, cnt=cnt, scores=scores), lens, w.budget)
    tie_set = set(ties)
    for i in range(len(every)):
        for kvh in range(w.n_kv_heads):
            c = int(cnt[i, kvh])
            want = gates[i, kvh] if (i, kvh) not in tie_set else oracle.block_gates(
                scores[i, kvh, :(int(lens[i]) - 1) // 64], g["sel"][i, kvh], c)
            check_gates(g["gates"][i, kvh], want, g["sel"][i, kvh], c, h.bt[0], kvh, h.wqn, g["gate_keys"], gk_o,
                        what=f"gates position {every[i]} kvh={kvh}")
    say(f"  selection of {len(every)} positions x {w.n_kv_heads} KV heads: boundary ties {len(ties)}")


def test_gate_backward_full_size():
    """sas_gate_backward on the qwen3_8b decode workload (32 sequences, 32K
    context, budget 2048): d_gates of sampled sequences and every output of a
    two-sequence sub-batch against the oracle, and the batch sums checked by
    linearity (the full batch equals the sum over its two halves)."""
    from test_gpu_backward import close
    w = wl.named("qwen3_8b", device=DEV)
    n_sel = w.budget // 64
    gk = gpu_pool(w)
    gen = torch.Generator(device=DEV).manual_seed(77)
    d_out = torch.randn((w.batch, w.n_q_heads, 128), generator=gen, device=DEV).to(torch.bfloat16)

    def run(sub):
        dec = ops.SparseDecoder(sub.batch, sub.n_q_heads, sub.n_kv_heads, sub.max_blocks, sub.strides, w.budget,
                                w.theta, True, device=DEV)
        gks = gpu_pool(sub)
        dec.select(sub.q, sub.w_q, sub.w_qnorm, gks, sub.block_table, sub.seq_lens)
        shape = ops.make_shape(sub.batch, sub.n_q_heads, sub.n_kv_heads, sub.max_blocks, sub.strides)
        return dec, ops.gate_backward(shape, sub.q, sub.k_pool, sub.v_pool, sub.block_table, sub.seq_lens, dec.sel,
                                      dec.gates, dec.cnt, n_sel, SM_SCALE, sub.w_q, sub.w_qnorm, sub.w_k,
                                      sub.w_knorm, gks, w.theta, d_out[torch.as_tensor(sub_idx[id(sub)], device=DEV)])

    sub_idx = {}

    def subset(seqs):
        sub = sub_workload(w, seqs)
        sub_idx[id(sub)] = list(seqs)
        return sub

    full = dataclasses.replace(w)
    sub_idx[id(full)] = list(range(w.batch))
    dec_f, bf = run(full)
    lo, hi = subset(range(0, 16)), subset(range(16, 32))
    _, b_lo = run(lo)
    _, b_hi = run(hi)
    torch.cuda.synchronize()
    for name in ("d_w_q", "d_w_qnorm", "d_w_k", "d_w_knorm"):
        close(wl.host(bf[name]), wl.host(b_lo[name]).astype(np.float64) + wl.host(b_hi[name]), 1e-5, name + " (halves)")
    # two sampled sequences against the oracle
    seqs = [3, 30]
    two = subset(seqs)
    dec2, b2 = run(two)
    torch.cuda.synchronize()
    h = Host(two)
    gk_o = np.zeros((two.n_pages, two.n_kv_heads, 128), np.uint16)
    from harness import complete_blocks
    cs, cb = complete_blocks(h.lens)
    oracle.pool_blocks(h.k, h.bt, two.strides, two.n_kv_heads, cs, cb, h.w_k, h.wkn, w.theta, gk_o)
    sel, gates, cnt, scores = oracle.gate_topk(h.q, h.w_q, h.wqn, gk_o, h.bt, h.lens, w.theta, w.budget,
                                               w.n_kv_heads)
    from gpu_harness import compare_selection
    g = dict(sel=wl.host(dec2.sel), gates=wl.host(dec2.gates), cnt=wl.host(dec2.cnt))
    assert compare_selection(g, dict(sel=sel, gates=gates, cnt=cnt, scores=scores), h.lens, w.budget) == []
    bo = oracle.gate_backward(h.q, h.k, h.v, h.bt, two.strides, two.n_kv_heads, h.lens, sel, gates, cnt, SM_SCALE,
                              h.w_q, h.wqn, h.w_k, h.wkn, gk_o, w.theta, wl.host(d_out)[seqs])
    for name in ("d_gates", "d_w_q", "d_w_qnorm", "d_w_k", "d_w_knorm"):
        close(wl.host(b2[name]), bo[name], 1e-3, name)
    # the full batch's gate gradients of those sequences are the same numbers
    close(wl.host(bf["d_gates"])[seqs], bo["d_gates"], 1e-3, "d_gates (full batch)")


def test_prefill_long_sequence_uses_the_per_position_selection():
    """A sequence longer than the batched selection holds (33,000 tokens: 516
    blocks) selects with the per-position gate kernel; sampled positions
    against the oracle, gated mode."""
    T = 33000
    w = wl.make_prefill(T, 8, 2, 2048, "paged", 7, DEV, random_norms=True)
    gk = prefill_gate_keys(w)
    pos = np.array([0, 4095, 32831, 32832, 32900, T - 1])
    sub = dataclasses.replace(w, batch=len(pos), q=w.q[torch.as_tensor(pos, device=DEV)],
                              seq_lens=torch.as_tensor(pos + 1, dtype=torch.int32, device=DEV),
                              block_table=w.block_table[:len(pos)])
    h = Host(sub)
    nb = T // 64
    gk_o = np.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), np.uint16)
    oracle.pool_blocks(h.k, h.bt[:1], w.strides, w.n_kv_heads, np.zeros(nb, np.int32), np.arange(nb, dtype=np.int32),
                       h.w_k, h.wkn, w.theta, gk_o)
    g = gpu_prefill(w, gk, True, w.budget, positions=pos)
    sel, gates, cnt, scores, out = oracle.prefill(wl.host(w.q), h.k, h.v, h.bt[0], w.strides, w.n_kv_heads, gk_o,
                                                  h.w_q, h.wqn, w.theta, w.budget, True, SM_SCALE, positions=pos)
    o = dict(gate_keys=gk_o, sel=sel, gates=gates, cnt=cnt, scores=scores, out=out)
    ties = compare_step(h, g, o, True, w.budget)
    say(f"prefill T={T}: boundary ties {ties}")


def test_prefill_gate_backward_full_size():
    """sas_prefill_gate_backward on the training-time workload of the
    benchmark (one 32,768-token sequence, Qwen3-8B heads, budget 2,048), in
    the launch configuration the benchmark times.  The gradient is linear in
    d_out, so with d_out zero except at sampled positions the GPU's whole
    backward must equal the oracle's backward summed over those positions
    alone (on the GPU's validated selection); d_gates vanish elsewhere.  The
    full-d_out run is then checked by linearity: it equals the sum of the
    sampled run and the run on the complementary positions."""
    from test_gpu_backward import close, gpu_prefill_backward, prefill_oracle_gates
    w = wl.named("prefill_8b", device=DEV)
    T = w.batch
    gk = prefill_gate_keys(w)
    pos = np.array([0, 63, 64, 130, 4095, 4096, 16000, 27000, 32767])
    gen = torch.Generator(device=DEV).manual_seed(81)
    d_full = torch.randn((T, w.n_q_heads, 128), generator=gen, device=DEV).to(torch.bfloat16)
    mask = torch.zeros(T, dtype=torch.bool, device=DEV)
    mask[torch.as_tensor(pos, device=DEV)] = True
    d_s = torch.where(mask[:, None, None], d_full, torch.zeros_like(d_full))
    d_c = torch.where(mask[:, None, None], torch.zeros_like(d_full), d_full)
    pf, b_s = gpu_prefill_backward(w, gk, w.budget, d_s)
    b_s = {k: v.clone() for k, v in b_s.items()}
    _, b_c = gpu_prefill_backward(w, gk, w.budget, d_c, pf=pf)
    b_c = {k: v.clone() for k, v in b_c.items()}
    _, b_f = gpu_prefill_backward(w, gk, w.budget, d_full, pf=pf)
    torch.cuda.synchronize()
    for name in ("d_w_q", "d_w_qnorm", "d_w_k", "d_w_knorm"):
        close(wl.host(b_f[name]), wl.host(b_s[name]).astype(np.float64) + wl.host(b_c[name]), 1e-5,
              name + " (sampled + complement)")
    np.testing.assert_array_equal(wl.host(b_f["d_gates"])[pos], wl.host(b_s["d_gates"])[pos])
    others = np.setdiff1d(np.arange(T), pos)
    assert not np.any(wl.host(b_s["d_gates"])[others])
    # the oracle at the sampled positions
    sub = dataclasses.replace(w, batch=len(pos), q=w.q[torch.as_tensor(pos, device=DEV)],
                              seq_lens=torch.as_tensor(pos + 1, dtype=torch.int32, device=DEV),
                              block_table=w.block_table[:len(pos)])
    h = Host(sub)
    nb = T // 64
    gk_o = np.zeros((w.n_pages, w.n_kv_heads, wl.GATE_DIM), np.uint16)
    oracle.pool_blocks(h.k, h.bt[:1], w.strides, w.n_kv_heads, np.zeros(nb, np.int32), np.arange(nb, dtype=np.int32),
                       h.w_k, h.wkn, w.theta, gk_o)
    q_all = wl.host(w.q)
    sel_o, gates_o, cnt_o, scores_o, _ = oracle.prefill(q_all, h.k, h.v, h.bt[0], w.strides, w.n_kv_heads, gk_o,
                                                        h.w_q, h.wqn, w.theta, w.budget, True, SM_SCALE,
                                                        positions=pos)
    sel_g, cnt_g, gates_g = wl.host(pf.sel), wl.host(pf.cnt), wl.host(pf.gates)
    o = dict(sel=sel_o, gates=gates_o, cnt=cnt_o, scores=scores_o)
    ties = compare_selection(dict(sel=sel_g[pos], gates=gates_g[pos], cnt=cnt_g[pos]), o, pos + 1, w.budget)
    say(f"prefill_8b backward: positions {pos.tolist()}, boundary ties {ties}")
    gates_for = gates_g.copy()
    gates_for[pos] = prefill_oracle_gates(o, sel_g[pos], cnt_g[pos])
    bo = oracle.prefill_gate_backward(q_all, h.k, h.v, h.bt[0], w.strides, w.n_kv_heads, sel_g, gates_for, cnt_g,
                                      SM_SCALE, h.w_q, h.wqn, h.w_k, h.wkn, gk_o, w.theta, wl.host(d_s),
                                      positions=pos)
    close(wl.host(b_s["d_gates"])[pos], bo["d_gates"], 1e-3, "d_gates")
    for name in ("d_w_q", "d_w_qnorm", "d_w_k", "d_w_knorm"):
        close(wl.host(b_s[name]), bo[name], 1e-3, name)
