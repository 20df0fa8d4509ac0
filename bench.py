#!/usr/bin/env python3
"""SAS sparse-decode benchmark on one MI355X.

One step = one decode query per sequence through one attention layer:
sas_decode_step, i.e. the gate query, block scores and per-KV-head Top-K of
sas_gate_topk followed by the block-sparse flash-decode of sas_sparse_decode
(one fused launch when the (sequence, KV head) pairs fill the GPU).  The
step writes the selection, gates, counts and output, not the optional
per-candidate scores.  Gate keys are pooled once by sas_pool_blocks before
timing.  Inputs are synthetic and
already resident in HBM.  Consecutive steps rotate over --layers independent
layers (own K/V pools, gate keys, gate weights, queries), as consecutive
attention calls of a model do, so no step re-reads data a previous step left
in the 256 MB last-level cache.

Steps are launched eagerly (the host stays ahead of the GPU; --graph replays
a per-layer HIP graph instead).  Prints one JSON line: queries/s (sequences x
steps / wall time of the timed steps), the roofline entry of the dominant
kernel (the fused step kernel, or sas_sparse_decode on the two-launch path,
launched back to back --steps times on its stream and bracketed by HIP
events), the attention alone, a gather ceiling measured by sas_probe_read over
the same selected K/V blocks (read_ceiling), bulk pooling, and the oracle
timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix throughput, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_step(cnt, block_bytes):
    return int(cnt.sum()) * 2 * block_bytes


def gk_bytes_per_step(lens, n_kv_heads):
    return int(sum((int(L) - 1) // 64 for L in lens)) * n_kv_heads * 128 * 2


def step_extra_bytes(w, n_sel, gated, scores=False):
    """Bytes the fused step moves besides K/V and gate keys, each once: the
    queries, Qproj rows, norm weights and block-table rows it reads; the
    output, selection, gates, counts (and, when requested, the optional
    per-candidate scores) it writes."""
    B, Hq, Hkv = w.batch, w.n_q_heads, w.n_kv_heads
    reads = B * Hq * 128 * 2 + Hq * 128 * 128 * 2 + 128 * 4 + B * w.max_blocks * 4
    writes = B * Hq * 128 * 2 + B * Hkv * n_sel * 4 * (2 if gated else 1) + B * Hkv * 4
    if scores:
        writes += B * Hkv * w.max_blocks * 4
    return reads + writes


def recorded_traffic(workload, budget, kernel):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs recorded in profiles/ (scaled by a plain copy's reading),
    or None when the workload or kernel differs or its sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "step_traffic.json")
    if workload != "qwen3_8b" or budget != 2048 or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec["kernel"] != kernel:
        return None
    h = hashlib.sha256()
    for f in rec["kernel_sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["kernel_sources_sha256"] else None


def cpu_baseline(layer, budget, gated, seconds):
    """The oracle (as it stands) on a bounded sample of the same workload:
    whole sequences of the first layer, gate stage + dense masked attention,
    repeated until `seconds` of host time have passed."""
    import numpy as np
    import oracle
    from learned_block_sparse_tok_amd import workloads as wl
    w = layer["w"]
    n_s = min(w.batch, 4)
    bt = wl.host(w.block_table)[:n_s]
    nblk = bt.shape[1]
    pages = bt.reshape(-1)
    import torch
    idx = torch.as_tensor(pages, device=w.k_pool.device, dtype=torch.int64)
    # both layouts are arrays of 64-token pages (page p of a contiguous cache is
    # sequence p // max_blocks, block p % max_blocks), so gather whole pages
    k = wl.host(w.k_pool.view(w.n_pages, -1).index_select(0, idx))
    v = wl.host(w.v_pool.view(w.n_pages, -1).index_select(0, idx))
    bt_sub = np.arange(n_s * nblk, dtype=np.int32).reshape(n_s, nblk)
    q = wl.host(w.q)[:n_s].copy()
    lens = wl.host(w.seq_lens)[:n_s].astype(np.int32)
    gk = np.zeros((n_s * nblk, w.n_kv_heads, 128), np.uint16)
    seq = np.repeat(np.arange(n_s, dtype=np.int32), [int(L) // 64 for L in lens])
    blk = np.concatenate([np.arange(int(L) // 64, dtype=np.int32) for L in lens])
    wk, wq = wl.host(w.w_k), wl.host(w.w_q)
    wkn, wqn = wl.host(w.w_knorm), wl.host(w.w_qnorm)
    oracle.pool_blocks(k, bt_sub, w.strides, w.n_kv_heads, seq, blk, wk, wkn, w.theta, gk)  # precomputed, untimed
    queries, t_total, reps = 0, 0.0, 0
    while t_total < seconds or reps == 0:
        t0 = time.perf_counter()
        sel, gates, cnt, _ = oracle.gate_topk(q, wq, wqn, gk, bt_sub, lens, w.theta, budget, w.n_kv_heads)
        oracle.attend(q, k, v, bt_sub, w.strides, w.n_kv_heads, lens, sel, gates if gated else None, cnt,
                      1.0 / math.sqrt(128))
        t_total += time.perf_counter() - t0
        queries += n_s
        reps += 1
    return dict(value=queries / t_total, unit="queries/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n_s} of {w.batch} sequences of the same workload ({'gated' if gated else 'plain'} mode), "
                       f"gate stage + dense masked attention over all {int(lens[0])} tokens, {reps} repetitions, "
                       f"{t_total:.1f} s; gate keys pooled beforehand (untimed, as on the GPU)")


def selection_check(layer, dec, budget):
    """Oracle leg: every (sequence, KV head)'s selection of the first layer's
    timed steps against the oracle's gate stage (its own pooling of every
    complete block from a host copy of K, gate scores, full sort).  Counts
    the units whose selection is identical, the boundary ties (sets that
    differ only inside the band of candidates within 1e-3 relative of the
    oracle's K-th score, the same number taken from it on both sides), and
    any other mismatch; for planted workloads also the recall of the planted
    blocks.  The timing of the oracle is cpu_baseline's; this only compares."""
    import numpy as np
    import oracle
    from learned_block_sparse_tok_amd import workloads as wl
    t0 = time.perf_counter()
    w = layer["w"]
    lens = wl.host(w.seq_lens).astype(np.int32)
    bt = wl.host(w.block_table)
    gk = np.zeros((w.n_pages, w.n_kv_heads, 128), np.uint16)
    seq = np.repeat(np.arange(w.batch, dtype=np.int32), [int(L) // 64 for L in lens])
    blk = np.concatenate([np.arange(int(L) // 64, dtype=np.int32) for L in lens])
    oracle.pool_blocks(wl.host(w.k_pool), bt, w.strides, w.n_kv_heads, seq, blk, wl.host(w.w_k),
                       wl.host(w.w_knorm), w.theta, gk)
    sel, _, cnt, scores = oracle.gate_topk(wl.host(w.q), wl.host(w.w_q), wl.host(w.w_qnorm), gk, bt, lens, w.theta,
                                           budget, w.n_kv_heads)
    gsel, gcnt = wl.host(dec.sel), wl.host(dec.cnt)
    identical = ties = other = 0
    for s in range(w.batch):
        n = (int(lens[s]) - 1) // 64
        k = min(budget // 64 - 1, n)
        for h in range(w.n_kv_heads):
            if np.array_equal(gsel[s, h], sel[s, h]) and gcnt[s, h] == cnt[s, h]:
                identical += 1
                continue
            if gcnt[s, h] != cnt[s, h] or gsel[s, h, k] != n or not 0 < k < n:
                other += 1
                continue
            sc = scores[s, h, :n].astype(np.float64)
            order = np.lexsort((np.arange(n), -np.where(np.isnan(sc), -np.inf, sc)))
            sk = sc[order[k - 1]]
            band = set(np.nonzero(np.abs(sc - sk) <= 1e-3 * max(abs(sk), 1.0))[0].tolist())
            gset, oset = set(gsel[s, h, :k].tolist()), set(sel[s, h, :k].tolist())
            if gset - band == oset - band and len(gset & band) == len(oset & band):
                ties += 1
            else:
                other += 1
    out = {"units": w.batch * w.n_kv_heads, "identical": identical, "boundary_ties": ties, "mismatches": other,
           "band_rel": 1e-3, "layer": 0, "seconds": round(time.perf_counter() - t0, 1)}
    if w.planted is not None and layer.get("planted"):
        hit = sum(len(set(gsel[s, h, :gcnt[s, h]].tolist()) & set(w.planted[s, h].tolist()))
                  for s in range(w.batch) for h in range(w.n_kv_heads))
        out["planted_recall"] = {"hit": int(hit), "planted": int(w.planted.size),
                                 "recall": round(hit / w.planted.size, 4), "delta": w.plant_delta}
    log(f"selection check: {identical} identical, {ties} boundary ties, {other} mismatches of {out['units']} units"
        + (f"; planted recall {out['planted_recall']['recall']}" if "planted_recall" in out else ""))
    return out


def prefill_flops(cnt, group):
    """Algorithmic attention flops of a training-time forward: every query
    head of position t does 4 x 128 flops (QK and PV) per attended key, the
    keys being the full historical blocks plus its own block up to t."""
    import numpy as np
    T = cnt.shape[0]
    own = (np.arange(T) % 64 + 1)[:, None]
    keys = (cnt.astype(np.int64) - 1) * 64 + own
    return float(keys.sum()) * group * 4 * 128


def prefill_executed_flops(sel, cnt, group):
    """Matrix work the kernel issues: a wave's 16 MFMA columns are 16/h
    queries x h heads (h = 4 for groups of 3 or more heads, else the group
    size), and per block in the union of those queries' selections the wave
    issues 32 MFMAs of 16x16x32 (QK + PV), once per group of h heads."""
    import numpy as np
    T, Hkv, _ = sel.shape
    hw = 4 if group >= 3 else group
    qw = 16 // hw
    visits = 0
    for t0 in range(0, T, qw):
        for k in range(Hkv):
            rows = [sel[t, k, :cnt[t, k]] for t in range(t0, min(T, t0 + qw))]
            visits += len(np.unique(np.concatenate(rows)))
    return float(visits) * ((group + hw - 1) // hw) * 32 * 16 * 16 * 32 * 2


def cpu_baseline_prefill(w, gk_o_fn, budget, gated, seconds):
    """The oracle's forward at a bounded sample of positions (the last ones,
    which attend the most), repeated until `seconds` of host time passed."""
    import numpy as np
    import oracle
    from learned_block_sparse_tok_amd import workloads as wl
    T = w.batch
    h_q, h_k, h_v = wl.host(w.q), wl.host(w.k_pool), wl.host(w.v_pool)
    bt = wl.host(w.block_table[0])
    gk = gk_o_fn(h_k, bt)
    pos = np.arange(T - 32, T)
    n, t_total, reps = 0, 0.0, 0
    while t_total < seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.prefill(h_q, h_k, h_v, bt, w.strides, w.n_kv_heads, gk, wl.host(w.w_q), wl.host(w.w_qnorm), w.theta,
                       budget, gated, 1.0 / math.sqrt(128), positions=pos)
        t_total += time.perf_counter() - t0
        n += len(pos)
        reps += 1
    return dict(value=n / t_total, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"positions {T - 32}..{T - 1} of the {T}-token sequence ({'gated' if gated else 'plain'} "
                       f"mode): gate stage + dense masked attention over each position's past, {reps} repetitions, "
                       f"{t_total:.1f} s; gate keys pooled beforehand (untimed, as on the GPU)")


def read_ceiling(layers, decs, steps):
    """The gather ceiling of the attention's own reads: sas_probe_read over
    exactly the K and V blocks the last steps selected (one 16 KiB chunk per
    selected (page, KV head) block of K and of V), rotated over the layers
    like the steps and bracketed by HIP events; the best of 1, 2, 4 and 8
    chunks per workgroup.  Paged head-major pools only (a block of a
    contiguous cache is not one 16 KiB chunk): None otherwise."""
    import numpy as np
    import torch
    from learned_block_sparse_tok_amd import ops
    w0 = layers[0]["w"]
    ps, ts, hs = w0.strides
    if ts != 128:
        return None
    addrs = []
    for L, d in zip(layers, decs):
        w = L["w"]
        sel = d.sel.long()
        n_sel = sel.shape[2]
        valid = torch.arange(n_sel, device=sel.device)[None, None, :] < d.cnt.long()[:, :, None]
        bt = w.block_table.long()
        pages = torch.gather(bt, 1, sel.clamp(min=0).reshape(w.batch, -1)).reshape(sel.shape)
        kvh = torch.arange(w.n_kv_heads, device=sel.device)[None, :, None].expand_as(sel)
        off = (pages * ps + kvh * hs)[valid] * 2
        addrs.append(torch.cat([off + w.k_pool.data_ptr(), off + w.v_pool.data_ptr()]).contiguous())
    chunk_bytes = 64 * 128 * 2
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sinks = [ops.probe_read(a, 4) for a in addrs]
    best = None
    for per, reps in [(1, 40), (2, 40), (4, 40), (8, 40), (None, steps)]:
        if per is None:
            per = best[1]
        sinks = [ops.probe_read(a, per) for a in addrs]
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(reps):
            ops.probe_read(addrs[i % len(addrs)], per, sinks[i % len(addrs)])
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) / reps * 1e3
        if reps != steps and (best is None or us < best[0]):
            best = (us, per)
    nbytes = float(np.mean([a.numel() for a in addrs])) * chunk_bytes
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"read ceiling (sas_probe_read over the selected K/V blocks, {best[1]} chunks per workgroup): "
        f"{us:.1f} us = {gbs:.0f} GB/s")
    return {"kernel": "sas_probe_read (read_probe_kernel)",
            "pattern": "the selected K and V blocks of the timed steps, one 16 KiB chunk each, gathered",
            "chunks_per_wg": best[1], "bytes_per_launch": nbytes, "avg_launch_us": round(us, 2),
            "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def run_prefill(args):
    import numpy as np
    import torch
    from learned_block_sparse_tok_amd import ops
    from learned_block_sparse_tok_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.lib()
    w = wl.named(args.workload, device=dev, budget=args.budget)
    T, G = w.batch, w.group
    bt_row = w.block_table[0]
    nb = T // 64
    gk = torch.zeros((w.n_pages, w.n_kv_heads, 128), dtype=torch.bfloat16, device=dev)
    shape1 = ops.make_shape(1, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
    ops.pool_blocks(shape1, w.k_pool, w.block_table[:1].contiguous(), torch.zeros(nb, dtype=torch.int32, device=dev),
                    torch.arange(nb, dtype=torch.int32, device=dev), w.w_k, w.w_knorm, w.theta, gk)
    torch.cuda.synchronize()
    log(f"{args.workload}: T={T}, gate keys pooled")
    steps = max(1, min(args.steps, 20))
    warm = max(1, min(args.warmup, 3))
    results = {}
    for mode in args.modes.split(","):
        gated = mode == "gated"
        pf = ops.Prefill(w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, T, args.budget, w.theta, gated, device=dev)
        for _ in range(warm):
            pf.forward(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, bt_row)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            pf.forward(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, bt_row)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for _ in range(steps):
            pf.select(w.q, w.w_q, w.w_qnorm, gk, bt_row)
        ev[1].record(stream)
        for _ in range(steps):
            pf.attend(w.q, w.k_pool, w.v_pool, bt_row)
        ev[2].record(stream)
        torch.cuda.synchronize()
        sel_ms, att_ms = ev[0].elapsed_time(ev[1]) / steps, ev[1].elapsed_time(ev[2]) / steps
        cnt, sel = wl.host(pf.cnt), wl.host(pf.sel)
        flops = prefill_flops(cnt, G)
        executed = prefill_executed_flops(sel, cnt, G)
        ms = elapsed * 1e3 / steps
        results[mode] = dict(tokens_per_s=T * steps / elapsed, ms_per_step=ms, select_ms=sel_ms, attend_ms=att_ms,
                             attend_tflops=flops / (att_ms * 1e-3) / 1e12, algorithmic_flops=flops,
                             executed_flops=executed, executed_tflops=executed / (att_ms * 1e-3) / 1e12)
        log(f"{mode}: {T * steps / elapsed:.0f} tokens/s, {ms:.2f} ms/step (select {sel_ms:.2f} ms, attend "
            f"{att_ms:.2f} ms = {results[mode]['attend_tflops']:.1f} TFLOP/s algorithmic, "
            f"{results[mode]['executed_tflops']:.1f} TFLOP/s issued)")
    worst = min(results, key=lambda m: results[m]["tokens_per_s"])
    r = results[worst]
    line = {
        "metric": "training-time forward tokens/s (one layer, every position selects its own blocks)",
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "seq_len": T, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": 128, "budget_tokens": args.budget, "kv_layout": w.layout,
                   "mode": f"{worst} (slower of {','.join(results)})", "launch": "eager"},
        "roofline": {"bound": "mfma", "kernel": "sas_prefill_attend (prefill_attend_kernel)",
                     "achieved": round(r["attend_tflops"], 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(r["attend_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": r["algorithmic_flops"], "avg_launch_us": round(r["attend_ms"] * 1e3, 1),
                     "issued_flops_per_launch": r["executed_flops"],
                     "issued_frac": round(r["executed_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)},
        "modes": {m: {k: round(v, 4) for k, v in d.items()} for m, d in results.items()},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle

        def pooled(h_k, bt):
            gk_o = np.zeros((w.n_pages, w.n_kv_heads, 128), np.uint16)
            oracle.pool_blocks(h_k, bt[None, :].copy(), w.strides, w.n_kv_heads, np.zeros(nb, np.int32),
                               np.arange(nb, dtype=np.int32), wl.host(w.w_k), wl.host(w.w_knorm), w.theta, gk_o)
            return gk_o

        line["cpu_baseline"] = cpu_baseline_prefill(w, pooled, args.budget, worst == "gated", args.cpu_seconds)
        log(f"cpu baseline: {line['cpu_baseline']['value']:.1f} tokens/s on {line['cpu_baseline']['cores']} threads")
    print(json.dumps(line), flush=True)
    if args.backward:
        bline = time_prefill_backward(args, w, gk, bt_row, steps, warm)
        if not args.no_cpu_baseline:
            bline["cpu_baseline"] = cpu_baseline_prefill_backward(w, pooled, args.budget, args.cpu_seconds)
            log(f"cpu baseline (backward): {bline['cpu_baseline']['value']:.1f} tokens/s on "
                f"{bline['cpu_baseline']['cores']} threads")
        print(json.dumps(bline), flush=True)


def cpu_baseline_prefill_backward(w, gk_o_fn, budget, seconds):
    """The oracle's gate backward of the training-time forward at a bounded
    sample of positions (the last ones), on its own selection of them,
    repeated until `seconds` of host time passed."""
    import numpy as np
    import oracle
    from learned_block_sparse_tok_amd import workloads as wl
    T = w.batch
    h_q, h_k, h_v = wl.host(w.q), wl.host(w.k_pool), wl.host(w.v_pool)
    bt = wl.host(w.block_table[0])
    gk = gk_o_fn(h_k, bt)
    pos = np.arange(T - 32, T)
    w_q, w_qn, w_k, w_kn = wl.host(w.w_q), wl.host(w.w_qnorm), wl.host(w.w_k), wl.host(w.w_knorm)
    bt_all = np.ascontiguousarray(np.broadcast_to(bt, (len(pos), len(bt))))
    sel_p, gates_p, cnt_p, _ = oracle.gate_topk(np.ascontiguousarray(h_q[pos]), w_q, w_qn, gk, bt_all,
                                                (pos + 1).astype(np.int32), w.theta, budget, w.n_kv_heads)
    n_sel = budget // 64
    sel = np.full((T, w.n_kv_heads, n_sel), -1, np.int32)
    gates = np.zeros((T, w.n_kv_heads, n_sel), np.float32)
    cnt = np.zeros((T, w.n_kv_heads), np.int32)
    sel[pos], gates[pos], cnt[pos] = sel_p, gates_p, cnt_p
    import torch
    d_out = wl.bf16_bits(torch.randn(h_q.shape, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16))
    n, t_total, reps = 0, 0.0, 0
    while t_total < seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.prefill_gate_backward(h_q, h_k, h_v, bt, w.strides, w.n_kv_heads, sel, gates, cnt,
                                     1.0 / math.sqrt(128), w_q, w_qn, w_k, w_kn, gk, w.theta, d_out, positions=pos)
        t_total += time.perf_counter() - t0
        n += len(pos)
        reps += 1
    return dict(value=n / t_total, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"positions {T - 32}..{T - 1} of the {T}-token sequence: the gate backward (gradients of "
                       f"every gate parameter and of the gates) on the oracle's own selection of those positions, "
                       f"{reps} repetitions, {t_total:.1f} s; selection and gate keys computed beforehand (untimed)")


def time_prefill_backward(args, w, gk, bt_row, steps, warm):
    """sas_prefill_gate_backward after the gated training-time forward (with
    its log-sum-exp), launched back to back and bracketed by HIP events on the
    launch stream."""
    import torch
    from learned_block_sparse_tok_amd import ops
    from learned_block_sparse_tok_amd import workloads as wl
    dev = w.q.device
    T, G, n_sel = w.batch, w.group, args.budget // 64
    pf = ops.Prefill(w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, T, args.budget, w.theta, True, device=dev)
    pf.forward(w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, bt_row)
    gen = torch.Generator(device=dev).manual_seed(901)
    d_out = torch.randn((T, w.n_q_heads, 128), generator=gen, device=dev).to(torch.bfloat16)
    shape1 = ops.make_shape(1, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
    ws_bytes = ops.prefill_gate_backward_workspace_bytes(shape1, T, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def one(out=None):
        return ops.prefill_gate_backward(shape1, w.q, w.k_pool, w.v_pool, bt_row, T, pf.sel, pf.gates, pf.cnt, n_sel,
                                         pf.sm_scale, pf.lse, w.w_q, w.w_qnorm, w.w_k, w.w_knorm, gk, w.theta, d_out,
                                         workspace=ws, out=out)

    out = one()
    for _ in range(warm):
        one(out)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        one(out)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    # the walk's algorithmic work: per query head, position and attended key,
    # 2 x 128 flops for the score and 2 x 128 for <dO, v> (the forward's count)
    flops = prefill_flops(wl.host(pf.cnt), G)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"training-time backward: {ms:.2f} ms per sequence = {T / (ms * 1e-3):.0f} tokens/s, walk work "
        f"{tflops:.1f} TFLOP/s over the whole call, workspace {ws_bytes / 2**20:.0f} MiB")
    return {"metric": "training-time backward tokens/s (continuous-gate gradients of one layer)",
            "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "higher_is_better": True, "n_gpus": 1,
            "steps": steps, "warmup": warm, "ms_per_step": round(ms, 4), "dtype": "bf16 inputs, fp32 gradients",
            "data": "synthetic",
            "config": {"workload": args.workload, "seq_len": T, "n_q_heads": w.n_q_heads,
                       "n_kv_heads": w.n_kv_heads, "budget_tokens": args.budget, "kv_layout": w.layout,
                       "workspace_bytes": ws_bytes},
            "roofline": {"bound": "mfma", "kernel": "sas_prefill_gate_backward (whole call, 7 kernels; the "
                                                     "block walk prefill_grad_kernel dominates)",
                         "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "flops_per_launch": flops, "avg_launch_us": round(ms * 1e3, 1)}}


def time_backward(args, layers, w0):
    """sas_gate_backward after a gated step of each layer, launched back to
    back over the rotated layers and bracketed by HIP events."""
    import numpy as np
    import torch
    from learned_block_sparse_tok_amd import ops
    from learned_block_sparse_tok_amd import workloads as wl
    dev = w0.q.device
    n_sel = args.budget // 64
    shape = ops.make_shape(w0.batch, w0.n_q_heads, w0.n_kv_heads, w0.max_blocks, w0.strides)
    ws = torch.empty(ops.gate_backward_workspace_bytes(shape, n_sel), dtype=torch.uint8, device=dev)
    jobs = []
    for l, L in enumerate(layers):
        w = L["w"]
        dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, args.budget, w.theta,
                                True, device=dev)
        dec.step(w.q, w.w_q, w.w_qnorm, L["gk"], w.k_pool, w.v_pool, w.block_table, w.seq_lens)
        gen = torch.Generator(device=dev).manual_seed(900 + l)
        d_out = torch.randn((w.batch, w.n_q_heads, 128), generator=gen, device=dev).to(torch.bfloat16)
        out = ops.gate_backward(shape, w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, dec.sel, dec.gates,
                                dec.cnt, n_sel, dec.sm_scale, w.w_q, w.w_qnorm, w.w_k, w.w_knorm, L["gk"], w.theta,
                                d_out, workspace=ws)
        jobs.append((w, L["gk"], dec, d_out, out))
    torch.cuda.synchronize()

    def one(i):
        w, gk, dec, d_out, out = jobs[i % len(jobs)]
        ops.gate_backward(shape, w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, dec.sel, dec.gates, dec.cnt,
                          n_sel, dec.sm_scale, w.w_q, w.w_qnorm, w.w_k, w.w_knorm, gk, w.theta, d_out, workspace=ws,
                          out=out)

    for i in range(args.warmup):
        one(i)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        one(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    kv_b = float(np.mean([kv_bytes_per_step(wl.host(j[2].cnt), 64 * 128 * 2) for j in jobs]))
    log(f"gate backward: {ms * 1e3:.1f} us per step, {kv_b / (ms * 1e-3) / 1e9:.0f} GB/s of selected K+V")
    return {"metric": "continuous-gate backward us/step (gate, gate-query and gate-key parameter gradients)",
            "value": round(ms * 1e3, 2), "unit": "us", "higher_is_better": False, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "dtype": "bf16 inputs, fp32 gradients", "data": "synthetic",
            "config": {"workload": args.workload, "batch": w0.batch, "budget_tokens": args.budget,
                       "layers_rotated": len(layers)},
            "roofline": {"bound": "hbm", "kernel": "sas_gate_backward (3 kernels)",
                         "achieved": round(kv_b / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(kv_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                         "bytes_per_launch": kv_b}}


def run_serve(args):
    """Incremental serving on the ragged workload: per step every sequence
    appends one token (sas_append_kv, which pools each block the token
    completes), then sas_gate_topk + sas_sparse_decode.  The lengths grow by
    one per step; warm-up steps are the first steps of the same run."""
    import numpy as np
    import torch
    from learned_block_sparse_tok_amd import ops
    from learned_block_sparse_tok_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.lib()
    warm = max(1, min(args.warmup, 16))
    steps = max(1, min(args.steps, 120))
    total = warm + steps
    budget = args.budget if args.budget != 2048 else 4096  # the ragged workload's budget unless given
    w = wl.named(args.workload, device=dev, budget=budget, steps=total)
    shape = ops.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
    gk = torch.zeros((w.n_pages, w.n_kv_heads, 128), dtype=torch.bfloat16, device=dev)
    lens0 = wl.host(w.seq_lens).astype(np.int64)
    seq = np.repeat(np.arange(w.batch, dtype=np.int32), [int(L) // 64 for L in lens0])
    blk = np.concatenate([np.arange(int(L) // 64, dtype=np.int32) for L in lens0])
    ops.pool_blocks(shape, w.k_pool, w.block_table, torch.as_tensor(seq, device=dev), torch.as_tensor(blk, device=dev),
                    w.w_k, w.w_knorm, w.theta, gk)
    q_new, k_new, v_new = wl.append_rows(w, total, seed=55)
    # per-step lengths: the new token is at position L, then L + 1 tokens are cached
    lens_all = torch.as_tensor((lens0[None, :] + 1 + np.arange(total)[:, None]).astype(np.int32), device=dev)
    completed = int(((lens0[None, :] + 1 + np.arange(total)[:, None]) % 64 == 0).sum())
    torch.cuda.synchronize()
    log(f"{args.workload}: B={w.batch}, lengths {int(lens0.min())}..{int(lens0.max())}, budget {budget}, "
        f"{total} steps ({completed} blocks completed on the way)")
    results = {}
    for mode in args.modes.split(","):
        gated = mode == "gated"
        # each mode replays the same steps from the same starting state: the
        # appends of a step rewrite the same rows and the same gate keys
        dec = ops.SparseDecoder(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides, budget, w.theta, gated,
                                device=dev)
        # The append runs on a second stream (default priority), overlapping
        # the selection: step i's select reads only gate keys of blocks before
        # its local block (the block the new token completes is that local
        # block), and the appends write rows and gate keys no earlier step
        # reads.  Only step i's attend waits for step i's append.
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream(device=dev)
        done = [torch.cuda.Event() for _ in range(total)]

        def one(i):
            with torch.cuda.stream(side):
                ops.append_kv(shape, k_new[i], v_new[i], w.k_pool, w.v_pool, w.block_table, lens_all[i], w.w_k,
                              w.w_knorm, w.theta, gk)
                done[i].record(side)
            dec.select(q_new[i], w.w_q, w.w_qnorm, gk, w.block_table, lens_all[i])
            main.wait_event(done[i])
            dec.attend(q_new[i], w.k_pool, w.v_pool, w.block_table, lens_all[i])

        for i in range(warm):
            one(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(warm, total):
            one(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        # the appends alone, on the main stream (idempotent: the same rows and
        # gate keys again)
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(warm, total):
            ops.append_kv(shape, k_new[i], v_new[i], w.k_pool, w.v_pool, w.block_table, lens_all[i], w.w_k,
                          w.w_knorm, w.theta, gk)
        ev[1].record(stream)
        torch.cuda.synchronize()
        app_us = ev[0].elapsed_time(ev[1]) / steps * 1e3
        # the selection and the attention alone (the last step's inputs),
        # each launched back to back on the main stream, bracketed by HIP events
        last = total - 1
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for _ in range(steps):
            dec.select(q_new[last], w.w_q, w.w_qnorm, gk, w.block_table, lens_all[last])
        ev[1].record(stream)
        for _ in range(steps):
            dec.attend(q_new[last], w.k_pool, w.v_pool, w.block_table, lens_all[last])
        ev[2].record(stream)
        torch.cuda.synchronize()
        sel_us = ev[0].elapsed_time(ev[1]) / steps * 1e3
        att_us = ev[1].elapsed_time(ev[2]) / steps * 1e3
        cnt = wl.host(dec.cnt)
        kv_b = kv_bytes_per_step(cnt, 64 * 128 * 2)
        gk_b = gk_bytes_per_step(wl.host(lens_all[total - 1]), w.n_kv_heads)
        ms = elapsed * 1e3 / steps
        results[mode] = dict(queries_per_s=w.batch * steps / elapsed, ms_per_step=ms, append_us=app_us,
                             step_gbs=(kv_b + gk_b) / (ms * 1e-3) / 1e9, kv_bytes=kv_b, gk_bytes=gk_b,
                             select_us=sel_us, select_gbs=gk_b / (sel_us * 1e-6) / 1e9,
                             attend_us=att_us, attend_gbs=kv_b / (att_us * 1e-6) / 1e9)
        log(f"{mode}: {results[mode]['queries_per_s']:.0f} queries/s, {ms * 1e3:.1f} us/step (append {app_us:.1f} us), "
            f"step {results[mode]['step_gbs']:.0f} GB/s of gate keys + selected K/V")
    worst = min(results, key=lambda m: results[m]["queries_per_s"])
    r = results[worst]
    line = {
        "metric": "incremental serving queries/s (append + incremental pooling + select + attend per step)",
        "value": round(r["queries_per_s"], 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.batch, "context": f"{int(lens0.min())}..{int(lens0.max())}",
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": 128, "budget_tokens": budget,
                   "kv_layout": w.layout, "mode": f"{worst} (slower of {','.join(results)})", "launch": "eager"},
        "roofline": {"bound": "hbm", "kernel": "sas_sparse_decode (decode_kernel)",
                     "achieved": round(r["attend_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["attend_gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": r["kv_bytes"], "bytes_note": "selected K/V blocks of the last step",
                     "avg_launch_us": round(r["attend_us"], 2)},
        "selection": {"kernel": "sas_gate_topk (gate_topk_kernel)", "avg_launch_us": round(r["select_us"], 2),
                      "bytes_per_launch": r["gk_bytes"], "achieved_gbs": round(r["select_gbs"], 1),
                      "frac": round(r["select_gbs"] / HBM_PEAK_GBS, 4)},
        "step_hbm_frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4),
        "modes": {m: {k: (round(v, 3) if isinstance(v, float) else v) for k, v in d.items()}
                  for m, d in results.items()},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_8b")
    ap.add_argument("--budget", type=int, default=2048)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--modes", default="plain,gated")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB --steps times (a kernel of "
                         "known traffic, for calibrating the HBM byte counters), then exit")
    ap.add_argument("--backward", action="store_true",
                    help="also time the continuous-gate backward (sas_gate_backward after the gated step, or "
                         "sas_prefill_gate_backward after the training-time forward): a second JSON line")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "sliced", "two_launches"],
                    help="sas_decode_step path (auto: one fused launch when the pairs fill the GPU)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each layer's step from a HIP graph instead of launching it eagerly "
                         "(eager is faster here: the host stays ahead of the GPU)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py: the SAS decode path here runs on one GPU only; multi-GPU runs are not "
                  f"supported (asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr, flush=True)
        sys.exit(2)

    if args.workload.startswith("prefill"):
        return run_prefill(args)
    if args.workload == "ragged":
        return run_serve(args)
    import numpy as np
    import torch
    from learned_block_sparse_tok_amd import ops
    from learned_block_sparse_tok_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_probe_mib} MiB x {args.steps}")
        return
    ops.lib()
    t_setup = time.perf_counter()
    layers = []
    for l in range(args.layers):
        w = wl.named(args.workload, seed=100 + l, device=dev, budget=args.budget)
        planted = False
        if w.planted is not None and not args.no_cpu_baseline:
            # the planted relevance spikes: their direction is the test recipe's
            # (tests/planting.py, which reads the oracle's gate query), so they
            # ride with the oracle leg
            sys.path.insert(0, os.path.join(ROOT, "tests"))
            from planting import plant
            plant(w)
            planted = True
        shape = ops.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
        gk = torch.zeros((w.n_pages, w.n_kv_heads, 128), dtype=torch.bfloat16, device=dev)
        lens = wl.host(w.seq_lens)
        seq = np.repeat(np.arange(w.batch, dtype=np.int32), [int(L) // 64 for L in lens])
        blk = np.concatenate([np.arange(int(L) // 64, dtype=np.int32) for L in lens])
        ops.pool_blocks(shape, w.k_pool, w.block_table, torch.as_tensor(seq, device=dev),
                        torch.as_tensor(blk, device=dev), w.w_k, w.w_knorm, w.theta, gk)
        layers.append(dict(w=w, gk=gk, planted=planted))
        torch.cuda.synchronize()
        log(f"layer {l}: {args.workload} inputs drawn and gate keys pooled")
    w0 = layers[0]["w"]
    log(f"setup {time.perf_counter() - t_setup:.1f} s")

    # bulk pooling alone (sas_pool_blocks over every complete block of a layer;
    # off the step, once per layer): again for each layer, bracketed by HIP events
    stream = torch.cuda.current_stream()
    pool_args = []
    for L in layers:
        w = L["w"]
        lens = wl.host(w.seq_lens)
        seq = np.repeat(np.arange(w.batch, dtype=np.int32), [int(x) // 64 for x in lens])
        blk = np.concatenate([np.arange(int(x) // 64, dtype=np.int32) for x in lens])
        pool_args.append((ops.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides), w,
                          torch.as_tensor(seq, device=dev), torch.as_tensor(blk, device=dev), len(seq)))
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    pe0.record(stream)
    for (shp, w, sq, bk, _), L in zip(pool_args, layers):
        ops.pool_blocks(shp, w.k_pool, w.block_table, sq, bk, w.w_k, w.w_knorm, w.theta, L["gk"])
    pe1.record(stream)
    torch.cuda.synchronize()
    pool_ms = pe0.elapsed_time(pe1) / len(layers)
    pool_blocks_n = float(np.mean([a[4] for a in pool_args]))
    pool_bytes = pool_blocks_n * w0.n_kv_heads * (64 * 128 * 2 + 128 * 2)  # keys read + gate keys written
    log(f"bulk pooling: {pool_ms:.3f} ms per layer ({int(pool_blocks_n)} blocks x {w0.n_kv_heads} KV heads), "
        f"{pool_bytes / (pool_ms * 1e-3) / 1e9:.0f} GB/s")

    results, mode_steps = {}, {}
    for mode in args.modes.split(","):
        gated = mode == "gated"
        # one decoder (outputs + workspaces) per layer, as a model keeps per-layer state
        # the timed step writes what a serving caller uses (selection, gates,
        # counts, output), not the optional per-candidate score output
        decs = [ops.SparseDecoder(w0.batch, w0.n_q_heads, w0.n_kv_heads, w0.max_blocks, w0.strides, args.budget,
                                  w0.theta, gated, device=dev, path=args.path, keep_scores=False)
                for _ in layers]

        # each layer's sas_decode_step with its arguments checked and
        # marshalled once (a serving loop keeps its buffers): a timed step is
        # one C call
        calls = [decs[l].prepare_step(L["w"].q, L["w"].w_q, L["w"].w_qnorm, L["gk"], L["w"].k_pool, L["w"].v_pool,
                                      L["w"].block_table, L["w"].seq_lens) for l, L in enumerate(layers)]

        def step_eager(l):
            calls[l]()

        for i in range(max(args.warmup, len(layers))):
            step_eager(i % len(layers))
        torch.cuda.synchronize()
        graphs = []
        if args.graph:
            # one HIP graph per layer holding sas_gate_topk + sas_sparse_decode
            for l in range(len(layers)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step_eager(l)
                graphs.append(g)
            torch.cuda.synchronize()
            run_step = lambda i: graphs[i % len(layers)].replay()
        else:
            run_step = lambda i: step_eager(i % len(layers))
        for i in range(args.warmup):
            run_step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            run_step(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

        # per-step GPU time: an event after every step of another pass of
        # --steps steps (the gaps between consecutive events), for p10/p50/p90
        stream = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            run_step(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        step_us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)])
        p10, p50, p90 = (float(x) for x in np.percentile(step_us, [10, 50, 90]))

        # the attention alone: sas_sparse_decode (decode_kernel, the two-launch
        # path's dominant kernel) launched back to back on the current stream
        # (selections from the steps above), bracketed by HIP events
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(len(layers)):
            L = layers[i]
            decs[i].attend(L["w"].q, L["w"].k_pool, L["w"].v_pool, L["w"].block_table, L["w"].seq_lens)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            l = i % len(layers)
            w = layers[l]["w"]
            decs[l].attend(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens)
        ev1.record(stream)
        torch.cuda.synchronize()
        dec_ms = ev0.elapsed_time(ev1) / args.steps
        # the path sas_decode_step took, told apart by its workspace size
        ws_of = lambda pth: ops.decode_step_workspace_bytes(decs[0].shape, args.budget, pth)
        ws_now = ws_of(args.path)
        fused = ws_now == 0  # one fused launch, one workgroup per pair, no workspace
        split_fused = not fused and ws_now == ws_of("fused")
        path_name = ("one fused launch" if fused else
                     "fused launch split over workgroups + partial merge" if split_fused else
                     "sliced selection" if ws_now == ws_of("sliced") else "two launches")

        # algorithmic bytes: selected K+V blocks (attention), every candidate's
        # gate key (selection), and, for the fused launch, the rest it moves once
        cnts = [wl.host(d.cnt) for d in decs]
        kv_b = float(np.mean([kv_bytes_per_step(c, 64 * 128 * 2) for c in cnts]))
        gk_b = float(np.mean([gk_bytes_per_step(wl.host(L["w"].seq_lens), w0.n_kv_heads) for L in layers]))
        ex_b = float(step_extra_bytes(w0, args.budget // 64, gated))
        ms = elapsed * 1e3 / args.steps
        # the dominant kernel: the fused step itself (one launch per step), else
        # the attention
        dom_ms = dec_ms
        if fused or split_fused:  # the step's launches, back to back, bracketed by HIP events
            # (untimed steps queued first, so that the GPU is busy when the first
            # event is taken and the bracket holds only the timed launches)
            for i in range(len(layers)):
                run_step(i)
            ev0.record(stream)
            for i in range(args.steps):
                run_step(i)
            ev1.record(stream)
            torch.cuda.synchronize()
            dom_ms = ev0.elapsed_time(ev1) / args.steps
        # algorithmic bytes: the gate keys of every candidate and the selected
        # K/V blocks (the queries, weights, indices and outputs the fused
        # launch also moves are reported apart, not counted)
        dom_b = kv_b + gk_b if fused or split_fused else kv_b
        mode_steps[mode] = step_eager
        results[mode] = dict(queries_per_s=w0.batch * args.steps / elapsed, ms_per_step=ms,
                             decode_ms=dec_ms, decode_gbs=kv_b / (dec_ms * 1e-3) / 1e9,
                             dominant_ms=dom_ms, dominant_bytes=dom_b, dominant_gbs=dom_b / (dom_ms * 1e-3) / 1e9,
                             step_gbs=(kv_b + gk_b) / (ms * 1e-3) / 1e9, kv_bytes=kv_b, gk_bytes=gk_b,
                             other_bytes=ex_b,
                             attended_tokens_per_query=float(np.mean([c.sum() for c in cnts])) * 64 / (
                                 w0.batch * w0.n_kv_heads),
                             step_us_p10=p10, step_us_p50=p50, step_us_p90=p90, fused=float(fused),
                             split_fused=float(split_fused),
                             path=path_name)
        log(f"{mode}: {results[mode]['queries_per_s']:.0f} queries/s, {ms * 1e3:.1f} us/step "
            f"({path_name}), step {results[mode]['step_gbs']:.0f} GB/s; "
            f"per-step p10/p50/p90 {p10:.1f}/{p50:.1f}/{p90:.1f} us; "
            f"attention alone (decode_kernel) {dec_ms * 1e3:.1f} us = {results[mode]['decode_gbs']:.0f} GB/s")

    worst = min(results, key=lambda m: results[m]["queries_per_s"])
    r = results[worst]
    ceiling = read_ceiling(layers, decs, args.steps)
    graph_us = graph_all_us = None
    if not args.graph:
        # the slower mode's steps replayed from one HIP graph per layer, after
        # every eager measurement (a capture made between them slowed the
        # eager launches that followed it)
        step_eager = mode_steps[worst]
        graphs = []
        for l in range(len(layers)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_eager(l)
            graphs.append(g)
        for i in range(max(args.warmup, len(layers))):
            graphs[i % len(layers)].replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for i in range(args.steps):
            graphs[i % len(layers)].replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - tg) * 1e6 / args.steps
        del graphs
        log(f"{worst} from HIP graphs: {graph_us:.1f} us/step")
        # one graph holding a step of every layer (one decode iteration through
        # the layers), so that a replay's launch cost is shared by the layers
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for l in range(len(layers)):
                step_eager(l)
        reps = max(1, args.steps // len(layers))
        for _ in range(max(2, args.warmup // len(layers))):
            g_all.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(reps):
            g_all.replay()
        torch.cuda.synchronize()
        graph_all_us = (time.perf_counter() - tg) * 1e6 / (reps * len(layers))
        del g_all
        log(f"{worst} from one HIP graph of all {len(layers)} layers: {graph_all_us:.1f} us/step")
    line = {
        "metric": "sparse-decode queries/s + % HBM roofline, Qwen3-8B shape, 32K ctx, 2K budget",
        "value": round(r["queries_per_s"], 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": w0.batch, "context": int(wl.host(w0.seq_lens).max()),
                   "n_q_heads": w0.n_q_heads, "n_kv_heads": w0.n_kv_heads, "head_dim": 128,
                   "budget_tokens": args.budget, "kv_layout": w0.layout, "layers_rotated": len(layers),
                   "mode": f"{worst} (slower of {','.join(results)})",
                   "launch": "hip graph per layer" if args.graph else "eager",
                   "path": r["path"]},
        "roofline": {"bound": "hbm",
                     "kernel": ("sas_decode_step (step_kernel, one fused launch)" if r["fused"] else
                                "sas_decode_step (step_kernel split over workgroups + decode_merge_kernel)"
                                if r["split_fused"]
                                else "sas_sparse_decode (decode_kernel)"),
                     "achieved": round(r["dominant_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["dominant_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(args.workload, args.budget,
                                                 "step_kernel" if r["fused"] else "decode_kernel"),
                     "bytes_per_launch": r["dominant_bytes"], "avg_launch_us": round(r["dominant_ms"] * 1e3, 2),
                     "bytes_note": ("gate keys of every candidate + selected K/V blocks"
                                    if r["fused"] or r["split_fused"] else
                                    "selected K/V blocks"),
                     "other_bytes_per_launch": r["other_bytes"] if r["fused"] else None},
        "attention_alone": {"kernel": "sas_sparse_decode (decode_kernel)", "avg_launch_us": round(r["decode_ms"] * 1e3, 2),
                            "bytes_per_launch": r["kv_bytes"], "achieved_gbs": round(r["decode_gbs"], 1),
                            "frac": round(r["decode_gbs"] / HBM_PEAK_GBS, 4)},
        "read_ceiling": ceiling,
        "hip_graph": (None if graph_us is None else
                      {"us_per_step": round(graph_us, 2), "mode": worst,
                       "queries_per_s": round(w0.batch * 1e6 / graph_us, 1),
                       "all_layers_us_per_step": round(graph_all_us, 2),
                       "note": "the same steps replayed from one HIP graph per layer, and from one graph holding "
                               "a step of every layer (eager is the primary figure)"}),
        "step_hbm_frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4),
        "pooling": {"kernel": "sas_pool_blocks (pool_kernel), every complete block of a layer, off the step",
                    "ms_per_layer": round(pool_ms, 4), "bytes": pool_bytes,
                    "achieved_gbs": round(pool_bytes / (pool_ms * 1e-3) / 1e9, 1),
                    "frac": round(pool_bytes / (pool_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "tokens_per_s": round(r["queries_per_s"], 1),
        "attended_kv_tokens_per_s": round(r["queries_per_s"] * r["attended_tokens_per_query"], 1),
        "modes": {m: {k: (round(v, 3) if isinstance(v, float) else v) for k, v in d.items()}
                  for m, d in results.items()},
    }
    if ceiling is not None:
        line["roofline"]["frac_of_read_ceiling"] = round(r["dominant_gbs"] / ceiling["achieved_gbs"], 4)
        line["attention_alone"]["frac_of_read_ceiling"] = round(r["decode_gbs"] / ceiling["achieved_gbs"], 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layers[0], args.budget, worst == "gated", args.cpu_seconds)
        log(f"cpu baseline: {line['cpu_baseline']['value']:.1f} queries/s on {line['cpu_baseline']['cores']} threads")
        line["selection_check"] = selection_check(layers[0], decs[0], args.budget)
    print(json.dumps(line), flush=True)
    if args.backward:
        print(json.dumps(time_backward(args, layers, w0)), flush=True)


if __name__ == "__main__":
    main()
