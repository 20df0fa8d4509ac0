"""sas_decode_step_noalloc (the entry point for callers that cannot allocate)
against sas_decode_step with a caller workspace, through the C ABI: the same
outputs bit for bit, on two calls in a row, the second with a smaller input
(so the second call runs on the first one's leftover scratch contents), on
the paths that use scratch (two launches, sliced) and on the fused path."""
from __future__ import annotations

import sys

import pytest
import torch

from gpu_harness import gpu_pool
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


def _outputs(w, budget, gated, path, noalloc, gk):
    shape = ops.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.max_blocks, w.strides)
    n_sel = budget // 64
    sel = torch.full((w.batch, w.n_kv_heads, n_sel), -7, dtype=torch.int32, device=DEV)
    gates = torch.full((w.batch, w.n_kv_heads, n_sel), 3.0, dtype=torch.float32, device=DEV)
    cnt = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device=DEV)
    scores = torch.full((w.batch, w.n_kv_heads, w.max_blocks), 5.0, dtype=torch.float32, device=DEV)
    out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    args = (shape, w.q, w.w_q, w.w_qnorm, gk, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.theta, budget, sel,
            gates, cnt, scores, out)
    if noalloc:
        ops.decode_step_noalloc(*args, 1.0 / 128 ** 0.5, gated, path=path)
    else:
        nws = ops.decode_step_workspace_bytes(shape, budget, path)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV) if nws else None
        ops.decode_step(*args, ws, 1.0 / 128 ** 0.5, gated, path=path)
    torch.cuda.synchronize()
    return [t.clone() for t in (sel, gates, cnt, scores, out)]


@pytest.mark.parametrize("path", ["two_launches", "sliced", "fused", "auto"])
def test_noalloc_step_equals_workspace_step(path):
    big = wl.make(6, 40, 8, [131072, 100000, 77777, 5000, 321, 64000], 2048, "paged", 97, DEV, max_blocks=2048)
    small = wl.make(2, 8, 2, [20000, 700], 1024, "paged", 98, DEV, max_blocks=320)
    shape = ops.make_shape(big.batch, big.n_q_heads, big.n_kv_heads, big.max_blocks, big.strides)
    need = ops.decode_step_workspace_bytes(shape, 2048, path)
    assert need <= ops.NOALLOC_SCRATCH_BYTES
    for w, budget in ((big, 2048), (small, 1024)):  # the second call smaller than the first
        gk = gpu_pool(w)
        for gated in (True, False):
            say(f"noalloc {path} B={w.batch} budget {budget} gated={gated}")
            a = _outputs(w, budget, gated, path, True, gk)
            b = _outputs(w, budget, gated, path, False, gk)
            for name, x, y in zip(("sel", "gates", "cnt", "scores", "out"), a, b):
                assert torch.equal(x, y), (path, w.batch, name)


def test_noalloc_rejects_steps_beyond_its_scratch():
    # two launches over a batch whose per-candidate scores alone exceed the
    # scratch array: rejected before anything runs, outputs untouched
    # (the call is refused on the host, so the pools and keys are small stand-ins)
    B, Hq, Hkv, mb = 64, 8, 8, 16384
    shape = ops.make_shape(B, Hq, Hkv, mb, (Hkv * 64 * 128, 128, 64 * 128))
    assert ops.decode_step_workspace_bytes(shape, 1024, "two_launches") > ops.NOALLOC_SCRATCH_BYTES
    bf = dict(dtype=torch.bfloat16, device=DEV)
    q, w_q = torch.zeros((B, Hq, 128), **bf), torch.zeros((Hq, 128, 128), **bf)
    pool, gk = torch.zeros((4, Hkv, 64, 128), **bf), torch.zeros((4, Hkv, 128), **bf)
    wqn = torch.ones(128, dtype=torch.float32, device=DEV)
    bt = torch.zeros((B, mb), dtype=torch.int32, device=DEV)
    lens = torch.full((B,), 100, dtype=torch.int32, device=DEV)
    sel = torch.full((B, Hkv, 16), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device=DEV)
    out = torch.zeros((B, Hq, 128), **bf)
    with pytest.raises(ops.SasError) as ei:
        ops.decode_step_noalloc(shape, q, w_q, wqn, gk, pool, pool, bt, lens, 1e6, 1024, sel, None, cnt, None, out,
                                1.0 / 128 ** 0.5, False, path="two_launches")
    assert ei.value.status == ops.SAS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(sel == -7) and torch.all(cnt == 0)
