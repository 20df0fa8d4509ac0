"""Seeded synthetic decode workloads (inputs only).

This module draws the arrays one SAS decode step consumes -- queries, paged
K/V pools, block tables, sequence lengths, gate weights -- and nothing else:
it holds none of the method's arithmetic, so the HIP path and the CPU oracle
can both be fed from it.

Shapes follow the workloads the SAS pages fix (64-token KV blocks, Qwen3
attention heads of width 128, 32,768-token training context, 1,024 / 2,048 /
4,096-token decode budgets) at the batch sizes of the benchmark configurations:

=========  =====  ======  ========  ==========  ======  =======================
name       batch  Hq/Hkv  context   layout      budget  extras
=========  =====  ======  ========  ==========  ======  =======================
tiny       1      4/1     4,096     contiguous  1,024   3 planted blocks, +2.0
qwen3_4b   8      32/8    32,768    contiguous  2,048
qwen3_8b   32     32/8    32,768    paged       2,048   (1,024 / 4,096 too)
qwen3_14b  4      40/8    131,072   paged       2,048   1% planted, +3.0
ragged     64     32/8    4K..64K   paged       4,096   128 append steps
prefill_8b 1      32/8    32,768    paged       2,048   every position a query
=========  =====  ======  ========  ==========  ======  =======================

Values: q, K, V ~ N(0, 1) drawn in fp32 and rounded to bf16 (RNE, by torch);
gate weights ~ N(0, 1/sqrt(fan_in)) drawn in fp32 and rounded to bf16; norm
weights ones (or 1 + 0.1 N(0,1) when ``random_norms``).  Projection weights
are stored output-major, as torch Linear weights are.  Paged pools are
head-major ``[P][Hkv][64][128]`` with a seeded random-permutation block table;
contiguous caches are ``[B][L][Hkv][128]`` with the identity block table.
Planted blocks are only *chosen* here (seeded); the direction that plants them
is part of the test recipe.

Every tensor is drawn from ``torch.Generator(device).manual_seed(seed + k)``
with a fixed stream index k per array, so a workload is identical for a given
(seed, device).  Large workloads are drawn on the GPU.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BLOCK = 64
HEAD_DIM = 128
GATE_DIM = 128
ROPE_THETA = 1.0e6  # Qwen3 rotary base

# fixed stream indices, one per drawn array
_S_Q, _S_K, _S_V, _S_WQ, _S_WK, _S_PERM, _S_PLANT, _S_LENS, _S_APPEND, _S_NORM, _S_SEL, _S_GK, _S_QALL = range(13)


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    max_blocks: int
    layout: str  # "paged" | "contiguous"
    budget: int
    theta: float
    seq_lens: torch.Tensor  # int32 [B]
    q: torch.Tensor  # bf16 [B][Hq][128]
    k_pool: torch.Tensor  # bf16, layout-dependent
    v_pool: torch.Tensor
    block_table: torch.Tensor  # int32 [B][max_blocks]
    w_q: torch.Tensor  # bf16 [Hq][128 out][128 in]  (torch Linear layout)
    w_k: torch.Tensor  # bf16 [Hkv][128 out][384 in]
    w_qnorm: torch.Tensor  # f32 [128]
    w_knorm: torch.Tensor  # f32 [128]
    strides: tuple  # (page, token, head) strides of the pools, in elements
    planted: np.ndarray | None = None  # int32 [B][Hkv][n_planted] block indices
    plant_delta: float = 0.0
    # training-time forward of one sequence: "sequence" t of the batch is
    # position t (length t+1, query q[t]); all positions share one cache and
    # one block-table row (block_table is that row expanded with stride 0)
    prefill: bool = False

    @property
    def n_pages(self) -> int:
        return self.k_pool.numel() // (self.n_kv_heads * BLOCK * HEAD_DIM)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    return g


def _normal_bf16(shape, device, seed, stream, std=1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, seed, stream), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; bf16 tensors become their uint16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().contiguous().cpu().numpy()


def make(batch: int, n_q_heads: int, n_kv_heads: int, seq_lens, budget: int, layout: str,
         seed: int, device="cpu", max_blocks: int | None = None, n_planted: int = 0,
         plant_delta: float = 0.0, random_norms: bool = False, theta: float = ROPE_THETA,
         name: str = "custom", extra_pages: int = 0) -> Workload:
    """Draw one workload.  seq_lens: int or sequence of B ints (each >= 1;
    a length counts the current token, whose K/V are already in the cache)."""
    if isinstance(seq_lens, (int, np.integer)):
        lens = np.full(batch, int(seq_lens), np.int64)
    else:
        lens = np.asarray(seq_lens, np.int64)
    assert lens.shape == (batch,) and lens.min() >= 1
    need_blocks = int(math.ceil(lens.max() / BLOCK))
    if max_blocks is None:
        max_blocks = need_blocks
    assert max_blocks >= need_blocks
    Hkv, Hq = n_kv_heads, n_q_heads
    q = _normal_bf16((batch, Hq, HEAD_DIM), device, seed, _S_Q)
    if layout == "contiguous":
        ctx = max_blocks * BLOCK
        k_pool = _normal_bf16((batch, ctx, Hkv, HEAD_DIM), device, seed, _S_K)
        v_pool = _normal_bf16((batch, ctx, Hkv, HEAD_DIM), device, seed, _S_V)
        strides = (BLOCK * Hkv * HEAD_DIM, Hkv * HEAD_DIM, HEAD_DIM)
        block_table = torch.arange(batch * max_blocks, dtype=torch.int32, device=device).reshape(batch, max_blocks)
    elif layout == "paged":
        n_pages = batch * max_blocks + extra_pages
        k_pool = _normal_bf16((n_pages, Hkv, BLOCK, HEAD_DIM), device, seed, _S_K)
        v_pool = _normal_bf16((n_pages, Hkv, BLOCK, HEAD_DIM), device, seed, _S_V)
        strides = (Hkv * BLOCK * HEAD_DIM, HEAD_DIM, BLOCK * HEAD_DIM)
        perm = torch.randperm(n_pages, generator=_gen("cpu", seed, _S_PERM))[: batch * max_blocks]
        block_table = perm.to(torch.int32).reshape(batch, max_blocks).to(device)
    else:
        raise ValueError(layout)
    w_q = _normal_bf16((Hq, HEAD_DIM, GATE_DIM), device, seed, _S_WQ, std=1.0 / math.sqrt(HEAD_DIM))
    w_k = _normal_bf16((Hkv, GATE_DIM, 3 * HEAD_DIM), device, seed, _S_WK, std=1.0 / math.sqrt(3 * HEAD_DIM))
    if random_norms:
        gn = torch.Generator(device="cpu").manual_seed(seed * 1000 + _S_NORM)
        w_qnorm = (1.0 + 0.1 * torch.randn(GATE_DIM, generator=gn)).to(device)
        w_knorm = (1.0 + 0.1 * torch.randn(GATE_DIM, generator=gn)).to(device)
    else:
        w_qnorm = torch.ones(GATE_DIM, device=device)
        w_knorm = torch.ones(GATE_DIM, device=device)
    planted = None
    if n_planted > 0:
        rng = np.random.Generator(np.random.PCG64(seed * 1000 + _S_PLANT))
        planted = np.zeros((batch, Hkv, n_planted), np.int32)
        for s in range(batch):
            local = int((lens[s] - 1) // BLOCK)
            for h in range(Hkv):
                planted[s, h] = np.sort(rng.choice(local, size=n_planted, replace=False))
    return Workload(name=name, batch=batch, n_q_heads=Hq, n_kv_heads=Hkv, max_blocks=max_blocks,
                    layout=layout, budget=budget, theta=theta,
                    seq_lens=torch.as_tensor(lens.astype(np.int32), device=device),
                    q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, w_q=w_q, w_k=w_k,
                    w_qnorm=w_qnorm.float(), w_knorm=w_knorm.float(), strides=strides,
                    planted=planted, plant_delta=plant_delta)


def make_prefill(seq_len: int, n_q_heads: int, n_kv_heads: int, budget: int, layout: str, seed: int,
                 device="cpu", max_blocks: int | None = None, random_norms: bool = False,
                 theta: float = ROPE_THETA, name: str = "prefill", extra_pages: int = 0) -> Workload:
    """One sequence of seq_len tokens for the training-time forward, as the
    batch of its positions (see Workload.prefill): K/V cache, gate weights and
    block table as make() draws them for one sequence, plus one query row per
    position, q [seq_len][Hq][128]."""
    base = make(1, n_q_heads, n_kv_heads, seq_len, budget, layout, seed, device, max_blocks=max_blocks,
                random_norms=random_norms, theta=theta, name=name, extra_pages=extra_pages)
    q = _normal_bf16((seq_len, n_q_heads, HEAD_DIM), device, seed, _S_QALL)
    lens = torch.arange(1, seq_len + 1, dtype=torch.int32, device=device)
    bt = base.block_table.expand(seq_len, base.max_blocks)
    return dataclasses.replace(base, batch=seq_len, q=q, seq_lens=lens, block_table=bt, prefill=True)


def ragged_lengths(batch: int, seed: int, lo: int = 4096, hi: int = 65536) -> np.ndarray:
    """Whole-token lengths uniform in [lo, hi] inclusive."""
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + _S_LENS))
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def named(name: str, seed: int | None = None, device="cpu", budget: int | None = None,
          **kw) -> Workload:
    """The benchmark workloads by name (see the module table)."""
    if name == "tiny":
        return make(1, 4, 1, 4096, budget or 1024, "contiguous", 1 if seed is None else seed, device,
                    n_planted=3, plant_delta=2.0, name=name, **kw)
    if name == "qwen3_4b":
        return make(8, 32, 8, 32768, budget or 2048, "contiguous", 2 if seed is None else seed, device,
                    name=name, **kw)
    if name == "qwen3_8b":
        return make(32, 32, 8, 32768, budget or 2048, "paged", 3 if seed is None else seed, device,
                    name=name, **kw)
    if name == "qwen3_14b":
        return make(4, 40, 8, 131072, budget or 2048, "paged", 4 if seed is None else seed, device,
                    n_planted=20, plant_delta=3.0, name=name, **kw)
    if name == "prefill_8b":
        # training-time forward at the training sequence length, Qwen3-8B heads
        return make_prefill(kw.pop("seq_len", 32768), 32, 8, budget or 2048, "paged", 6 if seed is None else seed,
                            device, name=name, **kw)
    if name == "ragged":
        sd = 5 if seed is None else seed
        lens = ragged_lengths(64, sd)
        steps = kw.pop("steps", 128)
        cap = int(math.ceil((65536 + steps) / BLOCK))
        return make(64, 32, 8, lens, budget or 4096, "paged", sd, device, max_blocks=cap, name=name, **kw)
    raise KeyError(name)


def append_rows(w: Workload, steps: int, seed: int, device=None):
    """Per-step new decode inputs for incremental serving: q [steps][B][Hq][128]
    and the new token's K/V rows [steps][B][Hkv][128] (bf16)."""
    device = device or w.q.device
    q = _normal_bf16((steps, w.batch, w.n_q_heads, HEAD_DIM), device, seed, _S_APPEND)
    k = _normal_bf16((steps, w.batch, w.n_kv_heads, HEAD_DIM), device, seed, _S_APPEND + 100)
    v = _normal_bf16((steps, w.batch, w.n_kv_heads, HEAD_DIM), device, seed, _S_APPEND + 200)
    return q, k, v


def random_selection(seq_lens: np.ndarray, n_kv_heads: int, budget: int, seed: int,
                     full: bool = False):
    """A valid block selection drawn at random (for exercising the attention
    stage on its own): per (sequence, KV head) min(budget/64 - 1, l) distinct
    historical blocks < l in ascending order, then the local block l =
    (L-1)/64, padded with -1; gates uniform in (0, 1), 1 for the local block.
    full=True keeps every historical block the budget allows, lowest first."""
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + _S_SEL))
    B = len(seq_lens)
    n_sel = budget // BLOCK
    sel = np.full((B, n_kv_heads, n_sel), -1, np.int32)
    gates = np.zeros((B, n_kv_heads, n_sel), np.float32)
    cnt = np.zeros((B, n_kv_heads), np.int32)
    for s in range(B):
        local = int((int(seq_lens[s]) - 1) // BLOCK)
        k = min(n_sel - 1, local)
        for h in range(n_kv_heads):
            hist = np.arange(k) if full else np.sort(rng.choice(local, size=k, replace=False))
            sel[s, h, :k] = hist
            sel[s, h, k] = local
            gates[s, h, :k] = rng.uniform(0.05, 0.95, size=k).astype(np.float32)
            gates[s, h, k] = 1.0
            cnt[s, h] = k + 1
    return sel, gates, cnt


def random_gate_keys(n_pages: int, n_kv_heads: int, seed: int, device="cpu") -> torch.Tensor:
    """Gate keys drawn directly (bf16 N(0,1)), for exercising the gate stage on
    its own."""
    return _normal_bf16((n_pages, n_kv_heads, GATE_DIM), device, seed, _S_GK)
