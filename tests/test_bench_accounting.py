"""The byte and flop accounting that bench.py's roofline lines divide by,
checked on the CPU against hand-counted figures: the decode step's
algorithmic bytes (every candidate's 256-byte gate key, 32 KiB of K and V
per selected block and KV head) and the training-time forward's
algorithmic flops (4 x 128 per attended key and query head)."""
import numpy as np

import bench


def test_decode_step_bytes_of_the_qwen3_8b_workload():
    # 32 sequences of 32,768 tokens: 511 candidate blocks each, 8 KV heads,
    # 31 historical + 1 local block selected per (sequence, KV head)
    lens = [32768] * 32
    gk = bench.gk_bytes_per_step(lens, 8)
    assert gk == 32 * 511 * 8 * 128 * 2 == 33_488_896
    cnt = np.full((32, 8), 32, np.int32)
    kv = bench.kv_bytes_per_step(cnt, 64 * 128 * 2)
    assert kv == 32 * 8 * 32 * (16384 + 16384) == 268_435_456
    assert gk + kv == 301_924_352


def test_decode_step_bytes_count_only_complete_blocks_before_the_local_one():
    # L tokens: (L - 1) // 64 candidates (a block is a candidate once complete
    # and before the block holding the current token)
    for L, n in [(1, 0), (64, 0), (65, 1), (128, 1), (129, 2), (4097, 64)]:
        assert bench.gk_bytes_per_step([L], 1) == n * 256
    assert bench.gk_bytes_per_step([65, 129], 3) == (1 + 2) * 3 * 256


def test_prefill_flops_by_hand():
    # every position t attends its historical selection (cnt - 1 whole blocks)
    # and its own block up to t
    rng = np.random.default_rng(5)
    T, Hkv, group = 300, 2, 3
    cnt = np.empty((T, Hkv), np.int64)
    for t in range(T):
        cnt[t] = 1 + rng.integers(0, t // 64 + 1, Hkv)
    want = 0
    for t in range(T):
        for k in range(Hkv):
            keys = 64 * (int(cnt[t, k]) - 1) + (t - 64 * (t // 64) + 1)
            want += keys * group * 128 * 4
    assert bench.prefill_flops(cnt, group) == float(want)


def test_prefill_flops_of_the_prefill_8b_workload():
    # 32,768 positions, 8 KV heads of 4 query heads, budget 2048: position t
    # selects min(31, t // 64) historical blocks; about 1.049 TFLOP per launch
    T = 32768
    t = np.arange(T)
    cnt = np.repeat((np.minimum(31, t // 64) + 1)[:, None], 8, axis=1)
    flops = bench.prefill_flops(cnt, 4)
    hist = np.minimum(31, t // 64) * 64
    own = t % 64 + 1
    assert flops == float(((hist + own).sum()) * 8 * 4 * 512)
    assert abs(flops / 1.049e12 - 1) < 1e-3


def test_prefill_issued_flops_when_every_query_selects_the_same_blocks():
    # a wave takes 16 / h queries of h heads (h = 4 for groups of 3 or more);
    # with identical selections each wave visits each selected block once
    T, Hkv, group = 64, 1, 4
    sel = np.tile(np.array([0, 3, 5], np.int32), (T, Hkv, 1))
    cnt = np.full((T, Hkv), 3, np.int32)
    waves = T // (16 // 4)
    mfma = 16 * 16 * 32 * 2  # flops of one 16x16x32 MFMA
    assert bench.prefill_executed_flops(sel, cnt, group) == float(waves * 3 * 32 * mfma)


def test_bench_refuses_more_than_one_gpu():
    # the path runs on one GPU: --gpus 2 (or a WORLD_SIZE above 1) exits with
    # a message and status 2 before touching any device
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2", "RANK": "0"})]:
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr
        assert r.stdout == ""
