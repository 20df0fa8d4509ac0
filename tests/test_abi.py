"""The C ABI library loads, exports every entry point include/sas.h declares,
and rejects bad arguments on the host before any GPU work (CPU only)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from learned_block_sparse_tok_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libsas.so not built")
    return ops.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"sas_pool_blocks", "sas_gate_topk", "sas_sparse_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.sas_status_str(0) == b"SAS_OK"
    assert lib.sas_status_str(3) == b"SAS_ERR_WORKSPACE"
    assert lib.sas_version() >= 100


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails its host-side checks


def _shape(**kw):
    d = dict(batch=2, n_q_heads=8, n_kv_heads=2, max_blocks=16, strides=(2 * 64 * 128, 128, 64 * 128))
    d.update(kw)
    return ops.make_shape(d["batch"], d["n_q_heads"], d["n_kv_heads"], d["max_blocks"], d["strides"])


def _gate(lib, shape, budget=1024, null_sel=False, theta=1e6):
    return lib.sas_gate_topk(ctypes.byref(shape) if shape is not None else None, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, theta, budget, None if null_sel else FAKE, FAKE, FAKE, FAKE, None)


def _decode(lib, shape, max_sel=16, ws_bytes=1 << 24, scale=0.088):
    return lib.sas_sparse_decode(ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, max_sel, scale,
                                 FAKE, FAKE, ws_bytes, None)


def test_gate_topk_rejects_bad_arguments(lib):
    assert _gate(lib, None) == ops.SAS_ERR_INVALID_ARG
    assert _gate(lib, _shape(), budget=1000) == ops.SAS_ERR_INVALID_ARG
    assert _gate(lib, _shape(), budget=0) == ops.SAS_ERR_INVALID_ARG
    assert _gate(lib, _shape(), budget=64 * 257) == ops.SAS_ERR_UNSUPPORTED
    assert _gate(lib, _shape(n_q_heads=6, n_kv_heads=4)) == ops.SAS_ERR_INVALID_ARG
    assert _gate(lib, _shape(n_q_heads=34, n_kv_heads=2)) == ops.SAS_ERR_UNSUPPORTED
    assert _gate(lib, _shape(batch=0)) == ops.SAS_ERR_INVALID_ARG
    assert _gate(lib, _shape(max_blocks=16385)) == ops.SAS_ERR_UNSUPPORTED
    assert _gate(lib, _shape(), null_sel=True) == ops.SAS_ERR_INVALID_ARG
    assert b"NULL" in lib.sas_last_error()
    assert _gate(lib, _shape(), theta=1.0) == ops.SAS_ERR_INVALID_ARG


def test_sparse_decode_rejects_bad_arguments(lib):
    assert _decode(lib, _shape(strides=(0, 128, 8192))) == ops.SAS_ERR_INVALID_ARG
    assert _decode(lib, _shape(strides=(2 * 64 * 128, 100, 64 * 128))) == ops.SAS_ERR_UNSUPPORTED
    assert _decode(lib, _shape(), max_sel=0) == ops.SAS_ERR_INVALID_ARG
    assert _decode(lib, _shape(), scale=0.0) == ops.SAS_ERR_INVALID_ARG
    assert _decode(lib, _shape(), ws_bytes=100) == ops.SAS_ERR_WORKSPACE


def _step(lib, shape, path=0, gated=0, gates=FAKE, ws=FAKE, ws_bytes=1 << 24, budget=1024, aggregate=0):
    return lib.sas_decode_step(ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e6, budget,
                               aggregate, gated, 0, 0.088, path, FAKE, gates, FAKE, None, FAKE, ws, ws_bytes, None)


def test_decode_step_rejects_bad_arguments(lib):
    sh = _shape()
    assert _step(lib, sh, path=7) == ops.SAS_ERR_INVALID_ARG
    assert _step(lib, sh, gated=2) == ops.SAS_ERR_INVALID_ARG
    assert _step(lib, sh, gated=1, gates=None) == ops.SAS_ERR_INVALID_ARG
    assert _step(lib, sh, budget=1000) == ops.SAS_ERR_INVALID_ARG
    assert _step(lib, sh, aggregate=5) == ops.SAS_ERR_INVALID_ARG
    assert _step(lib, _shape(strides=(0, 128, 8192))) == ops.SAS_ERR_INVALID_ARG
    # the two-launch path (forced, or chosen for 4 (sequence, KV head) pairs) checks its workspace
    assert _step(lib, sh, path=ops.STEP_PATH["two_launches"], ws_bytes=100) == ops.SAS_ERR_WORKSPACE
    assert _step(lib, sh, path=ops.STEP_PATH["sliced"], ws_bytes=100) == ops.SAS_ERR_WORKSPACE
    assert _step(lib, sh, path=ops.STEP_PATH["auto"], ws=None) == ops.SAS_ERR_INVALID_ARG


def test_decode_step_workspace_bytes(lib):
    small, big = _shape(), _shape(batch=32, n_q_heads=32, n_kv_heads=8)
    # fused: no workspace when every pair has its own workgroup (256 pairs on
    # 256 CUs); with few pairs, the partials of the workgroups a pair spans
    assert ops.decode_step_workspace_bytes(big, 2048, "fused") == 0
    assert ops.decode_step_workspace_bytes(small, 2048, "fused") == ops.sparse_decode_workspace_bytes(small, 32)
    for sh in (small, big):
        two = ops.decode_step_workspace_bytes(sh, 2048, "two_launches")
        # the attention's partials plus room for the scores
        assert two >= ops.sparse_decode_workspace_bytes(sh, 32) + sh.batch * sh.n_kv_heads * sh.max_blocks * 4
    # automatic: fused, or the sliced selection for few pairs once the block
    # table is over 1,024 blocks
    long = _shape(max_blocks=2048)
    assert ops.decode_step_workspace_bytes(big, 2048, "auto") == 0
    assert ops.decode_step_workspace_bytes(small, 2048, "auto") == ops.decode_step_workspace_bytes(small, 2048,
                                                                                                  "fused")
    assert ops.decode_step_workspace_bytes(long, 2048, "auto") == ops.decode_step_workspace_bytes(long, 2048,
                                                                                                 "sliced")
    # the sliced path adds each pair's slice lists (score key, block, page per entry)
    assert ops.decode_step_workspace_bytes(small, 2048, "sliced") > ops.decode_step_workspace_bytes(small, 2048,
                                                                                                   "two_launches")


def test_pool_rejects_bad_arguments_and_accepts_empty_list(lib):
    sh = _shape()
    assert lib.sas_pool_blocks(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, 1e6, FAKE, None) == \
        ops.SAS_ERR_INVALID_ARG
    assert lib.sas_pool_blocks(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, 3, FAKE, FAKE, 0.5, FAKE, None) == \
        ops.SAS_ERR_INVALID_ARG
    assert lib.sas_pool_blocks(ctypes.byref(sh), None, FAKE, FAKE, FAKE, 3, FAKE, FAKE, 1e6, FAKE, None) == \
        ops.SAS_ERR_INVALID_ARG
    # an empty list enqueues nothing and succeeds
    assert lib.sas_pool_blocks(ctypes.byref(sh), None, None, None, None, 0, None, None, 1e6, None, None) == ops.SAS_OK


def test_append_rejects_bad_arguments(lib):
    sh = _shape()

    def call(sh=sh, k_new=FAKE, theta=1e6, pool=FAKE):
        return lib.sas_append_kv(ctypes.byref(sh), k_new, FAKE, pool, FAKE, FAKE, FAKE, FAKE, FAKE, theta, FAKE,
                                 None)

    assert call(k_new=None) == ops.SAS_ERR_INVALID_ARG
    assert call(theta=1.0) == ops.SAS_ERR_INVALID_ARG
    assert call(pool=ctypes.c_void_p(4096 + 2)) == ops.SAS_ERR_UNSUPPORTED  # not 16-byte aligned
    assert call(sh=_shape(strides=(2 * 64 * 128, 0, 64 * 128))) == ops.SAS_ERR_INVALID_ARG
    assert call(sh=_shape(n_kv_heads=3)) == ops.SAS_ERR_INVALID_ARG  # 8 query heads not a multiple of 3


def test_prefill_rejects_bad_arguments(lib):
    sh1 = _shape(batch=1)

    def sel_call(sh=sh1, T=100, budget=128, q=FAKE):
        return lib.sas_prefill_select(ctypes.byref(sh), q, FAKE, FAKE, FAKE, FAKE, T, 1e6, budget, FAKE, FAKE, FAKE,
                                      None, None)

    def att_call(sh=sh1, T=100, max_sel=2, out=FAKE):
        return lib.sas_prefill_attend(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, T, FAKE, None, FAKE, max_sel, 0.088,
                                      out, None, None)

    assert sel_call(sh=_shape(batch=2)) == ops.SAS_ERR_INVALID_ARG  # one sequence per call
    assert sel_call(T=0) == ops.SAS_ERR_INVALID_ARG
    assert sel_call(T=16 * 64 + 1) == ops.SAS_ERR_INVALID_ARG  # needs 17 blocks, max_blocks 16
    assert sel_call(budget=100) == ops.SAS_ERR_INVALID_ARG
    assert sel_call(q=None) == ops.SAS_ERR_INVALID_ARG
    assert att_call(sh=_shape(batch=3)) == ops.SAS_ERR_INVALID_ARG
    assert att_call(T=-5) == ops.SAS_ERR_INVALID_ARG
    assert att_call(max_sel=0) == ops.SAS_ERR_INVALID_ARG
    assert att_call(max_sel=65) == ops.SAS_ERR_UNSUPPORTED
    assert att_call(out=None) == ops.SAS_ERR_INVALID_ARG
    assert att_call(out=ctypes.c_void_p(4096 + 8)) == ops.SAS_ERR_UNSUPPORTED  # not 16-byte aligned


def test_variant_entry_points_reject_bad_modes(lib):
    sh = _shape()
    gate = lambda agg, shp=sh: lib.sas_gate_topk_ex(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e6, 1024,
                                                   agg, FAKE, FAKE, FAKE, FAKE, None)
    assert gate(2) == ops.SAS_ERR_INVALID_ARG
    assert gate(1, _shape(n_q_heads=32, n_kv_heads=2)) == ops.SAS_ERR_UNSUPPORTED  # group 16 > 8 for max
    dec = lambda mode: lib.sas_sparse_decode_ex(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mode,
                                                FAKE, 16, 0.088, FAKE, FAKE, 1 << 24, None)
    assert dec(5) == ops.SAS_ERR_INVALID_ARG
    assert dec(-1) == ops.SAS_ERR_INVALID_ARG


def test_gate_backward_rejects_bad_arguments(lib):
    sh = _shape()
    need = lib.sas_gate_backward_workspace_bytes(ctypes.byref(sh), 16)
    assert need > 0

    def call(gates=FAKE, max_sel=16, ws_bytes=need, theta=1e6):
        return lib.sas_gate_backward(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, gates, FAKE, max_sel, 0.088,
                                     FAKE, FAKE, FAKE, FAKE, FAKE, theta, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     ws_bytes, None)

    assert call(gates=None) == ops.SAS_ERR_INVALID_ARG  # gated steps only
    assert call(max_sel=0) == ops.SAS_ERR_INVALID_ARG
    assert call(theta=0.5) == ops.SAS_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == ops.SAS_ERR_WORKSPACE


def test_workspace_sizes(lib):
    # 256 (sequence, KV head) units fill the CUs: one workgroup each, no partials
    sh = _shape(batch=32, n_q_heads=32, n_kv_heads=8, max_blocks=512)
    assert lib.sas_sparse_decode_workspace_bytes(ctypes.byref(sh), 32) >= 0
    # few units: each is split over several workgroups whose partials need room
    sh = _shape(batch=4, n_q_heads=40, n_kv_heads=8, max_blocks=2048)
    assert lib.sas_sparse_decode_workspace_bytes(ctypes.byref(sh), 32) >= 2 * 4 * 40 * 130 * 4
    assert lib.sas_sparse_decode_workspace_bytes(ctypes.byref(sh), 0) == 0


def test_probe_read_rejects_bad_arguments_and_accepts_empty_list(lib):
    aligned = ctypes.c_void_p(0x10000)
    assert lib.sas_probe_read(FAKE, -1, 1, aligned, 64, None) == ops.SAS_ERR_INVALID_ARG
    assert lib.sas_probe_read(FAKE, 4, 0, aligned, 64, None) == ops.SAS_ERR_INVALID_ARG
    assert lib.sas_probe_read(FAKE, 4, 65, aligned, 64, None) == ops.SAS_ERR_INVALID_ARG
    assert lib.sas_probe_read(None, 4, 1, aligned, 64, None) == ops.SAS_ERR_INVALID_ARG
    assert lib.sas_probe_read(FAKE, 4, 1, None, 64, None) == ops.SAS_ERR_INVALID_ARG
    assert lib.sas_probe_read(FAKE, 4, 1, ctypes.c_void_p(0x10008), 64, None) == ops.SAS_ERR_INVALID_ARG
    assert lib.sas_probe_read(FAKE, 5, 2, aligned, 47, None) == ops.SAS_ERR_INVALID_ARG  # needs 3 words
    assert lib.sas_probe_read(None, 0, 1, None, 0, None) == ops.SAS_OK


def test_prefill_gate_backward_rejects_bad_arguments(lib):
    sh1 = _shape(batch=1)
    T = 1000
    need = lib.sas_prefill_gate_backward_workspace_bytes(ctypes.byref(sh1), T, 16)
    # the dense position x block matrix dominates: Hkv * T * (blocks rounded up to 64) floats
    assert need >= 2 * T * 64 * 4
    assert lib.sas_prefill_gate_backward_workspace_bytes(ctypes.byref(sh1), 0, 16) == 0

    def call(sh=sh1, T=T, lse=FAKE, max_sel=16, ws_bytes=need, theta=1e6, ws=FAKE):
        return lib.sas_prefill_gate_backward(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, T, FAKE, FAKE, FAKE, max_sel,
                                             0.088, lse, FAKE, FAKE, FAKE, FAKE, FAKE, theta, FAKE, FAKE, FAKE, FAKE,
                                             FAKE, FAKE, ws, ws_bytes, None)

    assert call(sh=_shape(batch=2)) == ops.SAS_ERR_INVALID_ARG  # one sequence per call
    assert call(T=0) == ops.SAS_ERR_INVALID_ARG
    assert call(T=16 * 64 + 1) == ops.SAS_ERR_INVALID_ARG  # needs 17 blocks, max_blocks 16
    assert call(lse=None) == ops.SAS_ERR_INVALID_ARG  # the forward's log-sum-exp is required
    assert call(max_sel=0) == ops.SAS_ERR_INVALID_ARG
    assert call(max_sel=65) == ops.SAS_ERR_UNSUPPORTED
    assert call(theta=1.0) == ops.SAS_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == ops.SAS_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(4096 + 4)) == ops.SAS_ERR_UNSUPPORTED  # not 16-byte aligned
