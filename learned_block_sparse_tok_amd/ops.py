"""Thin Python binding of libsas (include/sas.h) over ctypes.

Argument marshalling only: every step of the SAS decode path runs in the HIP
kernels of libsas.so.  torch supplies device memory (tensors) and the stream
(the current torch stream unless one is given).  There is no fallback: if
libsas.so is missing or cannot load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsas.so")
BLOCK = 64
HEAD_DIM = 128
GATE_DIM = 128

SAS_OK, SAS_ERR_INVALID_ARG, SAS_ERR_UNSUPPORTED, SAS_ERR_WORKSPACE, SAS_ERR_HIP = range(5)


class SasError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn} failed: {_status_str(status)}: {detail}")
        self.status = status


class SasShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("page_stride", ctypes.c_int64), ("tok_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


_lib = None
_VP, _I32, _F32, _F64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
_SIGS = {
    "sas_pool_blocks": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _F64, _VP, _VP]),
    "sas_append_kv": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F64, _VP, _VP]),
    "sas_gate_topk_ex": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _F64, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "sas_sparse_decode_ex": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _I32, _F32, _VP, _VP, _SZ,
                                    _VP]),
    "sas_gate_topk": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _F64, _I32, _VP, _VP, _VP, _VP, _VP]),
    "sas_sparse_decode_workspace_bytes": (_SZ, [_VP, _I32]),
    "sas_sparse_decode": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _F32, _VP, _VP, _SZ, _VP]),
    "sas_decode_step_workspace_bytes": (_SZ, [_VP, _I32, _I32]),
    "sas_probe_read": (_I32, [_VP, _I32, _I32, _VP, _SZ, _VP]),
    "sas_decode_step": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F64, _I32, _I32, _I32, _I32, _F32, _I32,
                               _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sas_decode_step_noalloc": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F64, _I32, _I32, _I32, _I32,
                                       _F32, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "sas_prefill_select": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _F64, _I32, _VP, _VP, _VP, _VP, _VP]),
    "sas_prefill_attend": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _F32, _VP, _VP, _VP]),
    "sas_prefill_gate_backward_workspace_bytes": (_SZ, [_VP, _I32, _I32]),
    "sas_prefill_gate_backward": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _I32, _F32, _VP, _VP, _VP,
                                         _VP, _VP, _VP, _F64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sas_gate_backward_workspace_bytes": (_SZ, [_VP, _I32]),
    "sas_gate_backward": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _F32, _VP, _VP, _VP, _VP, _VP,
                                 _F64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sas_status_str": (ctypes.c_char_p, [_I32]),
    "sas_last_error": (ctypes.c_char_p, []),
    "sas_version": (_I32, []),
}


def lib() -> ctypes.CDLL:
    """Load libsas.so (built in-tree by learned_block_sparse_tok_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m learned_block_sparse_tok_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _status_str(st: int) -> str:
    return lib().sas_status_str(st).decode()


def _check(st: int, fn: str):
    if st != SAS_OK:
        raise SasError(st, fn, lib().sas_last_error().decode())


def _ptr(t: torch.Tensor | None, dtype=None, name="tensor"):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(batch, n_q_heads, n_kv_heads, max_blocks, strides=(0, 0, 0)) -> SasShape:
    ps, ts, hs = strides
    return SasShape(batch, n_q_heads, n_kv_heads, max_blocks, ps, ts, hs)


def sparse_decode_workspace_bytes(shape: SasShape, max_sel: int) -> int:
    return int(lib().sas_sparse_decode_workspace_bytes(ctypes.byref(shape), max_sel))


def pool_blocks(shape: SasShape, k_pool, block_table, pool_seq, pool_blk, w_k, w_knorm, theta,
                gate_keys, stream=None):
    n = int(pool_seq.numel())
    st = lib().sas_pool_blocks(ctypes.byref(shape), _ptr(k_pool, torch.bfloat16, "k_pool"),
                               _ptr(block_table, torch.int32, "block_table"),
                               _ptr(pool_seq, torch.int32, "pool_seq"), _ptr(pool_blk, torch.int32, "pool_blk"),
                               n, _ptr(w_k, torch.bfloat16, "w_k"), _ptr(w_knorm, torch.float32, "w_knorm"),
                               float(theta), _ptr(gate_keys, torch.bfloat16, "gate_keys"), _stream(stream))
    _check(st, "sas_pool_blocks")


def append_kv(shape: SasShape, k_new, v_new, k_pool, v_pool, block_table, seq_lens, w_k, w_knorm, theta,
              gate_keys, stream=None):
    """The new token's K/V rows ([B][Hkv][128]) into the pools at position
    seq_lens[s]-1; blocks this completes are pooled into gate_keys."""
    st = lib().sas_append_kv(ctypes.byref(shape), _ptr(k_new, torch.bfloat16, "k_new"),
                             _ptr(v_new, torch.bfloat16, "v_new"), _ptr(k_pool, torch.bfloat16, "k_pool"),
                             _ptr(v_pool, torch.bfloat16, "v_pool"), _ptr(block_table, torch.int32, "block_table"),
                             _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(w_k, torch.bfloat16, "w_k"),
                             _ptr(w_knorm, torch.float32, "w_knorm"), float(theta),
                             _ptr(gate_keys, torch.bfloat16, "gate_keys"), _stream(stream))
    _check(st, "sas_append_kv")


AGGREGATE = {"mean": 0, "max": 1}  # SAS_AGG_MEAN, SAS_AGG_MAX
GATE_MODE = {"scale": 0, "logit": 1}  # SAS_GATE_SCALE, SAS_GATE_LOGIT


def gate_topk(shape: SasShape, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, theta, budget_tokens,
              sel, gates, cnt, scores, stream=None, aggregate="mean"):
    """sas_gate_topk (aggregate "mean") or sas_gate_topk_ex."""
    args = (ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"), _ptr(w_q, torch.bfloat16, "w_q"),
            _ptr(w_qnorm, torch.float32, "w_qnorm"), _ptr(gate_keys, torch.bfloat16, "gate_keys"),
            _ptr(block_table, torch.int32, "block_table"), _ptr(seq_lens, torch.int32, "seq_lens"),
            float(theta), int(budget_tokens))
    outs = (_ptr(sel, torch.int32, "sel"), _ptr(gates, torch.float32, "gates"), _ptr(cnt, torch.int32, "cnt"),
            _ptr(scores, torch.float32, "scores"), _stream(stream))
    if aggregate == "mean":
        st = lib().sas_gate_topk(*args, *outs)
    else:
        st = lib().sas_gate_topk_ex(*args, AGGREGATE[aggregate], *outs)
    _check(st, "sas_gate_topk")


def sparse_decode(shape: SasShape, q, k_pool, v_pool, block_table, seq_lens, sel, gates, cnt, max_sel,
                  sm_scale, out, workspace, stream=None, gate_mode="scale"):
    """sas_sparse_decode (gate_mode "scale") or sas_sparse_decode_ex."""
    head = (ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.bfloat16, "k_pool"),
            _ptr(v_pool, torch.bfloat16, "v_pool"), _ptr(block_table, torch.int32, "block_table"),
            _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(sel, torch.int32, "sel"), _ptr(gates, torch.float32, "gates"))
    tail = (_ptr(cnt, torch.int32, "cnt"), int(max_sel), float(sm_scale), _ptr(out, torch.bfloat16, "out"),
            _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    if gate_mode == "scale":
        st = lib().sas_sparse_decode(*head, *tail)
    else:
        st = lib().sas_sparse_decode_ex(*head, GATE_MODE[gate_mode], *tail)
    _check(st, "sas_sparse_decode")


# SAS_STEP_AUTO, SAS_STEP_FUSED, SAS_STEP_TWO_LAUNCHES, SAS_STEP_SLICED
STEP_PATH = {"auto": 0, "fused": 1, "two_launches": 2, "sliced": 3}


def probe_read(chunk_addr, chunks_per_wg, sink=None, stream=None):
    """sas_probe_read (measurement utility): reads the 16 KiB chunks whose
    device addresses chunk_addr (int64 device tensor) lists; returns sink,
    int32 [ceil(n / chunks_per_wg)][4]: the XOR of each workgroup's words."""
    n = chunk_addr.numel()
    words = (n + chunks_per_wg - 1) // chunks_per_wg
    if sink is None:
        sink = torch.empty((max(words, 1), 4), dtype=torch.int32, device=chunk_addr.device)
    st = lib().sas_probe_read(_ptr(chunk_addr, torch.int64, "chunk_addr"), int(n), int(chunks_per_wg),
                              _ptr(sink, torch.int32, "sink"), sink.numel() * 4, _stream(stream))
    _check(st, "sas_probe_read")
    return sink


def decode_step_workspace_bytes(shape: SasShape, budget_tokens: int, path="auto") -> int:
    return int(lib().sas_decode_step_workspace_bytes(ctypes.byref(shape), int(budget_tokens), STEP_PATH[path]))


def _decode_step_args(shape: SasShape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, theta,
                      budget_tokens, sel, gates, cnt, scores, out, workspace, sm_scale, gated, stream=None,
                      aggregate="mean", gate_mode="scale", path="auto"):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"), _ptr(w_q, torch.bfloat16, "w_q"),
            _ptr(w_qnorm, torch.float32, "w_qnorm"), _ptr(gate_keys, torch.bfloat16, "gate_keys"),
            _ptr(k_pool, torch.bfloat16, "k_pool"), _ptr(v_pool, torch.bfloat16, "v_pool"),
            _ptr(block_table, torch.int32, "block_table"), _ptr(seq_lens, torch.int32, "seq_lens"),
            float(theta), int(budget_tokens), AGGREGATE[aggregate], int(bool(gated)),
            GATE_MODE[gate_mode], float(sm_scale), STEP_PATH[path], _ptr(sel, torch.int32, "sel"),
            _ptr(gates, torch.float32, "gates"), _ptr(cnt, torch.int32, "cnt"),
            _ptr(scores, torch.float32, "scores"), _ptr(out, torch.bfloat16, "out"),
            _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream))


def decode_step(shape: SasShape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, theta,
                budget_tokens, sel, gates, cnt, scores, out, workspace, sm_scale, gated, stream=None,
                aggregate="mean", gate_mode="scale", path="auto"):
    """sas_decode_step: selection then attention in one call (one fused launch
    on the "fused" path); gates / scores / workspace may be None where the
    header allows."""
    args = _decode_step_args(shape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, theta,
                             budget_tokens, sel, gates, cnt, scores, out, workspace, sm_scale, gated, stream,
                             aggregate, gate_mode, path)
    _check(lib().sas_decode_step(*args), "sas_decode_step")


class PreparedCall:
    """One C-ABI call whose arguments were checked and marshalled once: each
    call() passes the same pointers and sizes again, as a serving loop that
    keeps its buffers does, on the given stream or, if none was given, on the
    stream current at the call (so that the call can be captured into a graph).
    It keeps the tensors it points to alive."""

    def __init__(self, fn, name, args, keep, stream=None):
        self._fn, self._name, self._keep = fn, name, keep
        self._args = args[:-1]
        self._stream = None if stream is None else args[-1]

    def __call__(self):
        st = self._fn(*self._args, self._stream if self._stream is not None else _stream(None))
        if st != SAS_OK:
            _check(st, self._name)


NOALLOC_SCRATCH_BYTES = 16 << 20  # SAS_NOALLOC_SCRATCH_BYTES


def decode_step_noalloc(shape: SasShape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, theta,
                        budget_tokens, sel, gates, cnt, scores, out, sm_scale, gated, stream=None, aggregate="mean",
                        gate_mode="scale", path="auto"):
    """sas_decode_step_noalloc: decode_step with the library's per-device
    scratch array in place of a workspace (no allocation in the call; calls
    that overlap on one device race)."""
    st = lib().sas_decode_step_noalloc(ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"),
                                       _ptr(w_q, torch.bfloat16, "w_q"), _ptr(w_qnorm, torch.float32, "w_qnorm"),
                                       _ptr(gate_keys, torch.bfloat16, "gate_keys"),
                                       _ptr(k_pool, torch.bfloat16, "k_pool"), _ptr(v_pool, torch.bfloat16, "v_pool"),
                                       _ptr(block_table, torch.int32, "block_table"),
                                       _ptr(seq_lens, torch.int32, "seq_lens"), float(theta), int(budget_tokens),
                                       AGGREGATE[aggregate], int(bool(gated)), GATE_MODE[gate_mode], float(sm_scale),
                                       STEP_PATH[path], _ptr(sel, torch.int32, "sel"),
                                       _ptr(gates, torch.float32, "gates"), _ptr(cnt, torch.int32, "cnt"),
                                       _ptr(scores, torch.float32, "scores"), _ptr(out, torch.bfloat16, "out"),
                                       _stream(stream))
    _check(st, "sas_decode_step_noalloc")


class SparseDecoder:
    """Holds the outputs and workspaces of one layer's decode step (allocated
    once, by torch).  step() runs sas_decode_step on the given path ("auto":
    one fused launch when there are enough (sequence, KV head) pairs to fill
    the GPU; see sas.h for the others); select() and attend() run
    sas_gate_topk and sas_sparse_decode.  keep_scores=False leaves the
    optional per-candidate score output off (scores is None), as a serving
    caller that needs only the selection and the attention output would."""

    def __init__(self, batch, n_q_heads, n_kv_heads, max_blocks, strides, budget, theta, gated,
                 device="cuda", sm_scale=None, aggregate="mean", gate_mode="scale", path="auto", keep_scores=True):
        self.shape = make_shape(batch, n_q_heads, n_kv_heads, max_blocks, strides)
        self.budget, self.theta, self.gated = budget, theta, gated
        self.aggregate, self.gate_mode, self.path = aggregate, gate_mode, path
        self.n_sel = budget // BLOCK
        self.sm_scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(HEAD_DIM)
        dev = torch.device(device)
        self.sel = torch.empty((batch, n_kv_heads, self.n_sel), dtype=torch.int32, device=dev)
        self.gates = torch.empty((batch, n_kv_heads, self.n_sel), dtype=torch.float32, device=dev)
        self.cnt = torch.empty((batch, n_kv_heads), dtype=torch.int32, device=dev)
        self.scores = (torch.empty((batch, n_kv_heads, max_blocks), dtype=torch.float32, device=dev)
                       if keep_scores else None)
        self.out = torch.empty((batch, n_q_heads, HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.ws_dec = torch.empty(sparse_decode_workspace_bytes(self.shape, self.n_sel), dtype=torch.uint8,
                                  device=dev)
        nws = decode_step_workspace_bytes(self.shape, budget, path)
        self.ws_step = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

    def select(self, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, stream=None):
        gate_topk(self.shape, q, w_q, w_qnorm, gate_keys, block_table, seq_lens, self.theta, self.budget,
                  self.sel, self.gates, self.cnt, self.scores, stream, aggregate=self.aggregate)

    def attend(self, q, k_pool, v_pool, block_table, seq_lens, stream=None):
        sparse_decode(self.shape, q, k_pool, v_pool, block_table, seq_lens, self.sel,
                      self.gates if self.gated else None, self.cnt, self.n_sel, self.sm_scale, self.out,
                      self.ws_dec, stream, gate_mode=self.gate_mode)

    def step(self, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, stream=None):
        decode_step(self.shape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, self.theta,
                    self.budget, self.sel, self.gates, self.cnt, self.scores, self.out, self.ws_step, self.sm_scale,
                    self.gated, stream, aggregate=self.aggregate, gate_mode=self.gate_mode, path=self.path)
        return self.out

    def prepare_step(self, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens, stream=None):
        """step() with its arguments checked and marshalled once: the returned
        call launches sas_decode_step on these tensors (and the stream current
        now) each time it is called."""
        keep = (self, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens)  # outputs live in self
        args = _decode_step_args(self.shape, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table, seq_lens,
                                 self.theta, self.budget, self.sel, self.gates, self.cnt, self.scores, self.out,
                                 self.ws_step, self.sm_scale, self.gated, stream, aggregate=self.aggregate,
                                 gate_mode=self.gate_mode, path=self.path)
        return PreparedCall(lib().sas_decode_step, "sas_decode_step", args, keep, stream)


def prefill_select(shape: SasShape, q, w_q, w_qnorm, gate_keys, block_table_row, seq_len, theta, budget_tokens,
                   sel, gates, cnt, scores=None, stream=None):
    """Gate query, block scores and Top-K for every position of one sequence
    (q [T][Hq][128]); sel / gates [T][Hkv][budget/64], cnt [T][Hkv]."""
    st = lib().sas_prefill_select(ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"), _ptr(w_q, torch.bfloat16, "w_q"),
                                  _ptr(w_qnorm, torch.float32, "w_qnorm"),
                                  _ptr(gate_keys, torch.bfloat16, "gate_keys"),
                                  _ptr(block_table_row, torch.int32, "block_table_row"), int(seq_len), float(theta),
                                  int(budget_tokens), _ptr(sel, torch.int32, "sel"),
                                  _ptr(gates, torch.float32, "gates"), _ptr(cnt, torch.int32, "cnt"),
                                  _ptr(scores, torch.float32, "scores"), _stream(stream))
    _check(st, "sas_prefill_select")


def prefill_attend(shape: SasShape, q, k_pool, v_pool, block_table_row, seq_len, sel, gates, cnt, max_sel, sm_scale,
                   out, lse=None, stream=None):
    """Attention of every position of one sequence over its own selection
    (gates None: plain mode); out bf16 [T][Hq][128]; lse (optional) fp32
    [T][Hq], the log-sum-exp of each query head's logits."""
    st = lib().sas_prefill_attend(ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"),
                                  _ptr(k_pool, torch.bfloat16, "k_pool"), _ptr(v_pool, torch.bfloat16, "v_pool"),
                                  _ptr(block_table_row, torch.int32, "block_table_row"), int(seq_len),
                                  _ptr(sel, torch.int32, "sel"), _ptr(gates, torch.float32, "gates"),
                                  _ptr(cnt, torch.int32, "cnt"), int(max_sel), float(sm_scale),
                                  _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream))
    _check(st, "sas_prefill_attend")


def prefill_gate_backward_workspace_bytes(shape: SasShape, seq_len: int, max_sel: int) -> int:
    return int(lib().sas_prefill_gate_backward_workspace_bytes(ctypes.byref(shape), int(seq_len), int(max_sel)))


def prefill_gate_backward(shape: SasShape, q, k_pool, v_pool, block_table_row, seq_len, sel, gates, cnt, max_sel,
                          sm_scale, lse, w_q, w_qnorm, w_k, w_knorm, gate_keys, theta, d_out, workspace=None,
                          stream=None, out=None):
    """Gradients of the gate parameters through the continuous gates of the
    training-time forward of one sequence.  Returns dict(d_gates, d_w_q,
    d_w_qnorm, d_w_k, d_w_knorm) (fp32 device tensors; `out` may supply
    them preallocated)."""
    dev = q.device
    T, Hq, _ = q.shape
    Hkv = shape.n_kv_heads
    if out is None:
        out = dict(d_gates=torch.empty((T, Hkv, max_sel), dtype=torch.float32, device=dev),
                   d_w_q=torch.empty((Hq, 128, 128), dtype=torch.float32, device=dev),
                   d_w_qnorm=torch.empty(128, dtype=torch.float32, device=dev),
                   d_w_k=torch.empty((Hkv, 128, 384), dtype=torch.float32, device=dev),
                   d_w_knorm=torch.empty(128, dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = torch.empty(prefill_gate_backward_workspace_bytes(shape, seq_len, max_sel), dtype=torch.uint8,
                                device=dev)
    st = lib().sas_prefill_gate_backward(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.bfloat16, "k_pool"),
        _ptr(v_pool, torch.bfloat16, "v_pool"), _ptr(block_table_row, torch.int32, "block_table_row"), int(seq_len),
        _ptr(sel, torch.int32, "sel"), _ptr(gates, torch.float32, "gates"), _ptr(cnt, torch.int32, "cnt"),
        int(max_sel), float(sm_scale), _ptr(lse, torch.float32, "lse"), _ptr(w_q, torch.bfloat16, "w_q"),
        _ptr(w_qnorm, torch.float32, "w_qnorm"), _ptr(w_k, torch.bfloat16, "w_k"),
        _ptr(w_knorm, torch.float32, "w_knorm"), _ptr(gate_keys, torch.bfloat16, "gate_keys"), float(theta),
        _ptr(d_out, torch.bfloat16, "d_out"), _ptr(out["d_gates"]), _ptr(out["d_w_q"]), _ptr(out["d_w_qnorm"]),
        _ptr(out["d_w_k"]), _ptr(out["d_w_knorm"]), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "sas_prefill_gate_backward")
    return out


class Prefill:
    """Outputs of the training-time forward of one sequence of seq_len tokens
    (selection + attention), allocated once; forward() runs both calls."""

    def __init__(self, n_q_heads, n_kv_heads, max_blocks, strides, seq_len, budget_tokens, theta, gated,
                 device="cuda", sm_scale=None, keep_scores=False):
        self.shape = make_shape(1, n_q_heads, n_kv_heads, max_blocks, strides)
        self.seq_len, self.budget, self.theta, self.gated = seq_len, budget_tokens, theta, gated
        self.max_sel = budget_tokens // 64
        self.sm_scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(128.0)
        self.sel = torch.empty((seq_len, n_kv_heads, self.max_sel), dtype=torch.int32, device=device)
        self.gates = torch.empty((seq_len, n_kv_heads, self.max_sel), dtype=torch.float32, device=device)
        self.cnt = torch.empty((seq_len, n_kv_heads), dtype=torch.int32, device=device)
        self.scores = (torch.empty((seq_len, n_kv_heads, max_blocks), dtype=torch.float32, device=device)
                       if keep_scores else None)
        self.out = torch.empty((seq_len, n_q_heads, 128), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((seq_len, n_q_heads), dtype=torch.float32, device=device)

    def select(self, q, w_q, w_qnorm, gate_keys, block_table_row, stream=None):
        prefill_select(self.shape, q, w_q, w_qnorm, gate_keys, block_table_row, self.seq_len, self.theta, self.budget,
                       self.sel, self.gates, self.cnt, self.scores, stream)

    def attend(self, q, k_pool, v_pool, block_table_row, stream=None):
        prefill_attend(self.shape, q, k_pool, v_pool, block_table_row, self.seq_len, self.sel,
                       self.gates if self.gated else None, self.cnt, self.max_sel, self.sm_scale, self.out,
                       self.lse, stream)

    def forward(self, q, w_q, w_qnorm, gate_keys, k_pool, v_pool, block_table_row, stream=None):
        self.select(q, w_q, w_qnorm, gate_keys, block_table_row, stream)
        self.attend(q, k_pool, v_pool, block_table_row, stream)


def gate_backward_workspace_bytes(shape: SasShape, max_sel: int) -> int:
    return int(lib().sas_gate_backward_workspace_bytes(ctypes.byref(shape), max_sel))


def gate_backward(shape: SasShape, q, k_pool, v_pool, block_table, seq_lens, sel, gates, cnt, max_sel, sm_scale,
                  w_q, w_qnorm, w_k, w_knorm, gate_keys, theta, d_out, workspace=None, stream=None, out=None):
    """Gradients of the gate parameters through the continuous gates of a gated
    decode step.  Returns dict(d_gates, d_w_q, d_w_qnorm, d_w_k, d_w_knorm)
    (fp32 device tensors; `out` may supply them preallocated)."""
    dev = q.device
    B, Hq, _ = q.shape
    Hkv = shape.n_kv_heads
    if out is None:
        out = dict(d_gates=torch.empty((B, Hkv, max_sel), dtype=torch.float32, device=dev),
                   d_w_q=torch.empty((Hq, 128, 128), dtype=torch.float32, device=dev),
                   d_w_qnorm=torch.empty(128, dtype=torch.float32, device=dev),
                   d_w_k=torch.empty((Hkv, 128, 384), dtype=torch.float32, device=dev),
                   d_w_knorm=torch.empty(128, dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = torch.empty(gate_backward_workspace_bytes(shape, max_sel), dtype=torch.uint8, device=dev)
    st = lib().sas_gate_backward(ctypes.byref(shape), _ptr(q, torch.bfloat16, "q"),
                                 _ptr(k_pool, torch.bfloat16, "k_pool"), _ptr(v_pool, torch.bfloat16, "v_pool"),
                                 _ptr(block_table, torch.int32, "block_table"), _ptr(seq_lens, torch.int32, "seq_lens"),
                                 _ptr(sel, torch.int32, "sel"), _ptr(gates, torch.float32, "gates"),
                                 _ptr(cnt, torch.int32, "cnt"), int(max_sel), float(sm_scale),
                                 _ptr(w_q, torch.bfloat16, "w_q"), _ptr(w_qnorm, torch.float32, "w_qnorm"),
                                 _ptr(w_k, torch.bfloat16, "w_k"), _ptr(w_knorm, torch.float32, "w_knorm"),
                                 _ptr(gate_keys, torch.bfloat16, "gate_keys"), float(theta),
                                 _ptr(d_out, torch.bfloat16, "d_out"), _ptr(out["d_gates"]), _ptr(out["d_w_q"]),
                                 _ptr(out["d_w_qnorm"]), _ptr(out["d_w_k"]), _ptr(out["d_w_knorm"]),
                                 _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    _check(st, "sas_gate_backward")
    return out
