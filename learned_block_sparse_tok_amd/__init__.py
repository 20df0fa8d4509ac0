"""MI355X-native SAS sparse decode: gated KV-block selection + block-sparse
flash-decode, as hand-written HIP kernels for gfx950 behind a C ABI
(``include/sas.h``).

``learned_block_sparse_tok_amd.ops`` is the thin Python binding (argument
marshalling over ctypes; torch supplies device memory and the stream).
``learned_block_sparse_tok_amd.workloads`` draws seeded synthetic inputs.
"""
__all__ = ["ops", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
