"""Flash-LoRA-Attention and the PreLRShared LR precompute for MI355X (gfx950).

The compute lives in ``liblra.so`` (hand-written HIP kernels behind a C ABI, declared in
``include/lra.h``); ``shared_rank_kv_amd.lra`` is its thin ctypes binding.  The binding
is imported lazily so that input generation and workload definitions work on hosts
without a GPU.
"""

__all__ = ["lra", "inputs", "workloads", "accounting"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
