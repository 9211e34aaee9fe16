"""libqb: block-wise dynamic quantization, nested quantization of the block
constants, and the fused 8-bit AdamW step, as HIP kernels for MI355X (gfx950)
behind a C ABI (include/qb.h).

`bit_optimizer_states_amd.binding` holds the thin ctypes binding (same names as
the C ABI; torch tensors in, device pointers out).  The shared library is
loaded on first use and an ImportError/OSError is raised loudly when it is
missing: there is no CPU fallback.
"""

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
