"""Expert-cached MoE layer for AMD Instinct MI355X (gfx950).

The compute path lives in ``libmoecache.so`` (hand-written HIP kernels and a C++
host library behind the C ABI of ``include/moe.h``).  ``binding`` exposes every
entry point under its C name; ``runtime`` allocates the device buffers a layer
needs with torch.  Build first: ``python -m expert_cached_moe_amd.build``.
"""


def __getattr__(name):
    if name in ("binding", "runtime"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
