"""libdora: the DoRA factored row-norm and magnitude compose on MI355X (gfx950).

The compute lives in hand-written HIP kernels inside ``libdora.so`` (a C ABI
declared in ``include/dora.h``). This package holds the ctypes binding that
marshals torch tensors to that ABI, the seeded input generators, and the
build helper. Importing the package does not load the library; the first
call does, and raises if the library is missing.
"""

__all__ = [
    "dora_factored_norm",
    "dora_compose",
    "dora_magnitude_scale",
    "dora_norm_workspace_size",
    "dora_norm_chunk_size",
]


def __getattr__(name):
    if name in __all__:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
