"""MI355X-native KDA (Kimi Delta Attention) chunked forward and paged decode.

The compute lives in a C-ABI shared library of hand-written gfx950 HIP
kernels (``csrc/``, declared in ``include/kda.h``); ``binding`` is a thin
ctypes layer over it.  Importing the package does not load the library; the
first call does, and raises if it is missing.
"""
_EXPORTS = ("KdaError", "chunk_kda", "kda_decode", "chunk_stages", "library_path",
            "load_library")


def __getattr__(name):
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)


__all__ = list(_EXPORTS)
