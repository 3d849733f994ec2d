"""MI355X-native score-and-select compression of a prompt's KV cache.

The compute path is libkvc.so (HIP for gfx950, C ABI in include/kvc.h);
``kvc`` is its thin ctypes binding, ``pipeline`` composes the calls,
``workload`` draws seeded synthetic inputs, ``build_lib`` builds the library.
Importing the package itself loads nothing; ``kvc`` loads the library and
raises if it is missing.
"""

__all__ = ["kvc", "pipeline", "workload", "build_lib"]
