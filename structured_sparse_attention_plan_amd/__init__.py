"""CoWindow Attention (CoWA) on AMD Instinct MI355X (gfx950).

The product is libcowa.so (include/cowa.h): a block-visibility planner and HIP kernels
for the forward, backward and decode passes.  ``api`` is a thin marshalling layer over
its C ABI (``_cowa``); ``inputs`` draws the seeded synthetic tensors.  Importing ``api``
loads libcowa.so and raises ImportError if it has not been built.
"""

import importlib

__all__ = ["api", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
