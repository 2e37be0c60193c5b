"""MI355X-native W4 mixture-of-experts layer.

The compute path lives in ``libmoe_w4.so`` (hand-written HIP for gfx950, built
from ``csrc/``) behind a C ABI declared in ``include/moe_w4.h``.  The Python
side is argument marshalling only:

* ``api``   -- torch-tensor wrappers over the C entry points (moe_route,
  moe_build_blocks, moe_w4_grouped_gemm, moe_ffn_forward).
* ``synth`` -- seeded synthetic inputs (no part of the layer's arithmetic).

Submodules are imported lazily so that ``synth`` can be used on a host
without the HIP library.
"""

__all__ = ["api", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
