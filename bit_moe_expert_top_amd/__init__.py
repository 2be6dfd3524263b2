"""Low-bit routed-expert MoE FFN for AMD MI355X (gfx950).

The compute lives in ``libbitmoe.so`` (HIP kernels behind the C ABI of
``include/bitmoe.h``); ``bit_moe_expert_top_amd.ops`` is its thin ctypes binding.  Build
the library with ``python -m bit_moe_expert_top_amd.build``.  Importing this package does
not load the library; importing ``ops`` does, and fails loudly if it is not built.
"""


def __getattr__(name):
    if name == "ops":
        from . import _lib

        return _lib
    raise AttributeError(name)
