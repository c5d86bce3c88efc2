"""MoE expert operation of a speculative-decoding verify pass, native to MI355X (gfx950).

The compute lives in ``libmoe_verify.so`` (hand-written HIP, C ABI in
``include/moe_verify.h``).  ``_lib`` binds it with ctypes; ``layer`` holds
device buffers for one layer and chains the entry points of one verify pass.
Attribute access loads the library lazily, so ``build`` works before it
exists; any use of an entry point without the built library raises.
"""


import importlib


def __getattr__(name):
    if name.startswith("__") or name in ("_lib", "build", "layer"):
        raise AttributeError(name)
    return getattr(importlib.import_module(__name__ + "._lib"), name)
