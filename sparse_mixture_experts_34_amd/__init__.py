"""MI355X (gfx950) sparse mixture-of-experts layer forward pass.

``binding`` is the Python binding of the C ABI in ``include/moe.h`` (the
HIP library ``libmoe.so``); ``synth`` holds seeded synthetic workloads.
Names of the binding are reachable from the package, e.g.
``sparse_mixture_experts_34_amd.moe_layer_forward``; touching any of them
loads the library and fails loudly if it is not built.
"""


import importlib


def __getattr__(name):
    if name.startswith("__") or name in ("binding", "synth", "build"):
        return importlib.import_module(f"{__name__}.{name}") \
            if not name.startswith("__") else _missing(name)
    binding = importlib.import_module(f"{__name__}.binding")
    try:
        return getattr(binding, name)
    except AttributeError:
        raise AttributeError(
            f"module 'sparse_mixture_experts_34_amd' has no attribute "
            f"{name!r}") from None


def _missing(name):
    raise AttributeError(name)
