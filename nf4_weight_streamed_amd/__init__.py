"""MI355X-native (gfx950) frozen-NF4-base LoRA linear with blockwise weight streaming.

The compute path is the HIP library libnf4lora.so behind the C ABI in
include/nf4lora.h; ``nf4_weight_streamed_amd.lib`` is its ctypes binding and
``nf4_weight_streamed_amd.stack`` drives a stack of layers through it (resident
or streamed). Importing the package itself loads nothing; importing ``lib``
loads the library and fails loudly if it is not built.
"""

__all__ = ["lib", "stack", "build"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
