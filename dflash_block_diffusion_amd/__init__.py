"""MI355X-native DFlash draft+verify step.

The compute path is the C-ABI library ``_lib/libdflash.so`` (hand-written
HIP for gfx950, declared in ``include/dflash.h``); ``binding`` marshals
arguments to it and ``runtime`` builds device models and drives the loop.
PyTorch only provides device memory and streams.
"""
__all__ = ["configs", "synth", "binding", "runtime"]
