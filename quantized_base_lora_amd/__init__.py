"""MI355X-native LoRA linear layer over a frozen block-quantized base.

The compute lives in ``libqlora.so`` (HIP for gfx950, C ABI declared in
``include/qlora.h``); ``binding`` is a thin ctypes layer over it.  Nothing here
computes on the CPU: if the library is missing, loading fails loudly.
"""

__all__ = ["binding", "synth"]
