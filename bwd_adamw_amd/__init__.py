"""MI355X-native LoRA-linear training hot path.

The compute runs in ``liblora.so`` (hand-written HIP for gfx950, C ABI in
``include/lora.h``).  ``bwd_adamw_amd.lora`` is the thin ctypes binding,
``bwd_adamw_amd.step`` sequences a whole optimizer step through it, and
``bwd_adamw_amd.workloads`` holds the workload shapes and seeded inputs.
Importing this package does not load the library; the first call does, and
fails loudly when it is missing.
"""

__all__ = ["lora", "step", "workloads"]
