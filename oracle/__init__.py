"""CPU oracle for the LoRA-linear training step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the ``bwd_adamw_amd``
package and its HIP library) may import, call or link this package.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.

The oracle is the plain definition of each step, evaluated in float64 with
numpy (a matrix product is the only library primitive it leans on).  It shares
no code, constants or helpers with the HIP path.

Pinning status of each function (what fixes it other than itself) is listed in
the docstrings of ``oracle.lora`` and ``oracle.quant`` (block-quantized frozen
weights).
"""

from .lora import *  # noqa: F401,F403
