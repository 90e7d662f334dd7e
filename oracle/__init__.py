"""CPU oracle for the MoE-LoRA expert layer (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP library never
calls it, and it shares no code with the HIP library.
"""
from .moe_lora_ref import *  # noqa: F401,F403
