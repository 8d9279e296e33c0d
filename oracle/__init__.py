"""CPU oracle of the MoE layer hot path -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  It shares
no code with the HIP path (``routing_dispatch_expert_gate_amd``) and imports
nothing from it; the only module both sides use is the seeded input generator
``moe_synth``, which holds no arithmetic of the method.

See ``oracle.moe_oracle`` for the definitions and their sources.
"""
from .moe_oracle import *  # noqa: F401,F403
