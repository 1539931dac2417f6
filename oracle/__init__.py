"""CPU fp64 oracle for attention forward/backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the GPU library.
"""
from .attention_ref import (  # noqa: F401
    LOG2E,
    attention_backward,
    attention_forward,
    delta_from_output,
    head_backward,
    head_forward,
    kv_head_of,
    visible_mask,
)
