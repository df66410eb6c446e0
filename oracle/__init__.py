"""Plain CPU oracle of the gated delta rule (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this package: only the tests, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, constant
generator or helper with the HIP library and imports nothing from it.

Modules
  recurrence  token-by-token forward, its manual adjoint, and the decode step
              (the oracle proper).
  chunked     the chunk (WY / transition) forms of the same method, written
              from their own definitions; used only as independent pins of
              ``recurrence`` in the tests, never as the oracle.
"""
from .recurrence import (  # noqa: F401
    EPS,
    SOFTPLUS_THRESHOLD,
    l2norm,
    l2norm_backward,
    forward,
    backward,
    decode_gating,
    decode_step,
)
