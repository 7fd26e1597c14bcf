"""CPU fp64 oracle for attention with a learnable per-head sink.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package. The product path (the HIP library and
its Python binding) never imports it and shares no code with it.
"""
from .sink_attention import (  # noqa: F401
    forward,
    backward,
    probabilities,
    forward_rows,
    dq_rows,
    dkdv_keys,
    dsink_heads,
    visible,
)
from .decode import decode_forward  # noqa: F401,E402
