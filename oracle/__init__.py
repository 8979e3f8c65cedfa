"""CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy implementations of what the lbq hot path
computes (group-wise MinMax INT4/INT2, NF4 with double quantization, packing,
dequantization, and the fp64-accumulated forward / input-gradient / LoRA
matmuls).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library under
``group_wise_minmax_amd`` never does, and the two share no code.
"""
from .lbq_oracle import *  # noqa: F401,F403
from . import lbq_oracle  # noqa: F401
