"""CPU oracle for trellis-coded linear layers.  TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never does.
It shares no code with the HIP path: no kernels, headers, tables or helpers.

Everything is numpy: exact integers for bit work, float64 for arithmetic, and a
single IEEE binary16 rounding where the format stores fp16 values.
"""
from .trellis_oracle import *  # noqa: F401,F403
