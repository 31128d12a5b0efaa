"""CPU oracle for the non-causal attention forward and its INT8-QK / FP8-PV variant.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library and does not import the product package.

Everything here is plain numpy in float64 unless a step fixes another
precision (the quantisation emulation works in the precisions the variant
defines).  Modules:

  rounding    fp32 -> bf16 / fp16 / fp8-e4m3fn from the format definitions
  attention   naive formula, blocked online softmax, two-pass softmax,
              sampled rows
  sage        exact emulation of the INT8-QK / FP8-PV variant
  accounting  FLOP and HBM-byte models printed on the handbook page

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, invariants or library routines.
"""
