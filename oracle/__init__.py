"""Float64 CPU oracle for the Gated DeltaNet layer prefill.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
are the only callers.  The product path never imports this package, and this package
imports nothing from the product package.

Two implementations of the same plain definition live here:

* ``gdn_oracle.c`` (built into ``liboracle.so``), a per-token float64 loop with threads over
  value heads, wrapped by :mod:`oracle.c_oracle`;
* :mod:`oracle.numpy_ref`, the same definition in numpy for tiny inputs.

Neither is trusted on its own: ``tests/test_oracle_pins.py`` pins both against closed forms,
brute-force matrix products, ``numpy.convolve`` and invariants of the recurrence.
"""
