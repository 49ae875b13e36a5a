"""Oracle: plain, slow CPU implementations of what the layer-streamed training path computes.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import anything under ``oracle/``. The product path (the HIP library and
its Python binding) never does, and the oracle imports nothing from the product.

* ``decoder``   - pre-norm decoder forward/backward, CE and sum-of-squares losses, MoE, LoRA,
                  micro-batch summation.
* ``adam``      - host fp32 Adam and the bf16 refresh of the low-precision copy.
* ``partition`` - the stage partition by exhaustive search (small L).
* ``async_opt`` - the staleness-1 asynchronous optimiser schedule (each call's gradient taken at the
                  parameters from before the previous call's update).

Every function is pinned by ``tests/test_oracle_*.py`` to something other than itself: finite
differences, library routines for special cases, closed forms, invariants and the worked
examples the pages print (``tests/golden/``).
"""
