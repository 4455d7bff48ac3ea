"""CPU oracle for SageAttention-style quantized attention (forward).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (no kernels, headers, helpers or constant tables); both sides only draw
their inputs from ``workloads.py``, which holds none of the method's arithmetic.

Plain NumPy (plus a few plain PyTorch CPU dtype casts), fp64 wherever the
method does not fix the precision, slow and meant to be read against the pages:

* ``fp8_e4m3``   -- OCP OFP8 E4M3 ("e4m3fn") codec written from the format
                    definition (bias 7, 3 mantissa bits, max 448, saturating).
* ``sage_ref``   -- the method step by step: K channel mean, K smoothing,
                    per-block INT8 Q/K, INT32 QK^T, dequantisation, tiled
                    online softmax, P to FP8 (or FP16), V to FP8 per channel,
                    two-level PV accumulation, epilogue.
* ``mxfp4``      -- OCP MXFP4 codec (E2M1 elements, E8M0 shared scales per
                    32 elements) written from the Microscaling specification,
                    for the FP4 variant of the method.
* ``exact``      -- fp64 exact softmax attention (the error bound the method
                    is measured against) and an fp64 tiled online softmax
                    with quantisation switched off.

Every function cites the passage it follows. Readings taken where the pages
are silent are listed in the module docstrings and are labelled ``[R#]``.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/`` against facts other than itself (format definition, brute force,
closed forms, invariances, exact arithmetic). Conventions the pages leave open
(rounding tie rule, block sizes, KV tile size, P scale, row-sum source) are
choices, not pinned facts; the tests pin the arithmetic *given* the choice.
"""
