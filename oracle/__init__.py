"""CPU oracle for blockwise absmax k-bit codebook quantization.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the method computes, written in numpy float32 with every
rounding step explicit.  It exists so that the HIP path can be checked against
something that shares no code with it.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The product (``blockwise_bit_codebook_amd``) never imports, calls or links
anything in here.

Sources (web pages, cited by title and section):

* [QLORA-2] bitsandbytes "compare main...QLORA-2" patch series, PATCH 001
  "Add k-bit quantization kernels (K=2-5, blocksize=32)" -- file
  ``tests/test_kbit_quantization.py`` (functions ``create_normal_float_codebook``,
  ``quantize_kbit_ref``, ``dequantize_kbit_ref``, ``pack_kbit_ref``,
  ``unpack_kbit_ref``) and ``csrc/kernels.cu`` (``kQuantizeBlockwise_kbit``,
  ``kDequantizeBlockwise_kbit``); PATCH 003 (Python API, stage 6 tests).
* [PR2051] bitsandbytes pull request 2051 "Fuse nested 4-bit scale
  reconstruction on SM103" -- sections Summary and Implementation.
* [ORBIT] orbitquant 0.2.2 -> 0.3.0 package diff -- README (W4A4 fast path),
  docs methodology audit (epsilon guard, Lloyd-Max codebook version 2,
  activation_eps, largest power-of-two Hadamard block).

Floating point: every array operation is on ``np.float32`` operands, so numpy
rounds each operation once to binary32 (round to nearest even).  numpy never
fuses a multiply and an add.  Subnormals are kept (checked at import).

Parity status per function is stated in each module header; the pins live in
``tests/test_oracle_*.py``.
"""

import numpy as _np

# Flush-to-zero on the host would silently change subnormal results.
assert _np.float32(1e-45) > 0, "host FPU flushes subnormals; oracle invalid"

from . import numerics, codebooks, kbit, nested, act, e4m4, linear  # noqa: E402,F401
