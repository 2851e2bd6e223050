"""fp64 CPU oracle for the SVDQuant W4A4 + low-rank linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the C-ABI library, its
kernels or its Python binding) imports, links or calls this package; only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, tables or constants with the GPU path.

The oracle is deliberately plain and slow: numpy, fp64 unless a step fixes a
narrower precision, one library primitive per step (matmul, SVD), no blocking
or fusion.  Each function cites the passage of the source pages it follows:

* "Zhou notes"      -- SVDQuant reading notes (Zhongzhu Zhou), sections 2-7,
                       Eqs. (1)-(13), Algorithms 1-2.
* "AutoRound doc"   -- AutoRound "SVDQuant (experimental)" documentation,
                       sections on processing flow, residual iteration,
                       smooth search and export.
* "msModelSlim doc" -- msModelSlim SVDQuant algorithm description (stages,
                       SVD decomposition process, forward equivalence).
* "MindStudio entry" -- MindStudio glossary entry "SVDQuant Quantization".

Parity status of every function is listed in the module headers; a function
without an independent pin says "parity unpinned" there.
"""

from . import rounding, quantizers, prepare, forward, accounting, search  # noqa: F401
