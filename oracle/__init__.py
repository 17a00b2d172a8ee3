"""CPU oracle for the exact integer matrix product computed in residues.

This package is TEST INFRASTRUCTURE.  Only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import,
call, link or execute anything in it.  The product path (the HIP library and
its Python binding) never touches it, and it shares no code, table or constant
generator with the product path.

Contents
--------
``oracle.py``       plain Python-int definitions: the primes below 256, the
                    prime-count rule, two's-complement limbs, balanced
                    residues, textbook CRT, the integer product by triple loop,
                    and step-by-step stage definitions of the residue method.
``oracle_gemm.c``   a plain C schoolbook multi-limb integer GEMM (OpenMP over
                    rows), for operand sizes the Python loops cannot finish.
``cgemm.py``        ctypes loader and builder for ``oracle_gemm.c``.

Every function cites the passage of the pages it follows.  Pins against values
fixed by the pages and by mathematics live in ``tests/test_oracle*.py``.
"""
