"""Oracle for the layout-permuting tile copy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import, call or execute anything in this package.  The product library (the HIP kernels,
the host planner and the C-ABI) never does, and the two share no code: no kernels,
headers, helpers, tables or generators.  The only module both sides use is
``synth_inputs`` (seeded input generators, none of the method's arithmetic).

Contents: ``ref`` (Python: layout map, copy, TileLang loop partition, gmem<->smem
``[outer, threads, vec]`` partition, XOR-swizzle chooser, bank-conflict counting, LDS
tile-plan brute force) and ``copy_ref.c`` (C odometer copy, OpenMP), built by ``build``.

Parity pins: see the header of each function and the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py``.
"""
from . import ref  # noqa: F401
