"""CPU oracle (float64 numpy) for the shifted-window attention block forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` import it; the HIP library never does,
and this package imports nothing from the library.
"""
