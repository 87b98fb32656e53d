"""CPU oracle (test infrastructure only): see ``oracle.nvfp4_ref``.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.
"""
