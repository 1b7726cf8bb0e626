"""Double-precision CPU oracle of the QSA path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.
"""
