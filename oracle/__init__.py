"""CPU oracle for the FP4 lightning-indexer scorer -- test infrastructure only.

Only tests/, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import
this package.  The GPU library never does.
"""
