"""CPU oracle for the bf16 allreduce share (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library's product path never does:
it shares no code with the oracle and must fail loudly, not fall back here,
when its HIP extension is missing.
"""
