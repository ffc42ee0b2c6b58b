"""CPU oracle for row-wise top-k. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import anything from this package. It shares no code with the GPU path.

* ``oracle.topk``   -- full sort per row under (value desc, index asc), in C++.
* ``oracle.brute``  -- O(N^2) rank counting for tiny rows (pins the C++ sort).
* ``oracle.model``  -- instrumented CPU model of DeepSelect (invariants, work counts,
                       the expected-work bound).
"""
