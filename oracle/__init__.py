"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP library and its
Python binding never do; they share no code with it.

``mla_ref``  -- vectorised NumPy float64 definition of every step.
``brute``    -- the same definition as scalar Python loops, for tiny shapes.
"""
