"""CPU oracle for the Echo error-compensated int4 all-reduce.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP library (no kernels, headers, helpers, constants or
pre/post-processing) and imports nothing from ``error_compensated_bit_echo_amd``.

Two independent implementations live here:

* :mod:`oracle.echo_oracle` -- plain numpy, one IEEE binary32 operation per
  step of the method, in the order the method states them.
* :mod:`oracle.exact` -- pure-Python ``fractions`` arithmetic that rounds to
  binary32 by hand after every operation and picks quantization codes by brute
  force.  It is slow and is used on tiny tensors to pin the numpy oracle.

Sources followed (the method is described in prose only; no code, formulas or
tables are printed):

* rit.work blog post "echo-4-bit-gpu-communication" (Russian), sections
  «Почему обычное 4-битное суммирование портит модель» and
  «Как Echo возвращает ошибку в следующие вызовы».
* heraldofai.com article «Come Echo permette ai modelli AI di grandi dimensioni
  di allenarsi più velocemente usando dati ultra-leggeri a 4 bit», sections
  «Il problema della larghezza di banda nei modelli AI giganti» and
  «Come Echo evita che gli errori si accumulino».

Every function is pinned by a CPU test (brute force, closed forms, special
cases or invariants); none is "parity unpinned".
"""
