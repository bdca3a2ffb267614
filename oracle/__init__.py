"""CPU oracle of the compressed-attention hot path (fp64 NumPy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  It shares no code with the GPU library
(``compressed_attention_csa_amd``) and neither imports the other; the seeded
input generator (``inputgen``) is the only module both sides use.

Modules
-------
formats  bf16 / e4m3fn rounding and decoding from the format definitions.
method   the method's steps (compress, visibility, indexer score, top-k,
         attention with window, HCA, split merge), vectorised NumPy.
brute    the same steps as pure-Python loops for tiny inputs.

Parity status: every function here is pinned by a test in
``tests/test_oracle_*.py`` against closed forms, library special cases or the
brute-force loops.  Fidelity to the real model's learned indexer/compressor
weights is parity unpinned: the pages print no formula or weights for them.
"""
from . import formats, method, brute  # noqa: F401
