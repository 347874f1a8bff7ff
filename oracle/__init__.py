"""Plain, slow, obviously-correct fp64 CPU attention oracle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
GPU path (``exact_tiled_attention_14_amd``) never imports it and it imports
nothing from the GPU path: the two share no kernels, helpers, tables or
pre/post-processing.  Inputs come from ``workloads`` (seeded generators that do
no attention arithmetic) or from the tests themselves.

Every function here is pinned by a ``-m "not gpu"`` test in ``tests/`` against
something other than itself (closed forms, invariants, a library routine,
brute force over every block size); see ``tests/test_oracle_pins.py`` and
``tests/test_oracle_blockwise.py``; the backward pass against torch autograd,
finite differences and invariants in ``tests/test_oracle_backward.py``; the
packed-sequence form against brute force and invariants in
``tests/test_oracle_varlen.py``; the key-block partials and the S-way merge
against brute force, the full definition and invariants in
``tests/test_oracle_partial.py``; the fp8 pieces (``oracle/fp8.py``: e4m3
rounding, per-tensor quantisation, the Hadamard rotation of incoherent
processing) against the e4m3 bit layout decoded by hand, torch's e4m3 cast,
closed forms of the Hadamard matrix and the invariance of attention under the
rotation, with planted mistakes, in ``tests/test_oracle_fp8.py``.  No
function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    admissible,
    attention,
    attention_backward,
    attention_partial,
    attention_varlen,
    blockwise_attention,
    kv_head_of,
    merge_many,
    merge_partials,
    merge_softmax,
    scores,
    softmax_rows,
)
