"""fp64 CPU oracle for the multi-pass TTT draft attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The GPU library never imports, links or
runs anything in this package, and this package imports nothing from the
library; the two share only the seeded input generator in `ttt_synth`.

Pins (tests/test_oracle.py): library softmax-attention brute force, the
two-part merge invariant, RoPE identities (relative shift, orthogonality,
complex-number form), closed forms (zero queries), fp64 autograd, central
finite differences, THD/BSHD equivalence and sequence isolation, GQA as
repeated K/V.  Every function here is pinned by at least one of them.
"""
from .ttt_oracle import *  # noqa: F401,F403
