"""CPU oracle for the causal attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import, call, link or execute anything
in this package.  It shares no code with the GPU library
(``tiled_online_softmax_causal_amd``) and neither imports the other; the only
module both sides use is ``workloads`` (seeded input generators).

Contents
--------
``dense``   fp64 dense attention in plain C (``attention_dense.c``), the
            definition the dense reference of the aiml.sh page "Speed up long
            contexts with FlashAttention" (lab.py, standard_attention) writes
            out, with a log-sum-exp added.  Pinned by ``tests/test_oracle_*``
            against 40-digit brute force, the page's printed outputs, closed
            forms and invariants.
``tiled``   the method itself -- Q row blocks, streamed K/V blocks, online
            softmax with a running max, running sum and rescaled accumulator --
            as a plain fp64 numpy loop in the order lab.py's
            tiled_flash_attention takes its steps.  Pinned against ``dense``
            (agreement near 1e-16, as the page's equivalence check reports), the
            page's counters (tiles visited) and block-size invariance.
``backward`` fp64 gradients (dQ, dK, dV) of that forward for an upstream dO,
            the chain rule in plain numpy; not on the pages.  Pinned by
            ``tests/test_oracle_backward.py`` against central finite
            differences of ``dense``, invariants and closed forms.
"""
from .dense import attention_dense, build_library, library_path  # noqa: F401
from .tiled import tiled_attention  # noqa: F401
from .backward import attention_backward, row_deltas  # noqa: F401
