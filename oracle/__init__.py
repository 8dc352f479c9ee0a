"""fp64 CPU oracle of the Gated DeltaNet-2 token mixer.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The GPU library and its
Python binding never import it.
"""
from .reference import (recurrent, chunked_wy, rel_l2, prologue, sigmoid, gated_rmsnorm, share_qk_heads, varlen,  # noqa: F401
                        FLAG_GATE_LOGITS, FLAG_NEG_EIGVAL, FLAG_QK_L2NORM)
