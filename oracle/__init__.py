"""fp64 CPU oracle for attention and its FlashAttention-2 style backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under ``oracle/``.  The
product path (the HIP library and its Python binding) never imports it, and it never
imports the product path: the two share no code.

Every function is pinned by ``tests/test_oracle.py`` to something other than itself
(finite differences against a brute-force loop forward, closed forms, identities,
a PyTorch fp64 autograd cross-check, hand-worked golden values).  Nothing here is
"parity unpinned".
"""
from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    attention_grads,
    kv_head_of,
    allowed_mask,
    grads_for_groups,
)
