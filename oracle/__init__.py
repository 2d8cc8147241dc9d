"""fp64 CPU oracle for exact attention.  TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it imports nothing from them.

Contents
--------
``attention``      the plain definition softmax(scale * Q K^T) V, two-pass, fp64
``online``         the tiled online-softmax recurrence, used only to pin ``attention``

``backward``       gradients dQ, dK, dV of the same definition (chain rule, fp64),
                   dense and variable-length

``attention.store_kvcache`` is the plain scatter of new K/V rows into the page pools.

Every function cites the passage of the source pages it follows.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    bf16_bits_to_f64,
    attention_rows,
    attention_dense,
    attention_varlen,
    attention_varlen_paged,
    attention_decode_paged,
    gather_paged,
    kv_head,
    probabilities,
    store_kvcache,
)
from .backward import attention_backward_dense, attention_backward_rows, attention_backward_varlen  # noqa: F401
from .online import online_attention  # noqa: F401
