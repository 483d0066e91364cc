"""CPU oracle for the attention forward and its gradients: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .sdpa import sdpa_fwd, sdpa_fwd_rows, sdpa_fwd_varlen, attention_weights  # noqa: F401
from .grad import (sdpa_bwd, attention_grads, attention_grads_dropout, sdpa_bwd_dropout,  # noqa: F401
                   attention_grads_biased, sdpa_bwd_masked, attention_grads_masked_dropout,
                   sdpa_bwd_masked_dropout)
from .block_sparse import sdpa_fwd_block_sparse  # noqa: F401
from .dropout import sdpa_fwd_dropout, sdpa_fwd_dropout_varlen, sdpa_fwd_masked_dropout  # noqa: F401
from .masked import sdpa_fwd_masked  # noqa: F401
