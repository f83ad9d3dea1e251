"""fp64 CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path
and imports nothing from the product package.
"""
from .slikl_ref import slikl_grad_ref, kl_loss_ref, kl_per_unit_ref, unit_backward  # noqa: F401
from .metadata_ref import metadata_ref  # noqa: F401
from .attn_p_ref import attn_softmax_l1norm_ref, lse_over_slots_ref  # noqa: F401
from .dense_ref import dense_grad_ref, visible_keys  # noqa: F401
