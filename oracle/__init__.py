"""fp64 CPU oracle of the log-linear Mamba-2 forward and its gradients.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything here.  It shares
no code with the HIP path in ``ssm_scan_amd`` and imports nothing from it.

Pins (see tests/test_oracle_*.py): Fenwick bucket invariants and a hand
derived level table; closed forms for T = 1, 2 and a hand-worked T = 4
example; reduction to the SSD recurrence when lambda does not depend on the
level; reduction to the causal prefix sum (linear attention) when a = 1 and
lambda = 1; the token-by-token Fenwick recurrence; superposition over levels
and per-bucket brute force.  The gradients (loglin_grad) are pinned to the
forward by finite differences and by superposition over levels.  The
log-linear gated DeltaNet forward (gdn_ref) is pinned to the textbook gated
DeltaNet recurrence, a per-level Fenwick recurrence, the log-linear Mamba-2
oracle (orthonormal keys) and closed forms.  Conventions the pages cannot fix (group
mapping, lambda layout, dtypes) are "parity unpinned".
"""
from . import fenwick, gdn_ref, loglin_grad, loglin_ref, recurrent  # noqa: F401
from .loglin_grad import loglin_grad as loglin_backward  # noqa: F401
from .loglin_ref import loglin_forward, loglin_forward_bh, loglin_rows  # noqa: F401
from .recurrent import loglin_recurrent  # noqa: F401
