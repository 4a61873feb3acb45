"""CPU float64 oracle for the owner-side Muon step (test infrastructure only).

Importable only from ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product package never imports it.
"""

from .ns_oracle import (  # noqa: F401
    CUBIC,
    MUON_QUINTIC,
    adamw_step,
    frobenius_normalize,
    gram_newton_schulz,
    momentum,
    muon_step,
    newton_schulz,
    orient,
    orthogonalize,
    update_scale,
)
