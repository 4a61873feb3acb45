"""CPU float64 oracles for the owner-side Muon and Shampoo steps (test infrastructure only).

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
from .shampoo_oracle import (  # noqa: F401
    accumulate,
    inverse_root_eigh,
    inverse_root_newton,
    root_scale,
    shampoo_step,
)
