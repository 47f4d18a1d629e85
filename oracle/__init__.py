"""CPU oracle for the Muon step -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never imports the product package.
"""

from .muon_ref import (  # noqa: F401
    DEFAULT_EPS,
    UPDATE_SCALES,
    decode,
    f32,
    frobenius_normalize,
    momentum_update,
    muon_step,
    newton_schulz,
    orient,
    orthogonalize,
    update_direction,
    update_scale,
)
