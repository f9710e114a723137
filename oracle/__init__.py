"""CPU oracle for the Muon optimizer step, and for the AdamW step it is
compared against (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The library itself never calls it, and it shares no code
with the HIP path.
"""
from .muon_oracle import (  # noqa: F401
    DEFAULT_COEFFS,
    DEFAULT_EPS,
    momentum_update,
    ns_source,
    orient_wide,
    frobenius_normalize,
    newton_schulz,
    newton_schulz_blockwise,
    newton_schulz_distributed,
    muon_step,
    newton_schulz_iteration_rows,
)
from .adamw_oracle import adamw_step  # noqa: F401,E402
