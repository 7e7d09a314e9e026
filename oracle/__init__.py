"""Float64 CPU oracle (test infrastructure only; see iskv_oracle.py)."""
from .iskv_oracle import (  # noqa: F401
    BLOCK, Factor, JointUnit, Oracle, Unit, bf16_round, brand_fold, drift, full_kv_bytes,
    persistent_kv_bytes, rope, rope_theta, store_round,
)
