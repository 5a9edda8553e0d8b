"""Seeded synthetic workloads for the CSA layer step: shapes (``configs``) and
input generators (``gen``).  Shared by the oracle tests, the GPU parity tests and
the benchmark; it holds none of the method's arithmetic."""
from .configs import CONFIGS, SHORT, PAGE, CsaConfig, get  # noqa: F401
from .gen import make_inputs, CsaInputs, rope_tables, quantize_rows_int8, f32_to_bf16_bits  # noqa: F401
