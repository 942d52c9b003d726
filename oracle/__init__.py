"""Float64 CPU oracle for block-sparse FP8/NVFP4 attention decode.

Test infrastructure: only tests, the smoke check and the benchmark's CPU-baseline
leg may import it. It shares no code with the HIP library.
"""
from .msa_oracle import *  # noqa: F401,F403
from .msa_oracle import (E4M3, E2M1, LOG2E, PAGE, GROUP, FMT_FP8, FMT_NVFP4,  # noqa: F401
                         f32, bf16_bits_to_f64)
