"""CPU oracle of the GPTQ layer quantizer.  Test infrastructure only: imported by
tests, by the entry point's smoke check and by the benchmark's CPU-baseline leg,
never by the product path."""
from .gptq_oracle import *  # noqa: F401,F403
