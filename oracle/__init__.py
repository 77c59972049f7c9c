"""Float64 CPU oracle for GPTQ layer quantization (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP product path never does."""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import NotSPD, GridSpec, SweepResult, LayerResult  # noqa: F401
from . import w4a16_oracle  # noqa: F401
from . import calibration_oracle  # noqa: F401
