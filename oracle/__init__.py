"""Float64 CPU oracle for the Deja Vu decode layer.  TEST INFRASTRUCTURE: only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it."""
from .dejavu_oracle import *  # noqa: F401,F403
from .dejavu_oracle import (LN_EPS, THRESHOLD, TOPK, LayerWeights, PredictorWeights,  # noqa: F401
                            Selection)
