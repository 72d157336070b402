"""CPU oracle (test infrastructure only; see ``tp_oracle``)."""
from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import (  # noqa: F401
    ACT_GELU, ACT_NONE, LAYOUT_LOCAL, LAYOUT_LOGICAL, OUT_BF16, OUT_F32, RMS_EPS, FP8_BLOCK,
)
