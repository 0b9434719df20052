"""CPU oracle (float64) for the encoder block. Test infrastructure: the product path never imports it."""
from .oracle import *  # noqa: F401,F403
from .oracle import LN_EPS, KEY_TILE, QBLOCK, QUANT_MATRICES, MX_BLOCK, MX_MATRICES, E4M3_MAX  # noqa: F401
