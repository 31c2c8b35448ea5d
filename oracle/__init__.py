"""Oracle: test infrastructure only (see hybrid_layer.py)."""
from .hybrid_layer import *  # noqa: F401,F403
