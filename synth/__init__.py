"""Seeded synthetic inputs (boundary-format buffers) for tests and bench."""
from .workloads import *  # noqa: F401,F403
from .workloads import CONFIGS, layer_inputs, rotation, qweight, activations  # noqa: F401
