"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the
oracle.  Holds random generation and grid rounding only -- none of the
method's arithmetic (no scores, no selection, no softmax)."""
from .synth import CONFIGS, make_inputs, scattered_ids, sweep_cases  # noqa: F401
