"""Shared helpers for the GPU tests: the tolerances, the device plumbing of
``kda_inputs.device`` and the oracle's parity metric."""
from kda_inputs.device import dev, device_inputs, to_dev  # noqa: F401
from oracle import rel_err  # noqa: F401

TOL = {"bf16": 2e-2, "f32": 1e-4}
