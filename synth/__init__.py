"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws numbers and casts them to the storage dtype; it holds
none of attention's arithmetic, so both the oracle side and the HIP side may
use it.  See `synth.workloads` for the five workloads and `synth.gen` for the
recipe.
"""

from .workloads import WORKLOADS, Workload, by_name  # noqa: F401
from .gen import device_normal, make_dout, make_inputs, make_signs  # noqa: F401
