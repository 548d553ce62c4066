"""Seeded synthetic inputs and workload shapes shared by tests, bench and the oracle.

Holds no step of the drafter pass: only shapes and random draws."""
from .configs import (DrafterConfig, Workload, WORKLOADS, TINY_FP32, QWEN3_8B_SHAPED,
                      LLAMA31_8B_SHAPED, SMALL_BF16)
from . import inputs
