"""Seeded synthetic workloads (shapes, layouts, input draws) shared by the
HIP path's tests and benchmark and by the CPU oracle's tests."""
from .configs import Workload, CONFIGS, BENCH, get  # noqa: F401
from .generate import Batch, make_batch, make_scores, to_numpy, quantize_e4m3, quantize_mx  # noqa: F401
from .shards import context_shards  # noqa: F401
