"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle."""
from .workloads import CONFIGS, Node, Request, Shape, Workload, rng, round_bf16  # noqa: F401
