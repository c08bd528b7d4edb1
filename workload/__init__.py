"""Seeded synthetic inputs shared by the CPU oracle and the HIP path (inputs only)."""
from .gen import CONFIGS, ROOT_SEED, Config, Workload, build_lib, small_config  # noqa: F401
