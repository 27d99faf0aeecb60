"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check.  Holds no arithmetic of the drafter itself."""
from .workloads import *  # noqa: F401,F403
from .workloads import WORKLOADS, Workload, custom, as_f64  # noqa: F401
