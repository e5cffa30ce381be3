"""Seeded synthetic inputs shared by the oracle side and the GPU side of the tests.

Holds no arithmetic of the eviction method: layouts, counter-based random draws,
planted keys, k-means beacons and the upstream log-sum-exp only.
"""
from .configs import ALL, LLAMA8B, LLAMA70B, RAGGED, RATCHET, TINY, Workload  # noqa: F401
