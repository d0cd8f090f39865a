"""Seeded synthetic inputs shared by the oracle's tests and the HIP path.

Holds no arithmetic of the decode path itself: only counter-based random
numbers (host twin in ``synth.py``, device twin in ``synth.hip``) and
workload recipes (``workloads.py``)."""
