"""Seeded synthetic inputs for the ZHA decode path.

This module is shared by the fp64 oracle side and the HIP side of the tests and
the benchmark.  It holds no arithmetic of the method itself: it only draws
keys, values, queries, reference queries and planted needles, and rounds them
to the storage dtype.  Everything it returns is a plain numpy array.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Config,
    bf16_round,
    bf16_to_f32,
    f32_to_bf16_bits,
    get_config,
    needles,
    queries,
    refs,
    scales,
    append_rows,
    unit_kv,
)
