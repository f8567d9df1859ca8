"""CPU oracle of the APB per-host path: test infrastructure only.

Imported only by the tests, the package entry's smoke check and the benchmark's
CPU-baseline leg.  See apb_oracle.py for the steps and their sources.
"""
from .apb_oracle import (SEGMENTS_ALL, block_attention, build_passing, compress_host, gather,
                         group_of, merge_attention, qkv_projection, rope, score_kv, topl, topl_one)

__all__ = ["SEGMENTS_ALL", "block_attention", "build_passing", "compress_host", "gather",
           "group_of", "merge_attention", "qkv_projection", "rope", "score_kv", "topl",
           "topl_one"]
