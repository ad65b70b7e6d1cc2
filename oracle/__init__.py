"""CPU oracle for dense and sparse MLA decode and its split planner.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this package.  The GPU library
and its Python binding never use it.
"""
from .mla_oracle import (attend, bf16_to_f64, dequantize_fp8_cache, e4m3_value, merge_partials,  # noqa: F401
                         mla_decode, mla_decode_rows, mla_decode_sparse, mla_decode_sparse_rows, online_attend,
                         request_keys, rescale_factor, sparse_keys, split_then_merge)
from .planner import plan, pieces_of  # noqa: F401
