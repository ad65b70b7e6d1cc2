"""Dense and sparse MLA decode (weight-absorbed, paged, split-KV) for AMD MI355X (gfx950).

The compute path lives in the HIP library ``libmla_decode.so`` (C ABI in
``include/mla_decode.h``); this package binds it with ctypes.
"""
from .binding import (EXPORTED, MlaError, attach_pages, get_mla_metadata, get_mla_metadata_device, get_mla_metadata_host, lib,  # noqa: F401,E501
                      get_mla_metadata_sparse, get_mla_metadata_sparse_host, mla_decode_fwd, mla_decode_fwd_noalloc,
                      mla_decode_sparse_fwd,
                      mla_plan, mla_workspace_bytes, profile_start, profile_stop)
