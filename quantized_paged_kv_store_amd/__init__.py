"""Quantized paged KV store and decode attention for MI355X (gfx950).

The compute path is libkvq.so (HIP kernels behind the C ABI in include/kvq.h);
``kvq`` is its ctypes binding and ``inputs`` the seeded synthetic input
generator shared by tests and the benchmark.
"""
from .kvq import (Cache, KVQError, kvq_alloc_pages, kvq_bytes_per_token, kvq_compute_scale,  # noqa: F401
                  kvq_compute_q_scale, kvq_decode, kvq_decode_append, kvq_decode_append_fp8q,
                  kvq_decode_fp8q, kvq_decode_noalloc, kvq_decode_workspace_bytes, kvq_dequantize_prev_kv,
                  kvq_extend_attention, kvq_profile_enable, kvq_profile_read, kvq_store, set_split_target,
                  split_target, library, make_desc)
