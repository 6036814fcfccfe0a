"""Sparse MLA decode over indexer top-k ids against a packed fp8_ds_mla cache, MI355X.

The compute lives in libsmla.so (hand-written HIP for gfx950, C ABI in include/smla.h);
this package is a thin ctypes binding with the same call names that marshals torch
tensors (device memory and streams only) into the C calls.
"""
from ._binding import (  # noqa: F401
    HEAD_DIM,
    LATENT_DIM,
    RECORD_BYTES,
    SmlaError,
    abi_version,
    cache_write,
    convert_index,
    dcp_local_seq_lens,
    decode,
    decode_noalloc,
    decode_workspace_size,
    dense_decode,
    lib_path,
    load_library,
    merge_lse,
    sparse_mla_cache_write,
    sparse_mla_convert_index,
    sparse_mla_dcp_local_seq_lens,
    sparse_mla_decode,
    sparse_mla_decode_bf16,
    sparse_mla_decode_noalloc,
    sparse_mla_decode_workspace_size,
    sparse_mla_dense_decode,
    sparse_mla_dense_decode_workspace_size,
    sparse_mla_merge_lse,
    workspace_for,
)
