"""Seeded synthetic inputs for sparse MLA decode over indexer top-k ids.

This package only draws and places data: query vectors, top-k id lists, paged
block tables and packed fp8_ds_mla cache records.  It holds no step of the
method itself (no index conversion, no dequantisation, no attention, no merge),
so that the oracle and the HIP path can both consume it without sharing any of
the method's arithmetic.
"""
from .gen import (  # noqa: F401
    BF16_RECORD_BYTES,
    CONFIGS,
    HEAD_DIM,
    LATENT_DIM,
    RECORD_BYTES,
    ROPE_DIM,
    SCALE_TILE,
    ShardCache,
    SparseCache,
    Workload,
    make_config,
    make_dense,
    make_random,
    pack_records,
    pack_records_bf16,
)
