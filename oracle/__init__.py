"""Plain fp64 CPU oracle for sparse MLA decode over top-k ids.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (the HIP library and its Python binding) never imports it and
shares no code, header, table or helper with it.
"""
from .smla_oracle import (  # noqa: F401
    attention_rows,
    bf16_encode,
    bf16_to_f64,
    cache_write,
    convert_index,
    dcp_local_seq_lens,
    dense_decode,
    decode_records,
    decode_records_bf16,
    e4m3fn_encode,
    e4m3fn_to_f64,
    flatten_bhs_lse,
    merge_lse,
    quantize_records,
    sparse_mla_decode,
    sparse_mla_decode_bf16,
    transpose_hT_lse,
)
