"""ctypes binding of libsmla.so: argument marshalling only.

Every function here checks dtypes, devices and layouts of torch tensors, passes raw
device pointers, strides and the current HIP stream to the C call of the same name, and
raises SmlaError on a non-zero status.  All arithmetic happens in the HIP kernels; there
is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

LATENT_DIM = 512
ROPE_DIM = 64
HEAD_DIM = LATENT_DIM + ROPE_DIM
RECORD_BYTES = 656

_BF16, _FP32 = 0, 1
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_lock = threading.Lock()
_lib = None


class SmlaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: status {status}: {text}")
        self.status = status


def lib_path() -> str:
    return os.environ.get("SMLA_LIB", os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsmla.so"))


def load_library():
    """Load libsmla.so once and declare the C signatures (include/smla.h)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(path)
        lib.smla_abi_version.restype = ctypes.c_int
        lib.smla_abi_version.argtypes = []
        lib.smla_status_string.restype = ctypes.c_char_p
        lib.smla_status_string.argtypes = [ctypes.c_int]
        lib.sparse_mla_convert_index.restype = ctypes.c_int
        lib.sparse_mla_convert_index.argtypes = [_P, _I64, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                 _P, _I64, _P, _P]
        lib.sparse_mla_decode_workspace_size.restype = _SZ
        lib.sparse_mla_decode_workspace_size.argtypes = [_I32, _I32, _I32, _I32]
        lib.sparse_mla_decode.restype = ctypes.c_int
        lib.sparse_mla_decode.argtypes = [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _I32, _I32, _I32, _F32, _P, _I32,
                                          _I64, _I64, _P, _I64, _I64, _I32, _P, _SZ, _P]
        lib.sparse_mla_decode_bf16.restype = ctypes.c_int
        lib.sparse_mla_decode_bf16.argtypes = lib.sparse_mla_decode.argtypes
        lib.sparse_mla_decode_noalloc.restype = ctypes.c_int
        lib.sparse_mla_decode_noalloc.argtypes = [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _I32, _I32, _I32, _F32, _P,
                                                  _I32, _I64, _I64, _P, _I64, _I64, _I32, _P]
        lib.sparse_mla_merge_lse.restype = ctypes.c_int
        lib.sparse_mla_merge_lse.argtypes = [_P, _I32, _I64, _I64, _I64, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _I32,
                                             _I64, _I64, _P, _I64, _I64, _P]
        lib.sparse_mla_dense_decode_workspace_size.restype = _SZ
        lib.sparse_mla_dense_decode_workspace_size.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32]
        lib.sparse_mla_dense_decode.restype = ctypes.c_int
        lib.sparse_mla_dense_decode.argtypes = [_P, _I64, _I64, _P, _I64, _P, _I64, _I32, _I32, _P, _I32, _I32, _I32,
                                                _I32, _I32, _I32, _I32, _I32, _F32, _P, _I32, _I64, _I64, _P, _I64,
                                                _I64, _P, _SZ, _P]
        lib.sparse_mla_cache_write.restype = ctypes.c_int
        lib.sparse_mla_cache_write.argtypes = [_P, _I64, _P, _I64, _I32, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32,
                                               _I32, _I32, _P, _I64, _P, _P]
        lib.sparse_mla_dcp_local_seq_lens.restype = ctypes.c_int
        lib.sparse_mla_dcp_local_seq_lens.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P]
        _lib = lib
        return lib


def abi_version() -> int:
    return load_library().smla_abi_version()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SmlaError(fn, status, load_library().smla_status_string(status).decode())


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")


def _st(t: torch.Tensor, d: int) -> int:
    """Stride of dim d in elements.  A dim of size 1 may carry any stride in torch (0 included);
    the C calls validate strides, so such a dim reports the stride a contiguous tensor would
    have there (its value is never used to address memory)."""
    if t.shape[d] > 1:
        return t.stride(d)
    n = 1
    for k in range(d + 1, t.dim()):
        n *= t.shape[k]
    return n


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return _BF16
    if dtype == torch.float32:
        return _FP32
    raise TypeError(f"unsupported dtype {dtype}: bfloat16 or float32")


# ------------------------------------------------------------------ raw C-named calls

def sparse_mla_convert_index(*args) -> int:
    return load_library().sparse_mla_convert_index(*args)


def sparse_mla_decode_workspace_size(T: int, H: int, K: int, num_splits: int = 0) -> int:
    return int(load_library().sparse_mla_decode_workspace_size(T, H, K, num_splits))


def sparse_mla_decode(*args) -> int:
    return load_library().sparse_mla_decode(*args)


def sparse_mla_decode_bf16(*args) -> int:
    return load_library().sparse_mla_decode_bf16(*args)


def sparse_mla_decode_noalloc(*args) -> int:
    return load_library().sparse_mla_decode_noalloc(*args)


def sparse_mla_merge_lse(*args) -> int:
    return load_library().sparse_mla_merge_lse(*args)


def sparse_mla_dense_decode_workspace_size(B: int, S: int, H: int, max_seq_len: int, dcp_size: int = 1,
                                           interleave: int = 1) -> int:
    return int(load_library().sparse_mla_dense_decode_workspace_size(B, S, H, max_seq_len, dcp_size, interleave))


def sparse_mla_dense_decode(*args) -> int:
    return load_library().sparse_mla_dense_decode(*args)


def sparse_mla_cache_write(*args) -> int:
    return load_library().sparse_mla_cache_write(*args)


def sparse_mla_dcp_local_seq_lens(*args) -> int:
    return load_library().sparse_mla_dcp_local_seq_lens(*args)


decode_workspace_size = sparse_mla_decode_workspace_size

# ------------------------------------------------------------------ tensor-level calls

_ws_cache = {}


def workspace_for(T: int, H: int, K: int, device, num_splits: int = 0) -> Optional[torch.Tensor]:
    """A workspace at least as large as the call needs, cached per (device, stream) and grown outside
    the hot path (the library itself never allocates).  Calls on one stream are ordered, so they may
    share a workspace; a call on another stream gets its own, and a replaced buffer is released on the
    stream that used it (the caching allocator orders its reuse after that stream's work)."""
    need = sparse_mla_decode_workspace_size(T, H, K, num_splits)
    if need == 0:
        return None
    device = torch.device(device)
    index = device.index if device.index is not None else torch.cuda.current_device()
    stream = torch.cuda.current_stream(index)
    key = (index, stream.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=torch.device("cuda", index))
        _ws_cache[key] = ws
    return ws


def convert_index(topk_ids: torch.Tensor, req_id_per_token: torch.Tensor, block_table: torch.Tensor,
                  block_size: int, dcp_size: int = 1, dcp_rank: int = 0, interleave: int = 1,
                  out: Optional[torch.Tensor] = None, with_valid_count: bool = True,
                  valid: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Global top-k ids [T,K] -> slots [T,K] (and per-row valid counts [T], written into ``valid``
    when given)."""
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(req_id_per_token, "req_id_per_token", torch.int32, 1)
    _need(block_table, "block_table", torch.int32, 2)
    T, K = topk_ids.shape
    if (K > 1 and topk_ids.stride(1) != 1) or (block_table.shape[1] > 1 and block_table.stride(1) != 1) or \
            (req_id_per_token.shape[0] > 1 and req_id_per_token.stride(0) != 1):
        raise ValueError("index arrays need a contiguous last dimension")
    if req_id_per_token.shape[0] < T:
        raise ValueError("req_id_per_token must cover every top-k row")
    if out is None:
        out = torch.empty((T, K), dtype=torch.int32, device=topk_ids.device)
    _need(out, "out", torch.int32, 2)
    if tuple(out.shape) != (T, K) or (K > 1 and out.stride(1) != 1):
        raise ValueError("out must be [T,K] with a contiguous last dimension")
    if valid is not None:
        _need(valid, "valid", torch.int32, 1)
        if valid.shape[0] != T or (T > 1 and valid.stride(0) != 1):
            raise ValueError("valid must be a contiguous [T] int32 tensor")
    elif with_valid_count:
        valid = torch.empty((T,), dtype=torch.int32, device=topk_ids.device)
    R, W = block_table.shape
    st = sparse_mla_convert_index(
        topk_ids.data_ptr(), _st(topk_ids, 0), req_id_per_token.data_ptr(), block_table.data_ptr(),
        _st(block_table, 0), R, W, T, K, block_size, dcp_size, dcp_rank, interleave, out.data_ptr(), _st(out, 0),
        valid.data_ptr() if valid is not None else None, _stream(topk_ids.device))
    _check("sparse_mla_convert_index", st)
    return out, valid


KV_LAYOUTS = {"fp8_ds_mla": RECORD_BYTES, "bf16": 2 * HEAD_DIM}


def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, slots: torch.Tensor, softmax_scale: float,
                   out: torch.Tensor, lse: torch.Tensor, num_splits: int = 0,
                   valid_count: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """sparse_mla_decode_noalloc: the fp8_ds_mla decode with the library's per-device scratch array
    as workspace.  The caller passes out [T,H,512] (bf16 or fp32) and lse viewable as [T,H]; nothing
    is allocated here or in the library.  Calls on one device must not overlap."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_cache, "kv_cache", torch.uint8, 2)
    _need(slots, "slots", torch.int32, 2)
    T, H, D = q.shape
    if D != HEAD_DIM or q.stride(2) != 1:
        raise ValueError("q must be [T,H,576] with contiguous dims")
    if kv_cache.shape[1] != RECORD_BYTES or not kv_cache.is_contiguous():
        raise ValueError(f"kv_cache must be a contiguous [num_slots,{RECORD_BYTES}] uint8 tensor")
    K = slots.shape[1]
    if slots.shape[0] != T or (K > 1 and slots.stride(1) != 1):
        raise ValueError("slots must be [T,K] with a contiguous last dimension")
    if valid_count is not None:
        _need(valid_count, "valid_count", torch.int32, 1)
        if valid_count.shape[0] != T or (T > 1 and valid_count.stride(0) != 1):
            raise ValueError("valid_count must be a contiguous [T] int32 tensor")
    _need(out, "out", out.dtype, 3)
    if tuple(out.shape) != (T, H, LATENT_DIM) or out.stride(2) != 1:
        raise ValueError("out must be [T,H,512] with contiguous dims")
    _need(lse, "lse", torch.float32, 2)
    if tuple(lse.shape) != (T, H):
        raise ValueError("lse must be viewable as [T,H]")
    st = sparse_mla_decode_noalloc(
        q.data_ptr(), _st(q, 0), _st(q, 1), kv_cache.data_ptr(), kv_cache.shape[0], slots.data_ptr(),
        _st(slots, 0), valid_count.data_ptr() if valid_count is not None else None, T, H, K, float(softmax_scale),
        out.data_ptr(), _dtype_code(out.dtype), _st(out, 0), _st(out, 1), lse.data_ptr(), _st(lse, 0), _st(lse, 1),
        num_splits, _stream(q.device))
    _check("sparse_mla_decode_noalloc", st)
    return out, lse


def decode(q: torch.Tensor, kv_cache: torch.Tensor, slots: torch.Tensor, softmax_scale: float,
           out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
           lse: Optional[torch.Tensor] = None, lse_layout: str = "TH", num_splits: int = 0,
           workspace: Optional[torch.Tensor] = None, kv_layout: str = "fp8_ds_mla",
           valid_count: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sparse MLA decode.  q [T,H,576] bf16, kv_cache [num_slots,656] uint8 (kv_layout "fp8_ds_mla")
    or [num_slots,1152] (kv_layout "bf16": 576 bf16 values per token), slots [T,K] int32,
    valid_count [T] int32 or None (the conversion's per-row counts: a row counted <= 0 is empty).

    Returns out [T,H,512] (out_dtype) and lse.  lse_layout "TH" gives a [T,H] tensor;
    "HT" writes the kernel-native [H,T] layout and returns its [T,H] transposed view.
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_cache, "kv_cache", torch.uint8, 2)
    _need(slots, "slots", torch.int32, 2)
    T, H, D = q.shape
    if D != HEAD_DIM or q.stride(2) != 1:
        raise ValueError("q must be [T,H,576] with contiguous dims")
    if kv_layout not in KV_LAYOUTS:
        raise ValueError(f"kv_layout must be one of {sorted(KV_LAYOUTS)}")
    rb = KV_LAYOUTS[kv_layout]
    if kv_cache.shape[1] != rb or not kv_cache.is_contiguous():
        raise ValueError(f"kv_cache must be a contiguous [num_slots,{rb}] uint8 tensor")
    K = slots.shape[1]
    if slots.shape[0] != T or (K > 1 and slots.stride(1) != 1):
        raise ValueError("slots must be [T,K] with a contiguous last dimension")
    dev = q.device
    if valid_count is not None:
        _need(valid_count, "valid_count", torch.int32, 1)
        if valid_count.shape[0] != T or (T > 1 and valid_count.stride(0) != 1):
            raise ValueError("valid_count must be a contiguous [T] int32 tensor")
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=out_dtype, device=dev)
    _need(out, "out", out.dtype, 3)
    if tuple(out.shape) != (T, H, LATENT_DIM) or out.stride(2) != 1:
        raise ValueError("out must be [T,H,512] with contiguous dims")
    if lse is None:
        if lse_layout == "TH":
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        elif lse_layout == "HT":
            lse = torch.empty((H, T), dtype=torch.float32, device=dev).t()
        else:
            raise ValueError("lse_layout must be 'TH' or 'HT'")
    _need(lse, "lse", torch.float32, 2)
    if tuple(lse.shape) != (T, H):
        raise ValueError("lse must be viewable as [T,H]")
    if workspace is None:
        workspace = workspace_for(T, H, K, dev, num_splits)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if workspace is not None \
        else (None, 0)
    if ws_ptr is not None and ws_ptr % 256:
        pad = (-ws_ptr) % 256
        ws_ptr, ws_bytes = ws_ptr + pad, ws_bytes - pad
    call = sparse_mla_decode if kv_layout == "fp8_ds_mla" else sparse_mla_decode_bf16
    st = call(
        q.data_ptr(), _st(q, 0), _st(q, 1), kv_cache.data_ptr(), kv_cache.shape[0], slots.data_ptr(),
        _st(slots, 0), valid_count.data_ptr() if valid_count is not None else None, T, H, K, float(softmax_scale),
        out.data_ptr(), _dtype_code(out.dtype), _st(out, 0),
        _st(out, 1), lse.data_ptr(), _st(lse, 0), _st(lse, 1), num_splits, ws_ptr, ws_bytes, _stream(dev))
    _check(call.__name__, st)
    return out, lse


def merge_lse(out_parts: torch.Tensor, lse_parts: torch.Tensor, out: Optional[torch.Tensor] = None,
              out_dtype: Optional[torch.dtype] = None, lse: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge S partials: out_parts [S,T,H,512], lse_parts [S,T,H] (any strides)."""
    _need(out_parts, "out_parts", out_parts.dtype, 4)
    _need(lse_parts, "lse_parts", torch.float32, 3)
    S, T, H, D = out_parts.shape
    if D != LATENT_DIM or out_parts.stride(3) != 1:
        raise ValueError("out_parts must be [S,T,H,512] with contiguous dims")
    if tuple(lse_parts.shape) != (S, T, H):
        raise ValueError("lse_parts must be [S,T,H]")
    dev = out_parts.device
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=out_dtype or out_parts.dtype, device=dev)
    if tuple(out.shape) != (T, H, LATENT_DIM) or out.stride(2) != 1:
        raise ValueError("out must be [T,H,512] with contiguous dims")
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(lse, "lse", torch.float32, 2)
    st = sparse_mla_merge_lse(
        out_parts.data_ptr(), _dtype_code(out_parts.dtype), _st(out_parts, 0), _st(out_parts, 1),
        _st(out_parts, 2), lse_parts.data_ptr(), _st(lse_parts, 0), _st(lse_parts, 1), _st(lse_parts, 2),
        S, T, H, out.data_ptr(), _dtype_code(out.dtype), _st(out, 0), _st(out, 1), lse.data_ptr(), _st(lse, 0),
        _st(lse, 1), _stream(dev))
    _check("sparse_mla_merge_lse", st)
    return out, lse


def cache_write(latent: torch.Tensor, rope: torch.Tensor, positions: torch.Tensor, req_id: torch.Tensor,
                block_table: torch.Tensor, kv_cache: torch.Tensor, block_size: int, dcp_size: int = 1,
                dcp_rank: int = 0, interleave: int = 1, slot_mapping: Optional[torch.Tensor] = None,
                with_slot_mapping: bool = True) -> Optional[torch.Tensor]:
    """Quantise tokens latent [N,512] / rope [N,64] (bf16 or fp32) into kv_cache [num_slots,656]
    at the slots this DCP rank owns; returns slot_mapping [N] (-1 = not written here)."""
    _need(latent, "latent", latent.dtype, 2)
    _need(rope, "rope", latent.dtype, 2)
    _need(positions, "positions", torch.int32, 1)
    _need(req_id, "req_id", torch.int32, 1)
    _need(block_table, "block_table", torch.int32, 2)
    _need(kv_cache, "kv_cache", torch.uint8, 2)
    N = latent.shape[0]
    if latent.shape[1] != LATENT_DIM or latent.stride(1) != 1 or tuple(rope.shape) != (N, ROPE_DIM) or \
            rope.stride(1) != 1:
        raise ValueError("latent must be [N,512] and rope [N,64], both with contiguous dims")
    if positions.shape[0] != N or req_id.shape[0] != N or (N > 1 and (positions.stride(0) != 1 or
                                                                      req_id.stride(0) != 1)):
        raise ValueError("positions and req_id must be contiguous [N]")
    if kv_cache.shape[1] != RECORD_BYTES or not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be a contiguous [num_slots,656] uint8 tensor")
    if block_table.shape[1] > 1 and block_table.stride(1) != 1:
        raise ValueError("block_table needs a contiguous last dimension")
    if slot_mapping is None and with_slot_mapping:
        slot_mapping = torch.empty((N,), dtype=torch.int32, device=latent.device)
    if slot_mapping is not None:
        _need(slot_mapping, "slot_mapping", torch.int32, 1)
        if slot_mapping.shape[0] != N or (N > 1 and slot_mapping.stride(0) != 1):
            raise ValueError("slot_mapping must be contiguous [N]")
    R, W = block_table.shape
    st = sparse_mla_cache_write(
        latent.data_ptr(), _st(latent, 0), rope.data_ptr(), _st(rope, 0), _dtype_code(latent.dtype),
        positions.data_ptr(), req_id.data_ptr(), block_table.data_ptr(), _st(block_table, 0), R, W, N, block_size,
        dcp_size, dcp_rank, interleave, kv_cache.data_ptr(), kv_cache.shape[0],
        slot_mapping.data_ptr() if slot_mapping is not None else None, _stream(latent.device))
    _check("sparse_mla_cache_write", st)
    return slot_mapping


def dcp_local_seq_lens(seq_lens: torch.Tensor, dcp_size: int, dcp_rank: int, interleave: int = 1,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Positions below each request's length that DCP rank ``dcp_rank`` owns, [R] int32."""
    _need(seq_lens, "seq_lens", torch.int32, 1)
    R = seq_lens.shape[0]
    if R > 1 and seq_lens.stride(0) != 1:
        raise ValueError("seq_lens must be contiguous")
    if out is None:
        out = torch.empty((R,), dtype=torch.int32, device=seq_lens.device)
    _need(out, "out", torch.int32, 1)
    if out.shape[0] != R or (R > 1 and out.stride(0) != 1):
        raise ValueError("out must be contiguous [R]")
    st = sparse_mla_dcp_local_seq_lens(seq_lens.data_ptr(), R, dcp_size, dcp_rank, interleave, out.data_ptr(),
                                       _stream(seq_lens.device))
    _check("sparse_mla_dcp_local_seq_lens", st)
    return out


_dense_ws = {}


def dense_decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                 S: int, softmax_scale: float, block_size: int, max_seq_len: int, dcp_size: int = 1,
                 dcp_rank: int = 0, interleave: int = 1, out: Optional[torch.Tensor] = None,
                 out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Whole-context decode: q [B*S,H,576] bf16 (row b*S + s), seq_lens [B] int32 (each <= max_seq_len).
    Returns out [B*S,H,512] and lse [B*S,H] (the [batch * seq_len, heads] rows)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_cache, "kv_cache", torch.uint8, 2)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    T, H, D = q.shape
    nb = seq_lens.shape[0]
    if D != HEAD_DIM or q.stride(2) != 1:
        raise ValueError("q must be [B*S,H,576] with contiguous dims")
    if T != nb * S:
        raise ValueError(f"q has {T} rows, seq_lens and S give {nb} x {S}")
    if kv_cache.shape[1] != RECORD_BYTES or not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be a contiguous [num_slots,656] uint8 tensor")
    if (block_table.shape[1] > 1 and block_table.stride(1) != 1) or (nb > 1 and seq_lens.stride(0) != 1):
        raise ValueError("block_table and seq_lens need a contiguous last dimension")
    dev = q.device
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=out_dtype, device=dev)
    if tuple(out.shape) != (T, H, LATENT_DIM) or out.stride(2) != 1:
        raise ValueError("out must be [B*S,H,512] with contiguous dims")
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(lse, "lse", torch.float32, 2)
    if workspace is None:
        need = sparse_mla_dense_decode_workspace_size(nb, S, H, max_seq_len, dcp_size, interleave)
        key = (dev.index if dev.index is not None else torch.cuda.current_device())
        workspace = _dense_ws.get(key)
        if workspace is None or workspace.numel() < need + 256:
            workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
            _dense_ws[key] = workspace
    ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    pad = (-ws_ptr) % 256
    R, W = block_table.shape
    st = sparse_mla_dense_decode(
        q.data_ptr(), _st(q, 0), _st(q, 1), kv_cache.data_ptr(), kv_cache.shape[0], block_table.data_ptr(),
        _st(block_table, 0), R, W, seq_lens.data_ptr(), nb, S, H, block_size, dcp_size, dcp_rank, interleave,
        max_seq_len, float(softmax_scale), out.data_ptr(), _dtype_code(out.dtype), _st(out, 0), _st(out, 1),
        lse.data_ptr(), _st(lse, 0), _st(lse, 1), ws_ptr + pad, ws_bytes - pad, _stream(dev))
    _check("sparse_mla_dense_decode", st)
    return out, lse
