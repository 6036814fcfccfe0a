"""CPU checks of the C ABI: the library loads, exports every declared call, and rejects bad
arguments from the host side without touching a GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import sparse_mla_decode_topk_amd as smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, MISALIGNED = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(smla.lib_path()):
        pytest.skip("libsmla.so not built")
    return smla.load_library()


def test_header_lists_the_calls():
    names = declared_functions()
    for n in ("smla_abi_version", "smla_status_string", "sparse_mla_convert_index", "sparse_mla_decode",
              "sparse_mla_decode_workspace_size", "sparse_mla_merge_lse", "sparse_mla_cache_write",
              "sparse_mla_dcp_local_seq_lens", "sparse_mla_dense_decode", "sparse_mla_dense_decode_workspace_size", "sparse_mla_decode_bf16"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(smla.lib_path())
    for n in declared_functions():
        assert hasattr(raw, n), f"{n} declared in smla.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.smla_abi_version() == 3
    for st in range(0, 7):
        assert isinstance(lib.smla_status_string(st), bytes) and lib.smla_status_string(st)


# fake, never dereferenced, device-looking addresses (the calls below fail validation first)
A16 = 0x10000
A4 = 0x10004


def convert_call(lib, **kw):
    a = dict(ids=A16, ids_ld=8, req=A16, bt=A16, bt_ld=4, bt_rows=2, bt_width=4, T=3, K=8, B=64, D=1, r=0, I=1,
             out=A16, out_ld=8, valid=None)
    a.update(kw)
    return lib.sparse_mla_convert_index(a["ids"], a["ids_ld"], a["req"], a["bt"], a["bt_ld"], a["bt_rows"],
                                        a["bt_width"], a["T"], a["K"], a["B"], a["D"], a["r"], a["I"], a["out"],
                                        a["out_ld"], a["valid"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(T=-1), INVALID), (dict(K=-1), INVALID), (dict(B=0), INVALID), (dict(D=0), INVALID),
    (dict(D=2, r=2), UNSUPPORTED), (dict(r=-1), INVALID), (dict(I=0), INVALID), (dict(ids_ld=4), INVALID),
    (dict(out_ld=4), INVALID), (dict(bt_ld=2), INVALID), (dict(bt_rows=0), INVALID), (dict(ids=None), INVALID),
    (dict(out=None), INVALID), (dict(req=None), INVALID), (dict(bt=None), INVALID),
    (dict(ids=A16 + 2), MISALIGNED), (dict(valid=A16 + 1), MISALIGNED),
    (dict(out=A16, ids=A16, out_ld=16), INVALID),  # exact alias with a different row stride
    (dict(T=0), OK), (dict(T=0, ids=None), OK), (dict(K=0), OK),
    (dict(K=0, ids=None, out=None, out_ld=3), OK),  # empty tensors carry null pointers
])
def test_convert_validation(lib, kw, want):
    assert convert_call(lib, **kw) == want


def test_convert_accepts_4_byte_aligned_index_arrays(lib):
    # passes validation up to the launch: with T=0 nothing is launched
    assert convert_call(lib, ids=A4, req=A4 + 8, bt=A4 + 4, out=A4, T=0) == OK


def decode_call(lib, **kw):
    a = dict(q=A16, qst=128 * 576, qsh=576, kv=A16, ns=100, slots=A16, sld=64, valid=None, T=2, H=128, K=64,
             scale=0.07, out=A16, odt=0, ost=128 * 512, osh=512, lse=A16, lst=128, lsh=1, splits=0, ws=None, wsb=0)
    a.update(kw)
    return lib.sparse_mla_decode(a["q"], a["qst"], a["qsh"], a["kv"], a["ns"], a["slots"], a["sld"], a["valid"],
                                 a["T"], a["H"], a["K"], a["scale"], a["out"], a["odt"], a["ost"], a["osh"], a["lse"],
                                 a["lst"], a["lsh"], a["splits"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(T=-1), INVALID), (dict(H=0), INVALID), (dict(K=-3), INVALID), (dict(ns=-1), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(odt=2), INVALID), (dict(splits=-1), INVALID), (dict(splits=65), INVALID), (dict(sld=32), INVALID),
    (dict(qst=-576), INVALID), (dict(H=136), UNSUPPORTED), (dict(H=40), UNSUPPORTED), (dict(H=200), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(lse=None), INVALID), (dict(slots=None), INVALID),
    (dict(kv=None), INVALID), (dict(q=A16 + 2), MISALIGNED), (dict(qsh=580), MISALIGNED),
    (dict(kv=A16 + 8), MISALIGNED), (dict(slots=A16 + 2), MISALIGNED), (dict(out=A16 + 8), MISALIGNED),
    (dict(odt=1, osh=514), MISALIGNED), (dict(lse=A16 + 2), MISALIGNED),
    (dict(K=8192, sld=8192, splits=1), UNSUPPORTED), (dict(K=128, sld=128, splits=2), WORKSPACE),
    (dict(K=128, sld=128, splits=2, ws=A16 + 64, wsb=1 << 30), MISALIGNED), (dict(valid=A16 + 2), MISALIGNED),
    (dict(T=0), OK), (dict(T=0, q=None, out=None), OK),
])
def test_decode_validation(lib, kw, want):
    assert decode_call(lib, **kw) == want
    # the bf16-record decode validates its arguments the same way
    a = dict(q=A16, qst=128 * 576, qsh=576, kv=A16, ns=100, slots=A16, sld=64, valid=None, T=2, H=128, K=64,
             scale=0.07, out=A16, odt=0, ost=128 * 512, osh=512, lse=A16, lst=128, lsh=1, splits=0, ws=None, wsb=0)
    a.update(kw)
    assert lib.sparse_mla_decode_bf16(a["q"], a["qst"], a["qsh"], a["kv"], a["ns"], a["slots"], a["sld"], a["valid"],
                                      a["T"], a["H"], a["K"], a["scale"], a["out"], a["odt"], a["ost"], a["osh"],
                                      a["lse"], a["lst"], a["lsh"], a["splits"], a["ws"], a["wsb"], None) == want


def test_workspace_size(lib):
    # one split needs nothing; s splits need (max, sum) pairs and fp32 partial outputs
    assert lib.sparse_mla_decode_workspace_size(256, 128, 2048, 1) == 0
    T, H, K, S = 32, 64, 2048, 8
    r = lambda x: (x + 255) // 256 * 256
    want = r(T * S * H * 2 * 4) + r(T * S * H * 512 * 4)
    assert lib.sparse_mla_decode_workspace_size(T, H, K, S) == want
    assert lib.sparse_mla_decode_workspace_size(0, 64, 2048, 0) == 0
    assert lib.sparse_mla_decode_workspace_size(4, 64, -1, 0) == 0


def merge_call(lib, **kw):
    a = dict(p=A16, pdt=1, pss=4 * 64 * 512, pst=64 * 512, psh=512, lp=A16, lss=4 * 64, lst=64, lsh=1, S=2, T=4, H=64,
             out=A16, odt=0, ost=64 * 512, osh=512, lse=A16, lo_t=64, lo_h=1)
    a.update(kw)
    return lib.sparse_mla_merge_lse(a["p"], a["pdt"], a["pss"], a["pst"], a["psh"], a["lp"], a["lss"], a["lst"], a["lsh"],
                                    a["S"], a["T"], a["H"], a["out"], a["odt"], a["ost"], a["osh"], a["lse"], a["lo_t"],
                                    a["lo_h"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(S=0), INVALID), (dict(S=65), UNSUPPORTED), (dict(T=-1), INVALID), (dict(H=0), INVALID),
    (dict(pdt=3), INVALID), (dict(odt=5), INVALID), (dict(p=None), INVALID), (dict(lp=None), INVALID),
    (dict(out=None), INVALID), (dict(pss=-1), INVALID), (dict(p=A16 + 4), MISALIGNED),
    (dict(psh=514), MISALIGNED), (dict(lp=A16 + 1), MISALIGNED), (dict(out=A16 + 8), MISALIGNED),
    (dict(T=0), OK),
])
def test_merge_validation(lib, kw, want):
    assert merge_call(lib, **kw) == want


def cache_write_call(lib, **kw):
    a = dict(lat=A16, lst=512, rope=A16, rst=64, dt=0, pos=A16, req=A16, bt=A16, bt_ld=4, bt_rows=2, bt_width=4, N=3,
             B=64, D=1, r=0, I=1, kv=A16, ns=100, sm=A16)
    a.update(kw)
    return lib.sparse_mla_cache_write(a["lat"], a["lst"], a["rope"], a["rst"], a["dt"], a["pos"], a["req"], a["bt"],
                                      a["bt_ld"], a["bt_rows"], a["bt_width"], a["N"], a["B"], a["D"], a["r"], a["I"],
                                      a["kv"], a["ns"], a["sm"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(N=-1), INVALID), (dict(ns=-1), INVALID), (dict(dt=2), INVALID), (dict(B=0), INVALID), (dict(D=0), INVALID),
    (dict(D=2, r=2), UNSUPPORTED), (dict(r=-1), INVALID), (dict(I=0), INVALID), (dict(bt_ld=2), INVALID), (dict(bt_rows=0), INVALID),
    (dict(lst=256), INVALID), (dict(rst=32), INVALID), (dict(lat=None), INVALID), (dict(rope=None), INVALID),
    (dict(pos=None), INVALID), (dict(req=None), INVALID), (dict(bt=None), INVALID), (dict(kv=None), INVALID),
    (dict(D=1 << 16, I=1 << 15), UNSUPPORTED),
    (dict(lat=A16 + 8), MISALIGNED), (dict(lst=516), MISALIGNED), (dict(dt=1, lst=514), MISALIGNED),
    (dict(rope=A16 + 1), MISALIGNED), (dict(dt=1, rope=A16 + 2), MISALIGNED), (dict(pos=A16 + 2), MISALIGNED),
    (dict(kv=A16 + 8), MISALIGNED), (dict(sm=A16 + 1), MISALIGNED),
    (dict(N=0), OK), (dict(N=0, lat=None, kv=None), OK),
])
def test_cache_write_validation(lib, kw, want):
    assert cache_write_call(lib, **kw) == want


@pytest.mark.parametrize("args,want", [
    ((A16, -1, 1, 0, 1, A16), INVALID), ((A16, 4, 0, 0, 1, A16), INVALID), ((A16, 4, 2, 2, 1, A16), UNSUPPORTED),
    ((A16, 4, 2, -1, 1, A16), INVALID),
    ((A16, 4, 2, 0, 0, A16), INVALID), ((None, 4, 2, 0, 1, A16), INVALID), ((A16, 4, 2, 0, 1, None), INVALID),
    ((A16 + 2, 4, 2, 0, 1, A16), MISALIGNED), ((A16, 4, 2, 0, 1, A16 + 1), MISALIGNED),
    ((None, 0, 2, 1, 1, None), OK),
])
def test_local_seq_lens_validation(lib, args, want):
    assert lib.sparse_mla_dcp_local_seq_lens(*args, None) == want


def dense_call(lib, **kw):
    a = dict(q=A16, qst=128 * 576, qsh=576, kv=A16, ns=100, bt=A16, bt_ld=8, bt_rows=2, bt_width=8, sl=A16, B=2, S=4,
             H=128, blk=64, D=1, r=0, I=1, maxlen=512, scale=0.07, out=A16, odt=0, ost=128 * 512, osh=512, lse=A16,
             lst=128, lsh=1, ws=A16 * 16, wsb=1 << 30)
    a.update(kw)
    return lib.sparse_mla_dense_decode(a["q"], a["qst"], a["qsh"], a["kv"], a["ns"], a["bt"], a["bt_ld"], a["bt_rows"],
                                       a["bt_width"], a["sl"], a["B"], a["S"], a["H"], a["blk"], a["D"], a["r"], a["I"],
                                       a["maxlen"], a["scale"], a["out"], a["odt"], a["ost"], a["osh"], a["lse"],
                                       a["lst"], a["lsh"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), INVALID), (dict(S=0), INVALID), (dict(H=0), INVALID), (dict(maxlen=-1), INVALID),
    (dict(blk=0), INVALID), (dict(D=2, r=2), UNSUPPORTED), (dict(r=-1), INVALID), (dict(I=0), INVALID),
    (dict(bt_ld=4), INVALID),
    (dict(bt_rows=0), INVALID), (dict(sl=None), INVALID), (dict(bt=None), INVALID), (dict(q=None), INVALID),
    (dict(scale=0.0), INVALID), (dict(H=40), UNSUPPORTED), (dict(maxlen=(1 << 18) + 1), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE), (dict(ws=A16 * 16 + 16), MISALIGNED),
    (dict(sl=A16 + 2), MISALIGNED), (dict(q=A16 + 2), MISALIGNED),
    (dict(B=0), OK), (dict(B=0, q=None, ws=None), OK),
])
def test_dense_validation(lib, kw, want):
    assert dense_call(lib, **kw) == want


def test_dense_workspace_size(lib):
    # slot lists (B*S rows of the list width) ahead of the decode's own workspace
    r = lambda x: (x + 255) // 256 * 256
    ws = lib.sparse_mla_dense_decode_workspace_size(2, 4, 128, 512, 1, 1)
    assert ws >= r(8 * 512 * 4)
    assert lib.sparse_mla_dense_decode_workspace_size(2, 4, 128, 1000, 2, 1) >= r(8 * 500 * 4)
    assert lib.sparse_mla_dense_decode_workspace_size(0, 4, 128, 512, 1, 1) == 0
    assert lib.sparse_mla_dense_decode_workspace_size(2, 4, 128, (1 << 18) + 1, 1, 1) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 16, 576, dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        smla.decode(q, torch.zeros(4, 656, dtype=torch.uint8), torch.zeros(1, 4, dtype=torch.int32), 0.1)


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "sparse_mla_decode_topk_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text
