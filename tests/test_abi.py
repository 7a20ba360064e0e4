"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before launching
anything (validation makes no HIP call, so these run on a CPU-only host)."""
import ctypes
import os
import re

import pytest

from tree_verify_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libsv.so not built")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_symbols()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_abi_version_and_empty_error():
    lib = _lib.load()
    assert lib.sv_abi_version() == 1
    assert lib.sv_last_error() in (b"",) or isinstance(lib.sv_last_error(), bytes)


def _kv(k=FAKE, v=FAKE, pt=None, ps=1, mp=0, stride=100, slots=1000):
    return _lib.SvKvCache(k, v, pt, ps, mp, stride, slots)


def _verify(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, dt=_lib.SV_BF16, B=1, N=8, Hq=32, Hkv=8, D=128, kv=_kv(), P=FAKE, P_max=32768,
             parent=None, rows=[0, 7], scale=0.0, out=FAKE, scores=FAKE, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    rows = a["rows"]
    arr = (ctypes.c_int32 * max(1, len(rows)))(*rows) if rows is not None else None
    if a["wsb"] == 0 and "wsb" not in kw:
        a["wsb"] = lib.sv_verify_workspace_size(a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], a["P_max"], a["dt"],
                                                int(a["parent"] is not None), len(rows or []), 0)
    st = lib.sv_verify_attn(a["q"], a["dt"], a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], ctypes.byref(a["kv"]),
                            a["P"], a["P_max"], a["parent"], arr, len(rows or []) if "nrows" not in kw else kw["nrows"],
                            a["scale"], a["out"], a["scores"], a["ws"], a["wsb"], a["stream"])
    return st, lib.sv_last_error().decode()


@pytest.mark.parametrize("kw,status,frag", [
    (dict(Hq=30), _lib.SV_E_INVALID, "multiple"),
    (dict(D=96), _lib.SV_E_UNSUPPORTED, "head dim"),
    (dict(N=257), _lib.SV_E_UNSUPPORTED, "exceeds"),
    (dict(N=0), _lib.SV_E_INVALID, "N must"),
    (dict(dt=7), _lib.SV_E_UNSUPPORTED, "dtype"),
    (dict(rows=[0, 8]), _lib.SV_E_INVALID, "not in [0, N)"),
    (dict(rows=[3, 3]), _lib.SV_E_INVALID, "twice"),
    (dict(scores=None), _lib.SV_E_INVALID, "scores is NULL"),
    (dict(q=None), _lib.SV_E_INVALID, "non-NULL"),
    (dict(kv=_kv(k=None)), _lib.SV_E_INVALID, "kv.k"),
    (dict(kv=_kv(slots=0)), _lib.SV_E_INVALID, "num_slots"),
    (dict(kv=_kv(pt=FAKE, ps=0, mp=4)), _lib.SV_E_INVALID, "page_size"),
    (dict(B=2, kv=_kv(stride=0)), _lib.SV_E_INVALID, "seq_stride"),
    (dict(wsb=16), _lib.SV_E_WORKSPACE, "workspace"),
    (dict(ws=None, wsb=1 << 40), _lib.SV_E_WORKSPACE, "workspace"),
    (dict(scale=-1.0), _lib.SV_E_INVALID, "softmax_scale"),
    (dict(scale=float("inf")), _lib.SV_E_INVALID, "softmax_scale"),
    (dict(P_max=-1), _lib.SV_E_INVALID, "P_max"),
])
def test_verify_rejects_bad_arguments(kw, status, frag):
    st, msg = _verify(**kw)
    assert st == status, msg
    assert frag in msg


def test_verify_empty_batch_is_ok_without_launch():
    st, msg = _verify(B=0, q=None, out=None)
    assert st == _lib.SV_OK, msg


def test_workspace_sizes_are_consistent():
    lib = _lib.load()
    chain = lib.sv_verify_workspace_size(1, 8, 32, 8, 128, 32768, _lib.SV_BF16, 0, 2, 0)
    tree = lib.sv_verify_workspace_size(1, 256, 32, 8, 128, 8192, _lib.SV_BF16, 1, 256, 0)
    assert chain > 32768 * 8 * 4 and tree > 0
    assert lib.sv_verify_workspace_size(1, 257, 32, 8, 128, 10, _lib.SV_BF16, 0, 0, 0) == 0
    # small pages shorten chunks (the page-table slice of a chunk is cached on chip): more partials
    p1 = lib.sv_verify_workspace_size(2, 8, 32, 8, 128, 65536, _lib.SV_BF16, 0, 2, 1)
    p16 = lib.sv_verify_workspace_size(2, 8, 32, 8, 128, 65536, _lib.SV_BF16, 0, 2, 16)
    assert p1 > p16 > 0
    assert lib.sv_sparse_workspace_size(1, 32, 8, 128, 2048) >= 32 * 32 * 128 * 4
    # selection: per row, 32 blocks of 512 candidate slots (value and index)
    assert lib.sv_topk_workspace_size(4, 131072) >= 4 * 32 * 512 * 8
    fused = lib.sv_verify_select_workspace_size(1, 8, 32, 8, 128, 32768, _lib.SV_BF16, 0, 2, 0)
    assert fused >= chain + lib.sv_topk_workspace_size(1, 32768)
    assert lib.sv_verify_select_workspace_size(1, 8, 32, 8, 128, 32768, _lib.SV_BF16, 0, 0, 0) == 0  # no scores
    assert lib.sv_verify_select_workspace_size(1, 8, 32, 8, 128, 131073, _lib.SV_BF16, 0, 2, 0) == 0  # too long


def test_verify_select_rejects_bad_arguments():
    lib = _lib.load()
    kv = _kv()
    rows = (ctypes.c_int32 * 2)(0, 7)
    f = lib.sv_verify_select

    def call(B=1, P_max=1000, n_rows=2, k=FAKE, k_max=64, idx=FAKE, ws_bytes=1 << 30):
        return f(FAKE, _lib.SV_BF16, B, 8, 32, 8, 128, ctypes.byref(kv), FAKE, P_max, None, rows, n_rows, 0.0, k,
                 k_max, FAKE, FAKE, idx, None, FAKE, ws_bytes, None)
    assert call(n_rows=0) == _lib.SV_E_INVALID           # selection needs scores
    assert call(P_max=131073) == _lib.SV_E_UNSUPPORTED   # longer prefixes: the two separate calls
    assert call(k=None) == _lib.SV_E_INVALID
    assert call(idx=None) == _lib.SV_E_INVALID
    assert call(k_max=-1) == _lib.SV_E_INVALID
    assert call(ws_bytes=16) == _lib.SV_E_WORKSPACE
    assert call(B=0) == _lib.SV_OK


def test_topk_and_sparse_reject_bad_arguments():
    lib = _lib.load()
    assert lib.sv_topk_select(FAKE, -1, 10, FAKE, FAKE, 4, FAKE, None, None, 0, None) == _lib.SV_E_INVALID
    assert lib.sv_topk_select(None, 1, 10, FAKE, FAKE, 4, FAKE, None, None, 0, None) == _lib.SV_E_INVALID
    assert lib.sv_topk_select(FAKE, 0, 10, FAKE, FAKE, 4, FAKE, None, None, 0, None) == _lib.SV_OK
    kv = _kv()
    sp = lib.sv_sparse_draft_attn
    assert sp(FAKE, _lib.SV_BF16, 1, 32, 8, 128, ctypes.byref(kv), FAKE, 10, FAKE, 20, 0.0, FAKE, FAKE, 1 << 30,
              None) == _lib.SV_E_INVALID                       # max_idx > idx_stride
    assert sp(FAKE, _lib.SV_BF16, 1, 32, 8, 100, ctypes.byref(kv), FAKE, 10, FAKE, 10, 0.0, FAKE, FAKE, 1 << 30,
              None) == _lib.SV_E_UNSUPPORTED
    assert sp(FAKE, _lib.SV_BF16, 1, 64, 2, 128, ctypes.byref(kv), FAKE, 10, FAKE, 10, 0.0, FAKE, FAKE, 1 << 30,
              None) == _lib.SV_E_UNSUPPORTED                   # 32 query heads per KV head
    assert sp(FAKE, _lib.SV_BF16, 1, 32, 8, 128, ctypes.byref(kv), FAKE, 10, FAKE, 10, 0.0, FAKE, FAKE, 8,
              None) == _lib.SV_E_WORKSPACE
    assert "workspace" in lib.sv_last_error().decode()


def test_compact_and_dense_draft_reject_bad_arguments():
    lib = _lib.load()
    kv = _kv()
    cp = lib.sv_compact_kv
    args = lambda **k: dict(dict(dt=_lib.SV_BF16, B=1, Hkv=8, D=128, idx=FAKE, stride=10, n=FAKE, max_idx=10,  # noqa: E731
                                 ck=FAKE, cv=FAKE, cap=16), **k)

    def compact(**k):
        a = args(**k)
        return cp(a["dt"], a["B"], a["Hkv"], a["D"], ctypes.byref(kv), a["idx"], a["stride"], a["n"], a["max_idx"],
                  a["ck"], a["cv"], a["cap"], None)
    assert compact(max_idx=11) == _lib.SV_E_INVALID                 # max_idx > idx_stride
    assert compact(cap=0) == _lib.SV_E_INVALID
    assert compact(D=96) == _lib.SV_E_UNSUPPORTED
    assert compact(dt=3) == _lib.SV_E_UNSUPPORTED
    assert compact(ck=FAKE + 8) == _lib.SV_E_INVALID
    assert "aligned" in lib.sv_last_error().decode()
    assert compact(n=None) == _lib.SV_E_INVALID
    assert compact(B=0, ck=None, cv=None) == _lib.SV_OK
    dd = lib.sv_dense_draft_attn
    need = lib.sv_dense_draft_workspace_size(1, 32, 8, 128, 4096, _lib.SV_BF16)
    # the decode is one verify query over a contiguous buffer of cap slots per sequence
    assert need == lib.sv_verify_workspace_size(1, 1, 32, 8, 128, 4095, _lib.SV_BF16, 0, 0, 0) > 0
    assert lib.sv_dense_draft_workspace_size(1, 32, 8, 128, 0, _lib.SV_BF16) == 0
    assert dd(FAKE, _lib.SV_BF16, 1, 32, 8, 128, FAKE, FAKE, 0, FAKE, 0.0, FAKE, FAKE, need, None) == _lib.SV_E_INVALID
    assert dd(FAKE, _lib.SV_BF16, 1, 30, 8, 128, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, FAKE, need, None) == _lib.SV_E_INVALID
    assert dd(FAKE, _lib.SV_BF16, 1, 32, 8, 128, FAKE, FAKE, 4096, None, 0.0, FAKE, FAKE, need, None) == _lib.SV_E_INVALID
    assert dd(FAKE, _lib.SV_BF16, 1, 32, 8, 128, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, FAKE, need - 1,
              None) == _lib.SV_E_WORKSPACE
    assert dd(None, _lib.SV_BF16, 0, 32, 8, 128, None, None, 4096, None, 0.0, None, None, 0, None) == _lib.SV_OK


def test_accept_commit_rejects_bad_arguments():
    lib = _lib.load()
    kv = _kv()
    ac = lib.sv_accept_commit

    def call(B=1, N=8, kvp=ctypes.byref(kv), P=FAKE, draft=FAKE, target=FAKE, path=FAKE, nacc=FAKE, newp=FAKE, D=128):
        return ac(_lib.SV_BF16, B, N, 8, D, kvp, P, 100, None, draft, target, path, nacc, None, newp, None)
    assert call(N=0) == _lib.SV_E_INVALID
    assert call(N=257) == _lib.SV_E_UNSUPPORTED
    assert call(D=96) == _lib.SV_E_UNSUPPORTED
    assert call(draft=None) == _lib.SV_E_INVALID
    assert call(path=None) == _lib.SV_E_INVALID
    assert call(P=None) == _lib.SV_E_INVALID                      # the K/V move needs P_b
    assert "prefix_len" in lib.sv_last_error().decode()
    assert call(B=0, draft=None, target=None, path=None, nacc=None) == _lib.SV_OK


def test_build_tree_rejects_bad_arguments():
    lib = _lib.load()
    bt = lib.sv_build_tree
    assert bt(1, 0, 8, 32, FAKE, FAKE, None, None, None) == _lib.SV_E_INVALID
    assert bt(1, 257, 8, 32, FAKE, FAKE, None, None, None) == _lib.SV_E_UNSUPPORTED
    assert bt(1, 16, 8, 300, FAKE, FAKE, None, None, None) == _lib.SV_E_UNSUPPORTED
    assert bt(1, 16, 2, 3, FAKE, FAKE, None, None, None) == _lib.SV_E_INVALID     # 1 + 3 + 9 = 13 reachable
    assert "reachable" in lib.sv_last_error().decode()
    assert bt(1, 2, 0, 32, FAKE, FAKE, None, None, None) == _lib.SV_E_INVALID     # depth 0: only the root
    assert bt(1, 16, 8, 32, None, FAKE, None, None, None) == _lib.SV_E_INVALID
    assert bt(0, 16, 8, 32, None, None, None, None, None) == _lib.SV_OK


def test_selection_variants_reject_bad_arguments():
    lib = _lib.load()
    sw = lib.sv_select_sink_window
    assert sw(1, 100, FAKE, 4, 8, 11, FAKE, None, None) == _lib.SV_E_INVALID     # k_max < sink + window
    assert sw(1, 100, FAKE, -1, 8, 11, FAKE, None, None) == _lib.SV_E_INVALID
    assert sw(1, 100, None, 4, 8, 12, FAKE, None, None) == _lib.SV_E_INVALID
    assert sw(0, 100, None, 4, 8, 12, None, None, None) == _lib.SV_OK
    kv = _kv()
    sp = lib.sv_sparse_draft_attn_per_head
    assert sp(FAKE, _lib.SV_BF16, 1, 32, 8, 128, ctypes.byref(kv), FAKE, 10, FAKE, 20, 0.0, FAKE, FAKE, 1 << 30,
              None) == _lib.SV_E_INVALID                       # max_idx > idx_stride
    vp = lib.sv_verify_attn_per_head
    rows = (ctypes.c_int32 * 2)(0, 7)
    assert vp(FAKE, _lib.SV_BF16, 1, 8, 30, 8, 128, ctypes.byref(kv), FAKE, 100, None, rows, 2, 0.0, FAKE, FAKE,
              FAKE, 1 << 30, None) == _lib.SV_E_INVALID          # Hq not a multiple of Hkv


def test_timing_events_must_pair():
    lib = _lib.load()
    assert lib.sv_set_verify_timing_events(FAKE, None) == _lib.SV_E_INVALID
    assert lib.sv_set_verify_timing_events(None, None) == _lib.SV_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_validators_reject_bad_arguments():
    """sv_validate_*: the error record must be a non-NULL aligned device
    pointer, sizes non-negative, arrays present; all checked before launching."""
    lib = _lib.load()
    kv = _kv()
    assert lib.sv_validate_kv(2, 8, ctypes.byref(kv), FAKE, 100, None, None) == 1
    assert lib.sv_validate_kv(2, 8, ctypes.byref(kv), FAKE, 100, FAKE + 2, None) == 1
    assert "aligned" in lib.sv_last_error().decode()
    assert lib.sv_validate_kv(-1, 8, ctypes.byref(kv), FAKE, 100, FAKE, None) == 1
    assert lib.sv_validate_kv(2, 8, ctypes.byref(kv), None, 100, FAKE, None) == 1
    assert lib.sv_validate_kv(2, 8, None, FAKE, 100, FAKE, None) == 1
    assert lib.sv_validate_kv(70000, 8, ctypes.byref(kv), FAKE, 100, FAKE, None) == 2
    assert lib.sv_validate_tree(2, 8, None, FAKE, None) == 1
    assert lib.sv_validate_tree(2, -1, FAKE, FAKE, None) == 1
    assert lib.sv_validate_tree(2, 8, FAKE, None, None) == 1
    assert lib.sv_validate_index(2, 0, ctypes.byref(kv), FAKE, 64, FAKE, 64, FAKE, None) == 1
    assert lib.sv_validate_index(2, 1, ctypes.byref(kv), FAKE, 32, FAKE, 64, FAKE, None) == 1
    assert lib.sv_validate_index(2, 1, ctypes.byref(kv), FAKE, 64, None, 64, FAKE, None) == 1
    assert lib.sv_validate_index(40000, 8, ctypes.byref(kv), FAKE, 64, FAKE, 64, FAKE, None) == 2
