"""sv_verify_attn_noalloc (static library scratch, no workspace argument)
against sv_verify_attn with a caller workspace, through the C ABI: two calls
in a row on one GPU, the second on a smaller input, must give the same bits
(the two entry points run the same kernels), and a call whose scratch need
exceeds the static array must fail before launching anything."""
import ctypes

import numpy as np
import pytest
import torch

import tree_verify_sparse_amd as sv
from tree_verify_sparse_amd import _lib
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _dev(wl):
    def t(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()

    def i(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()

    return t, i


def _call(L, noalloc, wl, q, kv, P, parent, out, scores, ws):
    rows = [int(r) for r in wl.score_rows]
    rows_arr = (ctypes.c_int32 * max(1, len(rows)))(*rows)
    dt = _lib.SV_BF16 if wl.dtype == "bf16" else _lib.SV_F32
    kvs = kv.c_struct()
    common = (q.data_ptr(), dt, wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, ctypes.byref(kvs), P.data_ptr(), wl.P_max,
              parent.data_ptr() if parent is not None else None, rows_arr, len(rows), 0.0, out.data_ptr(),
              scores.data_ptr())
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        return L.sv_verify_attn_noalloc(*common, stream)
    return L.sv_verify_attn(*common, ws.data_ptr(), ws.numel(), stream)


def _run_pair(L, wl):
    t, i = _dev(wl)
    q = t(wl.q)
    kv = sv.KVCache(t(wl.k), t(wl.v), seq_stride=wl.seq_stride)
    P = i(wl.P)
    parent = i(wl.parent) if wl.parent is not None else None
    dt = _lib.SV_BF16 if wl.dtype == "bf16" else _lib.SV_F32
    n = sv.verify_workspace_size(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, wl.P_max, dt, parent is not None,
                                 len(wl.score_rows))
    assert 0 < n <= 64 << 20
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")  # garbage: contents are not needed
    res = []
    for noalloc in (False, True):
        out = torch.full_like(q, float("nan"))
        scores = torch.full((wl.B, wl.P_max), float("nan"), dtype=torch.float32, device="cuda")
        st = _call(L, noalloc, wl, q, kv, P, parent, out, scores, ws)
        assert st == 0, L.sv_last_error().decode()
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy(), scores.cpu().numpy()))
    (o_ref, s_ref), (o_na, s_na) = res
    assert np.isfinite(o_na).all()
    assert np.array_equal(o_ref.view(np.uint32), o_na.view(np.uint32)), "outputs differ"
    for b in range(wl.B):
        Pb = int(wl.P[b])
        assert np.array_equal(s_ref[b, :Pb].view(np.uint32), s_na[b, :Pb].view(np.uint32)), f"scores differ, seq {b}"


def test_noalloc_matches_workspace_entry_point_twice():
    L = sv.lib()
    print("noalloc case 1: tree B=2 N=64 P=[3000,1500] bf16", flush=True)
    big = make_custom(seed=[41, 1], B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[3000, 1500], N=64,
                      tree="best_first", tree_depth=6, score_rows="all", k_sel=64, decode_steps=0, q_std_mult=4.0)
    _run_pair(L, big)
    print("noalloc case 2: chain B=1 N=8 P=700 bf16", flush=True)
    small = make_custom(seed=[41, 2], B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=[700], N=8, tree=None,
                        score_rows=[0, 7], k_sel=64, decode_steps=0, q_std_mult=4.0)
    _run_pair(L, small)


def test_noalloc_rejects_oversized_call():
    L = sv.lib()
    cap = 64 << 20
    # 16 sequences of 65536 positions with 64-node trees need far more scratch
    n = L.sv_verify_workspace_size(16, 64, 32, 8, 128, 65536, _lib.SV_BF16, 1, 64, 16)
    assert n > cap
    q = torch.zeros((16, 64, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((16, 8, 128), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((16, 4100), dtype=torch.int32, device="cuda")
    kvs = _lib.SvKvCache(k.data_ptr(), k.data_ptr(), pt.data_ptr(), 16, 4100, 0, 16)
    P = torch.full((16,), 65536, dtype=torch.int32, device="cuda")
    parent = torch.zeros((16, 64), dtype=torch.int32, device="cuda")
    rows = (ctypes.c_int32 * 64)(*range(64))
    out = torch.empty_like(q)
    scores = torch.empty((16, 65536), dtype=torch.float32, device="cuda")
    st = L.sv_verify_attn_noalloc(q.data_ptr(), _lib.SV_BF16, 16, 64, 32, 8, 128, ctypes.byref(kvs), P.data_ptr(),
                                  65536, parent.data_ptr(), rows, 64, 0.0, out.data_ptr(), scores.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == _lib.SV_E_WORKSPACE
    assert b"static array" in L.sv_last_error()
