"""GPU parity of the draft loop over a compacted KV: the selected rows gathered
once (sv_compact_kv, bit-exact copies) and each draft token's decode over them
plus its tail (sv_dense_draft_attn) against the CPU oracle, on seeded inputs
spanning several chunks and ragged per-sequence row counts, with the edge
cases (no rows, one row, a full buffer, counts past the buffer)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import KVCache as OKV
from workloads import make_custom, make_tail_rows
from tests.gpu_util import DevWorkload, as_f64, check_out, i32, to_torch

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


def _bits(t: torch.Tensor) -> np.ndarray:
    """Storage bits of a device tensor (uint16 for bf16, float32 otherwise)."""
    x = t.detach().cpu()
    return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()


def _case(seed, dtype, D, G, paged, B=3, P=(700, 64, 300), N=4):
    Hkv = 4
    return make_custom(seed=seed, B=B, Hq=G * Hkv, Hkv=Hkv, D=D, dtype=dtype, P=list(P), N=N, score_rows="all",
                       k_sel=10, decode_steps=3, q_std_mult=6.0, layout="paged" if paged else "contiguous",
                       page_size=16, seq_extra=8)


def _lists_to_dev(lists, stride):
    arr = np.full((len(lists), stride), -1, np.int32)
    for b, li in enumerate(lists):
        arr[b, : len(li)] = li
    return i32(arr), i32(np.array([len(x) for x in lists], np.int32))


@pytest.mark.parametrize("dtype,paged", [("bf16", False), ("f32", True), ("bf16", True)])
def test_compact_kv_bit_exact(dtype, paged):
    """Rows < n_b are exactly the listed cache rows (any order, prefix and
    verify tokens alike); rows >= n_b keep what was there; n_idx past max_idx
    or past cap is clamped."""
    wl = _case(300 + int(paged), dtype, 128, 4, paged)
    dw = DevWorkload(wl)
    rng = np.random.default_rng(11)
    lists = [rng.choice(704, 257, replace=False).astype(np.int32),
             np.zeros(0, np.int32),
             rng.permutation(304)[:65].astype(np.int32)]
    idx, n = _lists_to_dev(lists, 300)
    cap = 200
    shape = (wl.B, cap, wl.Hkv, wl.D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ck = torch.full(shape, 7.0, dtype=tdt, device="cuda")
    cv = torch.full(shape, -3.0, dtype=tdt, device="cuda")
    sv.compact_kv(dw.kv, idx, n, cap, max_idx=260, ck=ck, cv=cv)
    ref_k, ref_v = oracle.compact_kv(OKV.of(wl), [li[:260] for li in lists], cap)
    gk, gv = _bits(ck), _bits(cv)
    sentinel_k, sentinel_v = _bits(torch.full((1,), 7.0, dtype=tdt))[0], _bits(torch.full((1,), -3.0, dtype=tdt))[0]
    for b, li in enumerate(lists):
        nb = min(len(li), 260, cap)
        assert np.array_equal(gk[b, :nb], ref_k[b, :nb]), f"K rows of sequence {b}"
        assert np.array_equal(gv[b, :nb], ref_v[b, :nb]), f"V rows of sequence {b}"
        assert (gk[b, nb:] == sentinel_k).all() and (gv[b, nb:] == sentinel_v).all(), f"rows past n_{b} touched"


@pytest.mark.parametrize("dtype,D,G", [("bf16", 128, 4), ("bf16", 64, 2), ("bf16", 128, 8), ("f32", 128, 4),
                                       ("f32", 64, 1)])
def test_dense_draft_parity(dtype, D, G):
    """Decode over rows [0, n_b) of dense buffers, ragged n_b: several key blocks
    and a ragged tail, one row, no rows, the whole buffer, a count past cap."""
    B, Hkv, cap = 5, 4, 700
    wl = make_custom(seed=320 + D + G, B=B, Hq=G * Hkv, Hkv=Hkv, D=D, dtype=dtype, P=[cap] * B, N=1,
                     score_rows="all", k_sel=10, decode_steps=1, q_std_mult=6.0)
    ck_np = wl.k.reshape(B, wl.seq_stride, Hkv, D)[:, :cap]
    cv_np = wl.v.reshape(B, wl.seq_stride, Hkv, D)[:, :cap]
    ck, cv = to_torch(ck_np, dtype), to_torch(cv_np, dtype)
    n_rows = np.array([517, 1, 0, cap, cap + 40], np.int32)
    out = sv.dense_draft_attn(to_torch(wl.dq[0], dtype), ck, cv, i32(n_rows))
    ref = oracle.dense_draft_attention(wl.dq[0], dtype, ck_np, cv_np, np.minimum(n_rows, cap), wl.scale, Hkv)
    g = as_f64(out)
    check_out(g, ref, dtype, "dense draft")
    assert (g[2] == 0).all()
    # one row: the output is that row's V (exactly, up to the output rounding)
    check_out(g[1], oracle.dense_draft_attention(wl.dq[0][1:2], dtype, ck_np[1:2], cv_np[1:2], [1], wl.scale, Hkv)[0],
              dtype, "one row")


@pytest.mark.parametrize("dtype,paged", [("bf16", False), ("f32", True)])
def test_draft_loop_with_tail(dtype, paged):
    """Compact once, then three draft tokens, each appending its own K/V row
    behind the set before its decode: every step matches the oracle, and the
    sparse step over the same positions (tail rows placed past the prefix)."""
    wl = _case(340 + int(paged), dtype, 128, 4, paged, P=(900, 300, 620))
    dw = DevWorkload(wl)
    rng = np.random.default_rng(5)
    lists = [np.sort(rng.choice(int(wl.P[b]), n, replace=False)).astype(np.int32)
             for b, n in enumerate((300, 77, 512))]
    idx, n = _lists_to_dev(lists, 512)
    steps = 3
    cap = 512 + steps
    ck, cv = sv.compact_kv(dw.kv, idx, n, cap)
    tail_k, tail_v = make_tail_rows(41, steps, wl.B, wl.Hkv, wl.D, dtype)
    ok, ov = oracle.compact_kv(OKV.of(wl), lists, cap)
    # the same tail rows in a cache copy, at logical positions P_b + N + s
    k2, v2 = wl.k.copy(), wl.v.copy()
    okv = OKV.of(wl)
    for b in range(wl.B):
        sl = okv.slots(b, int(wl.P[b]) + wl.N + np.arange(steps))
        k2[sl], v2[sl] = tail_k[:, b], tail_v[:, b]
    kv2 = sv.KVCache(to_torch(k2, dtype), to_torch(v2, dtype), seq_stride=wl.seq_stride,
                     page_table=dw.kv.page_table, page_size=wl.page_size)
    okv2 = OKV(k2, v2, dtype, wl.layout, wl.seq_stride, wl.page_size, wl.page_table)
    for s in range(steps):
        for b in range(wl.B):
            r = len(lists[b]) + s
            ck[b, r] = to_torch(tail_k[s, b], dtype)
            cv[b, r] = to_torch(tail_v[s, b], dtype)
            ok[b, r], ov[b, r] = tail_k[s, b], tail_v[s, b]
        rows = np.array([len(li) + s + 1 for li in lists], np.int32)
        q = dw.dq[s]
        dense = as_f64(sv.dense_draft_attn(q, ck, cv, i32(rows)))
        ref = oracle.dense_draft_attention(wl.dq[s], dtype, ok, ov, rows, wl.scale, wl.Hkv)
        check_out(dense, ref, dtype, f"dense step {s}")
        ext = [np.concatenate([lists[b], int(wl.P[b]) + wl.N + np.arange(s + 1)]).astype(np.int32)
               for b in range(wl.B)]
        eidx, en = _lists_to_dev(ext, 512 + steps)
        sparse = as_f64(sv.sparse_draft_attn(q, kv2, eidx, en))
        check_out(sparse, oracle.sparse_draft_attention(wl.dq[s], dtype, okv2, ext, wl.scale, wl.Hkv), dtype,
                  f"sparse step {s}")
        check_out(dense, sparse, dtype, f"dense vs sparse step {s}")


def test_dense_draft_workspace_garbage_and_determinism():
    """The workspace is scratch (garbage in it changes nothing) and results
    are bit-identical from call to call."""
    B, Hkv, D, G, cap = 2, 8, 128, 4, 4100
    wl = make_custom(seed=360, B=B, Hq=G * Hkv, Hkv=Hkv, D=D, dtype="bf16", P=[cap] * B, N=1, score_rows="all",
                     k_sel=10, decode_steps=1, q_std_mult=6.0)
    ck_np = wl.k.reshape(B, wl.seq_stride, Hkv, D)[:, :cap]
    cv_np = wl.v.reshape(B, wl.seq_stride, Hkv, D)[:, :cap]
    ck, cv = to_torch(ck_np, "bf16"), to_torch(cv_np, "bf16")
    n_rows = np.array([4097, 2049], np.int32)
    q = to_torch(wl.dq[0], "bf16")
    ws = sv.Workspace()
    ws.get(sv.dense_draft_workspace_size(B, G * Hkv, Hkv, D, cap, sv.SV_BF16), "cuda")
    ref = oracle.dense_draft_attention(wl.dq[0], "bf16", ck_np, cv_np, n_rows, wl.scale, Hkv)
    first = None
    for fill in ("random", 0xFF, 0x00):
        if fill == "random":
            ws.buf.copy_(torch.randint(0, 256, ws.buf.shape, dtype=torch.uint8, device="cuda"))
        else:
            ws.buf.fill_(fill)
        out = sv.dense_draft_attn(q, ck, cv, i32(n_rows), workspace=ws)
        check_out(as_f64(out), ref, "bf16", f"fill={fill}")
        if first is None:
            first = out.clone()
        assert torch.equal(out, first)
