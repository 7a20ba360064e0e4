#!/usr/bin/env python3
"""Benchmark of the verification-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
sv_verify_attn (dense tree/chain verification + fused criticality scores) ->
sv_topk_select -> the draft steps (one draft query per sequence, or the
workload's number of draft steps over the same selected set): each step
sv_sparse_draft_attn over the selected positions, or (--draft-path compact,
the default for several draft steps) sv_compact_kv once and then
sv_dense_draft_attn per step over the gathered rows -- the same attention.

Default workload: the 32k-context Llama-3-8B-shaped layer (B=1, 32 query /
8 KV heads, D=128, bf16, prefix 32768, chain of 8 verify queries,
Collect-2-Query scoring, k=2048, one sparse draft step).

Prints ONE JSON line.  `value` is the whole step's algorithmic bytes divided
by the measured step time (GB/s), timed over K plain steps; `roofline` is for
the dominant kernel (the verify main kernel), timed with start/stop events
that its own dispatch records on the call stream, over a second pass of the
same K steps (those timestamped dispatches cost about 5 us per step, so they
stay out of the step time); `cpu_baseline` is the CPU oracle timed on a
bounded sample on the host.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
F32_MFMA_PEAK_TFS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kv-copies", type=int, default=0,
                    help="KV copies rotated between steps so that no step hits the 256 MB MALL (0 = auto)")
    ap.add_argument("--draft-path", choices=["auto", "sparse", "compact"], default="auto",
                    help="draft steps gather the selected rows each time (sparse), or the set is gathered "
                         "once into dense buffers and every step streams them (compact); auto: compact "
                         "when the workload has more than one draft step")
    ap.add_argument("--selection", choices=["scores", "per_head", "sink_window"], default="scores",
                    help="scores: one key set per sequence from the fused scores (the method); per_head: one "
                         "set per KV head from per-head scores; sink_window: the first 64 and the last k - 64 "
                         "positions, no scores (the query-agnostic baseline)")
    ap.add_argument("--select-path", choices=["fused", "separate"], default="fused",
                    help="fused: sv_verify_select (the selection inside the verification's last kernel); "
                         "separate: sv_verify_attn then sv_topk_select (same results)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweeps", action="store_true", help="skip the 4K..128K prefix sweep")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-oracle sample time")
    ap.add_argument("--copy-reference-mib", type=int, default=0,
                    help="before timing, run 3 plain device-to-device copies of this many MiB (a known-size "
                         "reference for HBM byte counters read by a profiler)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(a sequence's KV heads and chunks would shard across GPUs, each GPU "
              "running this same path on its share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_verify_sparse_amd as sv
    from tree_verify_sparse_amd import _lib
    from workloads import make_workload, CONFIG_NAMES

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = sv.lib()

    wl = make_workload(args.workload, args.seed)
    es = 2 if wl.dtype == "bf16" else 4
    n_draft = int(wl.dq.shape[0])

    def to_dev(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    kv_bytes = wl.k.nbytes + wl.v.nbytes
    copies = args.kv_copies or max(1, min(8, int(np.ceil(600e6 / kv_bytes))))
    k0, v0 = to_dev(wl.k), to_dev(wl.v)
    kcs = [k0] + [k0.clone() for _ in range(copies - 1)]
    vcs = [v0] + [v0.clone() for _ in range(copies - 1)]
    q = to_dev(wl.q)
    dqs = [to_dev(wl.dq[s]) for s in range(n_draft)]
    P = i32(wl.P)
    ksel = i32(wl.k_sel)
    parent = i32(wl.parent) if wl.parent is not None else None
    pt = i32(wl.page_table) if wl.page_table is not None else None
    out = torch.empty_like(q)
    scores = torch.empty((wl.B, wl.P_max), dtype=torch.float32, device=dev)
    kmax = wl.k_max
    idx = torch.empty((wl.B, kmax), dtype=torch.int32, device=dev)
    count = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    douts = [torch.empty_like(d) for d in dqs]
    dt = _lib.SV_BF16 if wl.dtype == "bf16" else _lib.SV_F32
    rows = [int(r) for r in wl.score_rows]
    rows_arr = (ctypes.c_int32 * max(1, len(rows)))(*rows)
    vws_n = sv.verify_workspace_size(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, wl.P_max, dt, parent is not None, len(rows),
                                     wl.page_size if pt is not None else 0)
    sws_n = sv.sparse_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.D, kmax)
    vws = torch.empty(max(1, vws_n), dtype=torch.uint8, device=dev)
    sws = torch.empty(max(1, sws_n), dtype=torch.uint8, device=dev)
    tws_n = sv.topk_workspace_size(wl.B, wl.P_max)
    tws = torch.empty(max(1, tws_n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    # prebuilt C arguments, one set per KV copy (keeps per-step host work to three C calls)
    kvs = [_lib.SvKvCache(kc.data_ptr(), vc.data_ptr(), pt.data_ptr() if pt is not None else None,
                          wl.page_size if pt is not None else 1, wl.max_pages, wl.seq_stride, wl.num_slots)
           for kc, vc in zip(kcs, vcs)]
    vargs = [(q.data_ptr(), dt, wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, ctypes.byref(kv), P.data_ptr(), wl.P_max,
              parent.data_ptr() if parent is not None else None, rows_arr, len(rows), 0.0, out.data_ptr(),
              scores.data_ptr(), vws.data_ptr(), vws_n, sp) for kv in kvs]
    targs = (scores.data_ptr(), wl.B, wl.P_max, P.data_ptr(), ksel.data_ptr(), kmax, idx.data_ptr(),
             count.data_ptr(), tws.data_ptr(), tws_n, sp)
    dargs = [[(dqs[s].data_ptr(), dt, wl.B, wl.Hq, wl.Hkv, wl.D, ctypes.byref(kv), idx.data_ptr(), kmax,
               count.data_ptr(), kmax, 0.0, douts[s].data_ptr(), sws.data_ptr(), sws_n, sp)
              for s in range(n_draft)] for kv in kvs]
    f_verify, f_topk, f_sparse, f_hook = L.sv_verify_attn, L.sv_topk_select, L.sv_sparse_draft_attn, \
        L.sv_set_verify_timing_events
    # fused verification + selection: one call, one workspace holding both
    fused = args.select_path == "fused" and args.selection == "scores" and rows and wl.P_max <= 131072
    if fused:
        fws_n = sv.verify_select_workspace_size(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, wl.P_max, dt, parent is not None,
                                                len(rows), wl.page_size if pt is not None else 0)
        fws = torch.empty(max(1, fws_n), dtype=torch.uint8, device=dev)
        fargs = [a[:14] + (ksel.data_ptr(), kmax, out.data_ptr(), scores.data_ptr(), idx.data_ptr(),
                           count.data_ptr(), fws.data_ptr(), fws_n, sp) for a in vargs]
    f_fused = L.sv_verify_select
    # compacted draft loop: the selected rows gathered once per step into dense
    # [B][k_max][Hkv][D] buffers, every draft step decoding over rows [0, count)
    draft_path = args.draft_path
    if draft_path == "auto":
        draft_path = "compact" if n_draft > 1 else "sparse"
    if draft_path == "compact" and n_draft > 0:
        cshape = (wl.B, max(1, kmax), wl.Hkv, wl.D)
        ck = torch.empty(cshape, dtype=q.dtype, device=dev)
        cv = torch.empty(cshape, dtype=q.dtype, device=dev)
        dws_n = L.sv_dense_draft_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.D, max(1, kmax), dt)
        dws = torch.empty(max(1, dws_n), dtype=torch.uint8, device=dev)
        cargs = [(dt, wl.B, wl.Hkv, wl.D, ctypes.byref(kv), idx.data_ptr(), kmax, count.data_ptr(), kmax,
                  ck.data_ptr(), cv.data_ptr(), max(1, kmax), sp) for kv in kvs]
        ddargs = [(dqs[s].data_ptr(), dt, wl.B, wl.Hq, wl.Hkv, wl.D, ck.data_ptr(), cv.data_ptr(), max(1, kmax),
                   count.data_ptr(), 0.0, douts[s].data_ptr(), dws.data_ptr(), dws_n, sp) for s in range(n_draft)]
    f_compact, f_dense = L.sv_compact_kv, L.sv_dense_draft_attn
    # selection variants (the method's fused scores by default)
    selection = args.selection
    if selection == "per_head":
        H = wl.Hkv
        hscores = torch.empty((wl.B, H, wl.P_max), dtype=torch.float32, device=dev)
        P_rows = i32(np.repeat(wl.P, H))
        k_rows = i32(np.repeat(wl.k_sel, H))
        hidx = torch.empty((wl.B, H, kmax), dtype=torch.int32, device=dev)
        hcount = torch.empty((wl.B, H), dtype=torch.int32, device=dev)
        tws_h = torch.empty(max(1, sv.topk_workspace_size(wl.B * H, wl.P_max)), dtype=torch.uint8, device=dev)
        vargs = [a[:15] + (hscores.data_ptr(),) + a[16:] for a in vargs]
        targs = (hscores.data_ptr(), wl.B * H, wl.P_max, P_rows.data_ptr(), k_rows.data_ptr(), kmax,
                 hidx.data_ptr(), hcount.data_ptr(), tws_h.data_ptr(), tws_h.numel(), sp)
        dargs = [[(dqs[s].data_ptr(), dt, wl.B, wl.Hq, wl.Hkv, wl.D, ctypes.byref(kv), hidx.data_ptr(), kmax,
                   hcount.data_ptr(), kmax, 0.0, douts[s].data_ptr(), sws.data_ptr(), sws_n, sp)
                  for s in range(n_draft)] for kv in kvs]
        f_verify, f_sparse = L.sv_verify_attn_per_head, L.sv_sparse_draft_attn_per_head
        draft_path = "sparse"  # one list per KV head: the per-head gathered step
    elif selection == "sink_window":
        sink = min(64, kmax)
        window = kmax - sink
        vargs = [a[:11] + (rows_arr, 0) + a[13:15] + (None,) + a[16:] for a in vargs]  # no scores
        targs = (wl.B, wl.P_max, P.data_ptr(), sink, window, kmax, idx.data_ptr(), count.data_ptr(), sp)
        f_topk = L.sv_select_sink_window

    def step(i, ev=None):
        c = i % copies
        if ev is not None:
            f_hook(ev[0].cuda_event, ev[1].cuda_event)
        if fused:
            st = f_fused(*fargs[c])
        else:
            st = f_verify(*vargs[c])
            st |= f_topk(*targs)
        if draft_path == "compact" and n_draft > 0:
            st |= f_compact(*cargs[c])
            for a in ddargs:
                st |= f_dense(*a)
        else:
            for a in dargs[c]:
                st |= f_sparse(*a)
        if st:
            raise RuntimeError(L.sv_last_error().decode())

    if args.copy_reference_mib > 0:
        n = args.copy_reference_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in kev:        # torch creates events lazily: force creation before handing them to the library
        a.record()
        b.record()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # timed region: K plain steps
    torch.cuda.synchronize()
    e0.record()
    for i in range(K):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / K
    # the same K steps again, this time with the verify kernel's dispatch recording
    # start/stop events on the call stream (its duration for the roofline).  Kept
    # out of the step timing: the timestamped dispatches add about 5 us per step.
    torch.cuda.synchronize()
    e0.record()
    for i in range(K):
        step(i, kev[i])
    e1.record()
    torch.cuda.synchronize()
    f_hook(None, None)
    ms_step_events = e0.elapsed_time(e1) / K
    k_ms = [a.elapsed_time(b) for a, b in kev]
    kern_ms = float(np.mean(k_ms))

    # ---- algorithmic work
    Pb = wl.P.astype(np.int64)
    kk = np.minimum(wl.k_sel.astype(np.int64), Pb)
    row_b = wl.Hkv * wl.D * es
    verify_bytes = int((Pb + wl.N).sum() * row_b * 2 + wl.q.nbytes * 2 + (Pb.sum() * 4 if rows else 0))
    select_bytes = int(Pb.sum() * 4 + kk.sum() * 4) if rows else 0
    draft_bytes = int(n_draft * (kk.sum() * row_b * 2 + 2 * wl.B * wl.Hq * wl.D * es + kk.sum() * 4))
    step_bytes = verify_bytes + select_bytes + draft_bytes
    # verify flops: QK^T and PV over every visible key of every query row
    vis = 0
    for b in range(wl.B):
        depth = np.zeros(wl.N, np.int64)
        for t in range(1, wl.N):
            depth[t] = depth[(t - 1) if wl.parent is None else wl.parent[b, t]] + 1
        vis += int(wl.N * Pb[b] + (depth + 1).sum())
    verify_flops = 4 * wl.Hq * wl.D * vis

    # the bound is the roof the kernel would hit first at full efficiency: MFMA when the
    # verify pass's arithmetic intensity (flops per algorithmic byte) exceeds the ridge
    # point peak_flops / peak_bytes, HBM otherwise
    peak = BF16_MFMA_PEAK_TFS if wl.dtype == "bf16" else F32_MFMA_PEAK_TFS
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_bound = verify_flops / verify_bytes >= ridge
    if mfma_bound:
        achieved = verify_flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        achieved = verify_bytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    # bf16 with at most 64 query rows per KV head runs the key-split streaming kernel
    if wl.dtype == "bf16":  # bf16: key-split streaming kernel up to 64 rows per KV head, tree kernel above
        roof["kernel"] = "verify_stream" if wl.N * (wl.Hq // wl.Hkv) <= 64 else "verify_tree"
    else:
        roof["kernel"] = "verify_main"
    roof["kernel_us"] = round(kern_ms * 1e3, 2)
    # the same launch against the other roof too (the tree workloads sit near the ridge)
    roof["hbm_frac"] = round(verify_bytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    roof["mfma_frac"] = round(verify_flops / (kern_ms * 1e-3) / 1e12 / peak, 4)
    roof["flops_per_byte"] = round(verify_flops / verify_bytes, 1)
    roof["ridge_flops_per_byte"] = round(ridge, 1)
    roof["algorithmic_bytes"] = verify_bytes
    roof["algorithmic_flops"] = verify_flops
    roof["traffic"] = _traffic(args.workload)

    # after the timed passes: acceptance of this workload's drafts with the
    # accepted branch's K/V moved in place, on KV copy 0.  Synthetic target
    # tokens always match some child, so every path runs to a leaf (the
    # longest walks and the most row moves)
    from workloads import make_accept_tokens
    par_np = wl.parent if wl.parent is not None else np.tile(np.arange(-1, wl.N - 1, dtype=np.int32), (wl.B, 1))
    d_tok, t_tok = make_accept_tokens([args.workload, args.seed], par_np, match_prob=1.0)
    d_tok, t_tok = i32(d_tok), i32(t_tok)
    apath = torch.empty((wl.B, wl.N), dtype=torch.int32, device=dev)
    an = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    abonus = torch.empty_like(an)
    anewp = torch.empty_like(an)
    aargs = (dt, wl.B, wl.N, wl.Hkv, wl.D, ctypes.byref(kvs[0]), P.data_ptr(), wl.P_max,
             parent.data_ptr() if parent is not None else None, d_tok.data_ptr(), t_tok.data_ptr(), apath.data_ptr(),
             an.data_ptr(), abonus.data_ptr(), anewp.data_ptr(), sp)
    for _ in range(3):
        L.sv_accept_commit(*aargs)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        if L.sv_accept_commit(*aargs):
            raise RuntimeError(L.sv_last_error().decode())
    e1.record()
    torch.cuda.synchronize()
    accept_us = e0.elapsed_time(e1) * 1e3 / K
    # device tree construction for tree workloads: this workload's tree shape
    # from seeded per-depth log-probabilities (the same generator as its trees)
    build_us = None
    if wl.parent is not None:
        from workloads import depth_logprobs
        dmax = {3: 8, 5: 6}.get(args.workload, 8)
        r = np.random.default_rng([args.workload, args.seed, 99])
        lps = torch.from_numpy(np.stack([depth_logprobs(r, dmax) for _ in range(wl.B)])).to(dev)
        bt_par = torch.empty((wl.B, wl.N), dtype=torch.int32, device=dev)
        bargs = (wl.B, wl.N, dmax, int(lps.shape[2]), lps.data_ptr(), bt_par.data_ptr(), None, None, sp)
        for _ in range(3):
            L.sv_build_tree(*bargs)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            if L.sv_build_tree(*bargs):
                raise RuntimeError(L.sv_last_error().decode())
        e1.record()
        torch.cuda.synchronize()
        build_us = e0.elapsed_time(e1) * 1e3 / K

    # tokens-per-time projection (KnapSpec §2) for chains, from this layer's
    # measured times: t_target = verification with selection (and the
    # compaction on that path), t_draft = one draft decode; gamma = the chain's
    # drafted tokens.  One attention layer only: the projection leaves out the
    # models' other layers and MLPs, and alpha is assumed, not measured.
    def timed(fn):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(K):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    def select_only(i):
        if f_topk(*targs):
            raise RuntimeError(L.sv_last_error().decode())

    def draft_only(i):
        st = f_dense(*ddargs[0]) if draft_path == "compact" else f_sparse(*dargs[i % copies][0])
        if st:
            raise RuntimeError(L.sv_last_error().decode())

    # the selection and one draft decode on their own (after a full step, so the
    # scores and the selected set are current), against the HBM roof: their
    # algorithmic bytes per call over the call's time (launch included)
    step(0)
    select_us = timed(select_only)
    per_draft_bytes = draft_bytes // n_draft if n_draft > 0 else 0
    draft_us = timed(draft_only) if n_draft > 0 else None
    other_roofs = {
        "select": {"us": round(select_us, 2), "algorithmic_bytes": select_bytes,
                   "achieved_GBs": round(select_bytes / select_us / 1e3, 1),
                   "frac": round(select_bytes / select_us / 1e3 / HBM_PEAK_GBS, 5)},
        "draft_decode": None if draft_us is None else {
            "us": round(draft_us, 2), "algorithmic_bytes": per_draft_bytes,
            "achieved_GBs": round(per_draft_bytes / draft_us / 1e3, 1),
            "frac": round(per_draft_bytes / draft_us / 1e3 / HBM_PEAK_GBS, 4)},
    }

    tpt_rows = None
    if wl.parent is None and n_draft > 0:

        def target(i):
            c = i % copies
            st = f_fused(*fargs[c]) if fused else (f_verify(*vargs[c]) | f_topk(*targs))
            if draft_path == "compact":
                st |= f_compact(*cargs[c])
            if st:
                raise RuntimeError(L.sv_last_error().decode())

        t_target, t_draft = timed(target), draft_us
        gamma = wl.N - 1
        tpt_rows = {"gamma": gamma, "t_target_us": round(t_target, 2), "t_draft_us": round(t_draft, 2),
                    "tokens_per_ms": {f"alpha={a}": round(tpt(a, gamma, t_draft, t_target) * 1e3, 2)
                                      for a in (0.6, 0.7, 0.8, 0.9)},
                    "scope": "one attention layer (verify + selection, one draft decode); assumed alpha"}

    # step-time distribution: the same K steps with an event between consecutive
    # steps (each step's time is the gap between its two events)
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    sev[0].record()
    for i in range(K):
        step(i)
        sev[i + 1].record()
    torch.cuda.synchronize()
    st_us = np.array([sev[i].elapsed_time(sev[i + 1]) * 1e3 for i in range(K)])
    dist = {"p10_us": round(float(np.percentile(st_us, 10)), 2),
            "median_us": round(float(np.median(st_us)), 2),
            "p90_us": round(float(np.percentile(st_us, 90)), 2),
            "how": "events between consecutive steps, a third pass of the K steps"}

    # scoring overhead (Vegas §4): the verification alone (no selection) with no
    # score rows, the workload's rows, and every verify row, each over the same K
    # steps with the KV copies rotated
    sweep_rows = None
    if selection == "scores":
        variants = {"0": [], str(len(rows)): rows, str(wl.N): list(range(wl.N))}
        sweep_rows = {}
        for name, rr in variants.items():
            ra = (ctypes.c_int32 * max(1, len(rr)))(*rr)
            wn = sv.verify_workspace_size(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, wl.P_max, dt, parent is not None,
                                          len(rr), wl.page_size if pt is not None else 0)
            wt = torch.empty(max(1, wn), dtype=torch.uint8, device=dev)
            va = [a[:11] + (ra, len(rr), 0.0, out.data_ptr(), scores.data_ptr() if rr else None,
                            wt.data_ptr(), wn, sp) for a in vargs]

            def verify_only(i, va=va):
                if L.sv_verify_attn(*va[i % copies]):
                    raise RuntimeError(L.sv_last_error().decode())

            sweep_rows[name] = round(timed(verify_only), 2)
        base = sweep_rows["0"]
        sweep_rows = {"verify_us_by_score_rows": sweep_rows,
                      "overhead_pct": {k2: round((v2 / base - 1.0) * 100.0, 1) for k2, v2 in sweep_rows.items()},
                      "what": "sv_verify_attn alone (fused scores, no selection), KV copies rotated"}

    # one whole draft-verify iteration of a chain workload, measured: the target
    # pass (verification + selection) and gamma = N - 1 draft decodes over the
    # selected set, with seeded synthetic draft queries
    iteration = None
    if wl.parent is None and selection == "scores" and fused and wl.N > 1 and n_draft > 0:
        gamma = wl.N - 1
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        gq = [(torch.randn((wl.B, wl.Hq, wl.D), generator=g, device=dev) / np.sqrt(wl.D)).to(q.dtype)
              for _ in range(gamma)]
        go = [torch.empty_like(x) for x in gq]
        it_sparse = [[(gq[s].data_ptr(),) + dargs[c][0][1:12] + (go[s].data_ptr(),) + dargs[c][0][13:]
                      for s in range(gamma)] for c in range(copies)]

        def iter_sparse(i):
            c = i % copies
            st = f_fused(*fargs[c])
            for a in it_sparse[c]:
                st |= f_sparse(*a)
            if st:
                raise RuntimeError(L.sv_last_error().decode())

        iteration = {"gamma": gamma, "sparse_us": round(timed(iter_sparse), 2)}
        if draft_path != "compact":
            cshape = (wl.B, max(1, kmax), wl.Hkv, wl.D)
            ck = torch.empty(cshape, dtype=q.dtype, device=dev)
            cv = torch.empty(cshape, dtype=q.dtype, device=dev)
            dws_n = L.sv_dense_draft_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.D, max(1, kmax), dt)
            dws = torch.empty(max(1, dws_n), dtype=torch.uint8, device=dev)
            cargs = [(dt, wl.B, wl.Hkv, wl.D, ctypes.byref(kv), idx.data_ptr(), kmax, count.data_ptr(), kmax,
                      ck.data_ptr(), cv.data_ptr(), max(1, kmax), sp) for kv in kvs]
        it_dense = [(gq[s].data_ptr(), dt, wl.B, wl.Hq, wl.Hkv, wl.D, ck.data_ptr(), cv.data_ptr(),
                     max(1, kmax), count.data_ptr(), 0.0, go[s].data_ptr(), dws.data_ptr(), dws_n, sp)
                    for s in range(gamma)]

        def iter_compact(i):
            c = i % copies
            st = f_fused(*fargs[c]) | f_compact(*cargs[c])
            for a in it_dense:
                st |= f_dense(*a)
            if st:
                raise RuntimeError(L.sv_last_error().decode())

        iteration["compact_us"] = round(timed(iter_compact), 2)
        best = min(v2 for k2, v2 in iteration.items() if k2.endswith("_us"))
        iteration["tokens_per_ms"] = {f"alpha={a}": round(tokens_per_round(a, gamma) / best * 1e3, 2)
                                      for a in (0.6, 0.7, 0.8, 0.9)}
        iteration["scope"] = "one attention layer: verification + selection + gamma draft decodes; assumed alpha"

    sweeps = {"step_time_distribution": dist, "scoring_overhead": sweep_rows, "measured_iteration": iteration}
    if args.workload == 2 and not args.no_sweeps:
        sweeps["prefix_sweep"] = prefix_sweep(sv, L, _lib, dev, sp, max(20, K // 4))
    sweeps["hbm_reference"] = hbm_reference(dev)

    value = step_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": "verify+select+sparse-draft us/step and HBM GB/s (% peak) at 32k ctx, 1 GPU",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1e3, 2),
        "us_per_step_with_kernel_events": round(ms_step_events * 1e3, 2),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded; no model weights or datasets)",
        "config": {"workload": CONFIG_NAMES[args.workload], "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D,
                   "prefix": int(wl.P_max) if wl.B == 1 else [int(x) for x in wl.P], "verify_nodes": wl.N,
                   "tree": wl.parent is not None, "score_rows": len(rows), "k": int(wl.k_sel.max()),
                   "draft_steps": n_draft, "draft_path": draft_path, "selection": selection,
                   "select_path": "fused" if fused else "separate",
                   "paged": wl.layout == "paged",
                   "kv_copies_rotated": copies,
                   "step_bytes": step_bytes, "parallelism": "single-gpu"},
        "roofline": roof,
        "next_rows": {"accept_commit_us": round(accept_us, 2),
                      "accepted_mean": round(float(an.float().mean().item()), 2),
                      "build_tree_us": round(build_us, 2) if build_us is not None else None,
                      "tpt_projection": tpt_rows,
                      "select_and_draft_rooflines": other_roofs},
        "measurements": sweeps,
    }
    if not args.no_cpu_baseline:
        if args.workload in (1, 2, 3):
            res["cpu_baseline"] = cpu_baseline(wl, step_bytes, args.cpu_seconds)
        else:
            res["cpu_baseline"] = cpu_baseline_sampled(wl, step_bytes, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def _traffic(workload: int):
    """HBM bytes per verify launch from the committed rocprofv3 counter summary,
    only if the verify kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"verify_pmc_workload{workload}.md")
    src = os.path.join(ROOT, "tree_verify_sparse_amd", "csrc", "verify.hip")
    try:
        text = open(path).read()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        m = re.search(r"verify\.hip sha256:\s*([0-9a-f]{64})", text)
        t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
        if m and t and m.group(1) == sha:
            return float(t.group(1))
    except OSError:
        pass
    return None


def tokens_per_round(alpha: float, gamma: int) -> float:
    """Expected tokens of one draft-verify round (KnapSpec §2): the accepted
    drafts plus the target's own token, (1 - alpha^(gamma+1)) / (1 - alpha)."""
    return gamma + 1.0 if alpha == 1.0 else (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def prefix_sweep(sv, L, _lib, dev, sp, steps):
    """The 32k layer's step (verification + fused selection + one sparse draft
    decode; B=1, 32 query / 8 KV heads, D=128, bf16, chain of 8 verify queries,
    score rows {0, 7}, k=2048) at prefixes 4K..128K (KnapSpec §1: attention
    time linear in the context).  Keys and values are seeded N(0, 1/D) draws
    made on the device; each point rotates enough cache copies that about 1 GB
    streams between reuses (the 256 MB last-level cache holds no prefix)."""
    import numpy as np
    import torch
    Hq, Hkv, D, N, k = 32, 8, 128, 8, 2048
    rows = [0, N - 1]
    dt = _lib.SV_BF16
    row_b = Hkv * D * 2
    pool_rows = 2 * (131072 + N)
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    kpool = (torch.randn((pool_rows, Hkv, D), generator=g, device=dev) / np.sqrt(D)).to(torch.bfloat16)
    vpool = (torch.randn((pool_rows, Hkv, D), generator=g, device=dev) / np.sqrt(D)).to(torch.bfloat16)
    q = (torch.randn((1, N, Hq, D), generator=g, device=dev) / np.sqrt(D)).to(torch.bfloat16)
    dq = (torch.randn((1, Hq, D), generator=g, device=dev) / np.sqrt(D)).to(torch.bfloat16)
    out, dout = torch.empty_like(q), torch.empty_like(dq)
    ra = (ctypes.c_int32 * 2)(*rows)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pts = []
    for P in (4096, 8192, 16384, 32768, 65536, 131072):
        ncp = max(1, min(64, pool_rows // (P + N)))
        kvs = [_lib.SvKvCache(kpool.data_ptr() + c * (P + N) * row_b, vpool.data_ptr() + c * (P + N) * row_b,
                              None, 1, 0, P + N, P + N) for c in range(ncp)]
        Pt = torch.tensor([P], dtype=torch.int32, device=dev)
        kt = torch.tensor([k], dtype=torch.int32, device=dev)
        scores = torch.empty((1, P), dtype=torch.float32, device=dev)
        idx = torch.empty((1, k), dtype=torch.int32, device=dev)
        cnt = torch.empty((1,), dtype=torch.int32, device=dev)
        fn = sv.verify_select_workspace_size(1, N, Hq, Hkv, D, P, dt, False, 2, 0)
        fw = torch.empty(max(1, fn), dtype=torch.uint8, device=dev)
        sn = sv.sparse_workspace_size(1, Hq, Hkv, D, k)
        sw = torch.empty(max(1, sn), dtype=torch.uint8, device=dev)
        fa = [(q.data_ptr(), dt, 1, N, Hq, Hkv, D, ctypes.byref(kv), Pt.data_ptr(), P, None, ra, 2, 0.0,
               kt.data_ptr(), k, out.data_ptr(), scores.data_ptr(), idx.data_ptr(), cnt.data_ptr(), fw.data_ptr(),
               fn, sp) for kv in kvs]
        da = [(dq.data_ptr(), dt, 1, Hq, Hkv, D, ctypes.byref(kv), idx.data_ptr(), k, cnt.data_ptr(), k, 0.0,
               dout.data_ptr(), sw.data_ptr(), sn, sp) for kv in kvs]

        def one(i):
            c = i % ncp
            if L.sv_verify_select(*fa[c]) | L.sv_sparse_draft_attn(*da[c]):
                raise RuntimeError(L.sv_last_error().decode())

        for i in range(5):
            one(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            one(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        byts = (P + N) * row_b * 2 + q.nbytes * 2 + P * 4 + (P * 4 + k * 4) + (k * row_b * 2 + 2 * dq.nbytes + k * 4)
        pts.append({"prefix": P, "us_per_step": round(us, 2), "GBs": round(byts / us / 1e3, 1),
                    "hbm_frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 4), "kv_copies_rotated": ncp})
        del scores, idx, cnt, fw, sw
    del kpool, vpool
    torch.cuda.empty_cache()
    return {"points": pts, "steps_per_point": steps,
            "step": "sv_verify_select + one sv_sparse_draft_attn (the 32k layer's shape)"}


def hbm_reference(dev):
    """Bandwidths of plain library kernels on this GPU, for scale: a 2 GiB
    device-to-device copy (bytes read + written) and a float32 sum over 2 GiB
    of bfloat16 (bytes read)."""
    import torch
    n = 1 << 30
    x = torch.ones(n, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, byts, reps=10):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(byts * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)

    r = {"copy_GBs": rate(lambda: y.copy_(x), 2 * x.nbytes),
         "sum_read_GBs": rate(lambda: x.sum(dtype=torch.float32), x.nbytes),
         "what": "torch copy_ of 2 GiB (read + write bytes) and torch sum over 2 GiB bf16 (read bytes)"}
    del x, y
    torch.cuda.empty_cache()
    return r


def tpt(alpha: float, gamma: int, t_draft: float, t_target: float) -> float:
    """Tokens per unit of time of a draft-verify round (KnapSpec §2, the TPT
    metric): (1 - alpha^(gamma+1)) / (1 - alpha) expected tokens (gamma + 1 at
    alpha = 1) over gamma draft steps and one target pass."""
    tokens = gamma + 1.0 if alpha == 1.0 else (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)
    return tokens / (gamma * t_draft + t_target)


def cpu_baseline_sampled(wl, step_bytes, target_s):
    """The CPU oracle on a per-(sequence, KV head) sample of a workload too
    large for full steps: each sample is one sequence's slice for one KV head
    (its group of query heads, its prefix rows, its draft query) run as a whole
    step; the full step's time is estimated as the mean sample time times the
    number of (sequence, KV head) pairs.  The selection runs once per sample
    (on that head's scores) instead of once per sequence, so the estimate is a
    little above a full step's CPU time."""
    import numpy as np
    import oracle
    from types import SimpleNamespace
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    G = wl.Hq // wl.Hkv
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hkv)]
    order = np.random.default_rng(11).permutation(len(pairs))
    t0 = time.perf_counter()
    taken = []
    for j in order:
        b, h = pairs[j]
        Pb = int(wl.P[b])
        sl = wl.slot(b, np.arange(Pb + wl.N))
        sub = SimpleNamespace(
            dtype=wl.dtype, B=1, Hq=G, Hkv=1, D=wl.D, N=wl.N, P=np.array([Pb], np.int32), P_max=Pb,
            scale=wl.scale, layout="contiguous", seq_stride=Pb + wl.N, page_size=1, page_table=None,
            num_slots=Pb + wl.N, q=wl.q[b:b + 1, :, h * G:(h + 1) * G], k=wl.k[sl, h:h + 1],
            v=wl.v[sl, h:h + 1], parent=None if wl.parent is None else wl.parent[b:b + 1],
            score_rows=wl.score_rows, k_sel=wl.k_sel[b:b + 1], dq=wl.dq[:1, b:b + 1, h * G:(h + 1) * G],
            max_pages=0)
        ts = time.perf_counter()
        oracle.run_step(sub)
        taken.append((b, h, Pb, time.perf_counter() - ts))
        if time.perf_counter() - t0 >= target_s:
            break
    # scale by prefix length: a sample's time is close to linear in its prefix
    per_pos = sum(t for *_, t in taken) / sum(p + wl.N for _, _, p, _ in taken)
    est = per_pos * float((wl.P.astype(np.int64) + wl.N).sum()) * wl.Hkv
    return {"value": round(step_bytes / est / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "seconds_per_step_estimated": round(est, 3), "numpy": np.__version__, "host_cpus": os.cpu_count(),
            "sample": f"{len(taken)} of {len(pairs)} (sequence, KV head) slices run as whole steps (verify rows, "
                      f"scores, top-k, first draft step), {sum(t for *_, t in taken):.1f} s; full step estimated "
                      f"as seconds per (prefix + verify) position x all positions x KV heads"}


def cpu_baseline(wl, step_bytes, target_s):
    """The CPU oracle (unchanged, float64 numpy) timed on this host: full steps
    of the same workload, repeated until about target_s seconds have passed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.run_step(wl)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or el / reps * (reps + 1) > 3 * target_s:
            break
    per = el / reps
    return {"value": round(step_bytes / per / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "seconds_per_step": round(per, 3), "numpy": np.__version__,
            "host_cpus": os.cpu_count(),
            "sample": f"{reps} full step(s) of the same workload (all verify rows, scores, top-k, "
                      f"{wl.dq.shape[0]} draft step(s))"}


if __name__ == "__main__":
    main()
