"""Throughput of blockwise causal GQA attention (forward + backward) on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
the device promise check, the forward kernel (O, LSE), then the backward
(promise check, dO.O pre-pass, dK/dV with the first contribution stored, dQ).
Default workload: one context-parallel rank's share at B64/S8192/Hq32/Hkv8/D256,
chunks 0 and 15 of 16 per sequence (65536 query rows against 524288 K/V rows).

Prints one JSON line.  `value` is causal TFLOP/s with FLOP = 14 * D per visible
(query, key) pair per query head (forward 4D, backward 10D), inputs resident in
HBM.  `roofline` reports the dominant kernel, timed with HIP events on the
stream it runs on; `cpu_baseline` times the FP64 oracle on a bounded sample of
the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--no-cpu] [--no-ring]
                       [--no-heads] [--no-a2a] [--recompute-dq]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention fwd+bwd TFLOP/s (causal) and % of BF16 MFMA peak, 1 MI355X"


def visible_pairs(seq_lens, chunks, causal) -> int:
    """Visible (query, key) pairs per query head (closed form per chunk)."""
    tot = 0
    for s, _, p0, n in chunks:
        L = int(seq_lens[s])
        p0, n = int(p0), int(n)
        if causal:
            # sum over p in [p0, p0+n) of min(p+1, L); p < L always holds
            tot += n * (p0 + 1) + n * (n - 1) // 2
        else:
            tot += n * L
    return tot


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-ring", action="store_true", help="skip the key-window ring-step timing")
    ap.add_argument("--no-heads", action="store_true", help="skip the head-group (strided view) timing")
    ap.add_argument("--no-a2a", action="store_true", help="skip the A2A swap-copy timing")
    ap.add_argument("--recompute-dq", action="store_true",
                    help="dQ forms S, P and dP again instead of multiplying the stored dS")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Short hash of the HIP sources (what the counter summaries were taken on)."""
    import hashlib
    d = os.path.join(ROOT, "context_causal_gqa_cpattn_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    src_hash, val = None, None
    for line in open(path):
        line = line.strip()
        if line.startswith("kernel_source_hash:"):
            src_hash = line.split(":", 1)[1].strip().strip("`")
        if line.startswith(f"hbm_bytes_per_launch[{kernel}]:"):
            val = float(line.split(":", 1)[1].strip().strip("`"))
    return val if (val is not None and src_hash == kernel_source_hash()) else None


def layout_copy_rates(cp, torch, reps=10):
    """BHSD <-> THD copies at B8/H32/S2048/D128 (256 MiB moved per call), GB/s."""
    B, H, S, D = 8, 32, 2048, 128
    x = torch.empty((B, H, S, D), dtype=torch.bfloat16, device="cuda").normal_()
    so = torch.arange(B, dtype=torch.int32, device="cuda") * S
    sl = torch.full((B,), S, dtype=torch.int32, device="cuda")
    thd = torch.empty((B * S, H, D), dtype=torch.bfloat16, device="cuda")
    back = torch.empty_like(x)
    err = cp.new_dev_err()
    out = {}
    for name, fn in (("pack", lambda: cp.pack(x, so, sl, B * S, thd=thd, dev_err=err)),
                     ("unpack", lambda: cp.unpack(thd, so, sl, B, S, bhsd=back, dev_err=err))):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name + "_gbs"] = round(2 * x.numel() * 2 / (ms * 1e-3) / 1e9, 1)
        out[name + "_ms"] = round(ms, 4)
    cp.check(err)
    out["bytes_per_call"] = 2 * x.numel() * 2
    return out


def a2a_copy_rates(cp, torch, reps=10):
    """The A2A swap copies of one rank at CP4, B64/S8192/Hq32/Hkv8/D128 (the pages' CP4/A2A
    coordinate): Q [131072, 32, 128] and K [131072, 8, 128] split into 4 head groups, the
    4 received blocks scattered into whole sequences [524288, Hc, 128], and O gathered
    and merged back.  GB/s counts the bytes read plus written."""
    import workloads as W
    B, S, Hq, Hkv, D, n = 64, 8192, 32, 8, 128, 4
    lens = np.full(B, S, np.int32)
    maps, rpr = W.a2a_rank_maps(lens, n)
    lay = cp.make_a2a_layout(maps, (np.arange(B) * S).astype(np.int32), lens)
    err = cp.new_dev_err()
    q = torch.empty((rpr, Hq, D), dtype=torch.bfloat16, device="cuda").normal_()
    k = torch.empty((rpr, Hkv, D), dtype=torch.bfloat16, device="cuda").normal_()
    q_send = torch.empty((n, rpr, Hq // n, D), dtype=torch.bfloat16, device="cuda")
    k_send = torch.empty((n, rpr, Hkv // n, D), dtype=torch.bfloat16, device="cuda")
    q_full = torch.empty((B * S, Hq // n, D), dtype=torch.bfloat16, device="cuda")
    k_full = torch.empty((B * S, Hkv // n, D), dtype=torch.bfloat16, device="cuda")
    o_back = torch.empty_like(q)
    ops = {
        "split_heads_q": (lambda: cp.a2a_split_heads(q, n, dst=q_send), q.numel()),
        "split_heads_kv": (lambda: cp.a2a_split_heads(k, n, dst=k_send), k.numel()),
        "scatter_rows_q": (lambda: cp.a2a_scatter_rows(q_send, lay, B * S, full=q_full, dev_err=err), q.numel()),
        "scatter_rows_kv": (lambda: cp.a2a_scatter_rows(k_send, lay, B * S, full=k_full, dev_err=err),
                            k.numel()),
        "gather_rows_o": (lambda: cp.a2a_gather_rows(q_full, lay, rpr, blocks=q_send, dev_err=err), q.numel()),
        "merge_heads_o": (lambda: cp.a2a_merge_heads(q_send, dst=o_back), q.numel()),
        "torch_split_heads_q": (lambda: q_send.copy_(q.view(rpr, n, Hq // n, D).transpose(0, 1)), q.numel()),
    }
    out = {"workload": "cp4_a2a_rank_share_b64_s8192_hq32_hkv8_d128"}
    for name, (fn, elems) in ops.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "gbs": round(2 * elems * 2 / (ms * 1e-3) / 1e9, 1)}
    cp.check(err)
    # one forward's copies: Q, K, V in (split + scatter each), O out (gather + merge)
    out["forward_swap_ms"] = round(sum(out[k]["ms"] for k in ("split_heads_q", "scatter_rows_q",
                                                               "gather_rows_o", "merge_heads_o"))
                                   + 2 * (out["split_heads_kv"]["ms"] + out["scatter_rows_kv"]["ms"]), 4)
    return out


def ring_step_rates(cp, torch, w, q, k, v, do, bias, lay, flop, windows=8, reps=2):
    """The workload split into `windows` key windows of equal length, as a ring of steps.

    Forward: one window forward per step, each merged into the running (O, LSE).
    Backward: one window backward per step (the pre-pass once), dQ added over the
    steps.  Timed separately from the main step (not part of `value`)."""
    Lmax = int(max(w.seq_lens))
    edges = [Lmax * i // windows for i in range(windows)] + [1 << 30]
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.q_rows), dtype=torch.float32, device="cuda")
    o_w = torch.empty_like(q)
    lse_w = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    prob = cp.problem(lay, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale, w.bias_len)
    # The dS store lets each window's dQ share multiply the dS its dK/dV pass stored;
    # the smaller workspace forms dS again for dQ (timed as bwd_recompute).
    ws_rc = torch.empty(max(cp.workspace_size(prob, cp.OP_BWD), 256), dtype=torch.uint8, device="cuda")
    ws = ws_rc
    if w.head_dim >= 32:
        ws = torch.empty(max(cp.workspace_size(prob, cp.OP_BWD_DS), 256), dtype=torch.uint8, device="cuda")
    err = cp.new_dev_err()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def fwd():
        for i in range(windows):
            lo, hi = edges[i], edges[i + 1]
            if i == 0:
                cp.fwd_window(q, k, v, lay, lo, hi, causal=w.causal, scale=w.scale, bias=bias, o=o, lse=lse,
                              dev_err=err)
            else:
                cp.fwd_window(q, k, v, lay, lo, hi, causal=w.causal, scale=w.scale, bias=bias, o=o_w,
                              lse=lse_w, dev_err=err)
                cp.merge(prob, lay, o, lse, o_w, lse_w, dev_err=err)

    def bwd(buf=None):
        for i in range(windows):
            cp.bwd_window(q, k, v, lay, o, lse, do, edges[i], edges[i + 1], causal=w.causal, scale=w.scale,
                          bias=bias, prepass=(i == 0), dq=dq, dq_accumulate=(i > 0), dk=dk, dv=dv,
                          ws=ws if buf is None else buf, dev_err=err)

    def merges():
        for _ in range(windows - 1):
            cp.merge(prob, lay, o, lse, o_w, lse_w, dev_err=err)

    out = {"windows": windows}
    fwd()
    bwd()
    torch.cuda.synchronize()
    runs = [("fwd", fwd), ("bwd", bwd), ("merges", merges)]
    if ws is not ws_rc:
        runs.append(("bwd_recompute", lambda: bwd(ws_rc)))
    for name, fn in runs:
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 3)
    cp.check(err)
    out["tflops"] = round(flop / ((out["fwd_ms"] + out["bwd_ms"]) * 1e-3) / 1e12, 2)
    out["merge_gbs"] = round(3 * q.numel() * 2 * (windows - 1) / (out["merges_ms"] * 1e-3) / 1e9, 1)
    return out


def head_group_rates(cp, torch, w, q, k, v, do, bias, lay, flop, groups=(16, 8, 4), reps=2):
    """The step run as head-group calls on strided views (query heads [h0, h0 + Hg) and
    their KV heads), one workspace sized for a group serving every group call.

    The backward workspace grows with the heads of a call (the stored dS above all), so
    a group call needs Hg / Hq of the full call's.  Timed separately from the main step
    (not part of `value`)."""
    G = w.hq // w.hkv
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.q_rows), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    err = cp.new_dev_err()

    def ws_need(Hg):
        pg = cp.problem(lay, w.q_rows, w.kv_rows, Hg, Hg // G, w.head_dim, w.causal, w.scale, w.bias_len,
                        w.hq, w.hkv)
        return max(cp.workspace_size(pg, cp.OP_BWD), cp.workspace_size(pg, cp.OP_BWD_DS))

    groups = [g for g in groups if g < w.hq and w.hq % g == 0 and g % G == 0]
    if not groups:
        return None
    ws = torch.empty(max(ws_need(g) for g in groups), dtype=torch.uint8, device="cuda")
    out = {"full_call_workspace_bytes": max(cp.workspace_size(cp.problem(
        lay, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale, w.bias_len), op)
        for op in (cp.OP_BWD, cp.OP_BWD_DS))}

    def run(Hg):
        for h0 in range(0, w.hq, Hg):
            hs, gs = slice(h0, h0 + Hg), slice(h0 // G, (h0 + Hg) // G)
            bv = None if bias is None else bias[hs]
            cp.fwd(q[:, hs], k[:, gs], v[:, gs], lay, causal=w.causal, scale=w.scale, bias=bv, o=o[:, hs],
                   lse=lse[hs], dev_err=err)
            cp.bwd(q[:, hs], k[:, gs], v[:, gs], lay, o[:, hs], lse[hs], do[:, hs], causal=w.causal,
                   scale=w.scale, bias=bv, dq=dq[:, hs], dk=dk[:, gs], dv=dv[:, gs], want_dbias=False, ws=ws,
                   dev_err=err)

    for Hg in groups:
        run(Hg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run(Hg)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"H{Hg}"] = {"calls": w.hq // Hg, "ms_per_step": round(ms, 3),
                         "tflops": round(flop / (ms * 1e-3) / 1e12, 2), "workspace_bytes": ws_need(Hg)}
    cp.check(err)
    return out


def cpu_baseline(w, q, k, v, do, bias, budget_s):
    """The FP64 oracle, as it stands, on whole (sequence, KV-head group) samples."""
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_info
    import torch

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    G = w.hq // w.hkv
    order = [(b, g) for b in range(w.num_seqs) for g in range(w.hkv)]
    rng = np.random.default_rng(0)
    rng.shuffle(order)
    done_flop, t_used, samples = 0, 0.0, []
    for b, g in order:
        sub, qi, ki = W.subset(w, seqs={b})
        tq = torch.from_numpy(qi).cuda()
        tk = torch.from_numpy(ki).cuda()
        f64 = lambda t, idx: t.index_select(0, idx).float().cpu().numpy().astype(np.float64)
        qs, dos = f64(q, tq), f64(do, tq)
        ks, vs = f64(k, tk), f64(v, tk)
        bs = None if bias is None else bias.cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.attention(qs, ks, vs, sub.seq_offsets, sub.seq_lens, sub.chunks, w.causal, w.scale,
                         bias=bs, do=dos, select=(None, {g}))
        t_used += time.perf_counter() - t0
        done_flop += visible_pairs(sub.seq_lens, sub.chunks, w.causal) * G * 14 * w.head_dim
        samples.append((b, g))
        if t_used >= budget_s:
            break
    return {
        "value": done_flop / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"FP64 NumPy oracle fwd+bwd on {len(samples)} (sequence, KV-head group) pairs "
                  f"{samples[:4]}{'...' if len(samples) > 4 else ''}: {done_flop:.3e} FLOP in {t_used:.1f} s",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is designed, not built)"}))
        sys.exit(2)
    import torch
    import context_causal_gqa_cpattn_amd as cp
    import workloads as W

    cp.load()
    w = W.make_config(args.config, materialize=False)
    q, k, v, do, bias = W.draw_on_device(w, 2000 + args.config)
    lay = cp.make_layout(w.seq_offsets, w.seq_lens, w.chunks, "cuda",
                         max_chunk_len=w.max_chunk_len, max_kv_len=w.max_kv_len)
    prob = cp.problem(lay, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale,
                      w.bias_len)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.q_rows), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dbias = torch.empty_like(bias) if bias is not None else None
    # With room for it (head_dim >= 64), dK/dV stores dS and dQ multiplies the stored dS.
    ws_ds = 0 if args.recompute_dq else cp.workspace_size(prob, cp.OP_BWD_DS)
    use_ds = ws_ds > 0
    ws = torch.empty(max(ws_ds, cp.workspace_size(prob, cp.OP_BWD), 256), dtype=torch.uint8, device="cuda")
    err = cp.new_dev_err()

    names = ["fwd", "validate", "prepass", "dkdv", "dq"] + (["dbias"] if bias is not None else [])

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        cp.fwd(q, k, v, lay, causal=w.causal, scale=w.scale, bias=bias, o=o, lse=lse, dev_err=err)
        mark(1)
        cp.validate(prob, lay, err)
        mark(2)
        cp.bwd_prepass(prob, lay, q, o, do, ws, err)
        mark(3)
        if use_ds:
            cp.bwd_dkdv_ds(prob, lay, q, k, v, bias, lse, do, ws, dk, dv, False, err)
            mark(4)
            cp.bwd_dq_ds(prob, lay, k, ws, dq, err)
        else:
            cp.bwd_dkdv(prob, lay, q, k, v, bias, lse, do, ws, dk, dv, False, err)
            mark(4)
            cp.bwd_dq(prob, lay, q, k, v, bias, lse, do, ws, dq, err)
        mark(5)
        if bias is not None:
            if use_ds:
                cp.bwd_dbias_ds(prob, lay, ws, dbias, err)
            else:
                cp.bwd_dbias(prob, lay, q, k, v, bias, lse, do, ws, dbias, err)
            mark(6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cp.check(err)

    n_ev = len(names) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cp.check(err)
    per_kernel = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1])
                                     for i in range(args.steps)])) for j, n in enumerate(names)}
    ms = wall * 1e3 / args.steps

    copy = layout_copy_rates(cp, torch)
    a2a = None if args.no_a2a else a2a_copy_rates(cp, torch)
    ring = None if args.no_ring else ring_step_rates(
        cp, torch, w, q, k, v, do, bias, lay, visible_pairs(w.seq_lens, w.chunks, w.causal) * w.hq * 14 * w.head_dim)

    heads = None if args.no_heads else head_group_rates(
        cp, torch, w, q, k, v, do, bias, lay, visible_pairs(w.seq_lens, w.chunks, w.causal) * w.hq * 14 * w.head_dim)

    pairs = visible_pairs(w.seq_lens, w.chunks, w.causal) * w.hq
    D = w.head_dim
    flop = pairs * 14 * D
    tflops = flop / (ms * 1e-3) / 1e12
    fwd_tflops = pairs * 4 * D / (per_kernel["fwd"] * 1e-3) / 1e12
    bwd_ms = sum(per_kernel[n] for n in names[1:])
    bwd_tflops = pairs * 10 * D / (bwd_ms * 1e-3) / 1e12
    # dominant kernel: the longest one; its algorithmic FLOP per launch
    algo = {"fwd": 4 * D, "dkdv": 8 * D, "dq": 2 * D}
    dom = max((n for n in per_kernel if n in algo), key=lambda n: per_kernel[n])
    dom_flop = pairs * algo[dom]
    achieved = dom_flop / (per_kernel[dom] * 1e-3) / 1e12
    # pre-pass: reads Q, O, dO; writes Delta and the Q^T / dO^T tiles (32 queries, zero
    # padded)
    n_tiles = int(sum(-(-int(n) // 32) for n in w.chunks[:, 3]))
    pre_bytes = (3 * w.q_valid_rows().sum() * w.hq * D * 2 + 4 * w.q_valid_rows().sum() * w.hq
                 + 2 * n_tiles * w.hq * 32 * D * 2)

    # stored dS: one 2 KB block per (32-query tile, head, 32-key block with a visible pair),
    # written by dK/dV and read by dQ
    ds_bytes = 0
    for b, r0, pos0, n in w.chunks:
        L = int(w.seq_lens[b])
        for t in range(-(-int(n) // 32)):
            last = int(pos0) + min(32 * (t + 1), int(n)) - 1
            ds_bytes += -(-min(L, last + 1 if w.causal else L) // 32)
    ds_bytes *= w.hq * 2048

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) BF16 drawn on the device, seeded",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "seq_len": int(w.seq_lens.max()),
                   "q_rows": w.q_rows, "kv_rows": w.kv_rows, "hq": w.hq, "hkv": w.hkv,
                   "head_dim": D, "causal": bool(w.causal), "chunks": w.num_chunks,
                   "flop_per_step": flop, "parallelism": "none (one GPU: one rank's share)"},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(bwd_tflops, 2),
        "kernel_ms": {n: round(x, 4) for n, x in per_kernel.items()},
        "prepass_gbs": round(pre_bytes / (per_kernel["prepass"] * 1e-3) / 1e9, 1),
        "dq_path": "stored dS" if use_ds else "recompute",
        "ds_bytes_per_step": ds_bytes if use_ds else 0,
        "layout_copy": copy,
        "a2a_copy": a2a,
        "ring_step": ring,
        "head_groups": heads,
        "peak_mem_gib": round(torch.cuda.max_memory_allocated() / 2 ** 30, 2),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name, dom),
                     "algorithmic_flop_per_launch": dom_flop},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, do, bias, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
