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

Timing follows the pages' protocol (page "Optimize context parallel attention
layouts and gradient accumulation", "Current public integration": five warmups,
then 50 timed iterations, eager, default allocator, no graphs and no profiler):
`value` comes from the median of the per-step HIP-event times; the mean wall time
of the K steps (bracketed by synchronizations) is reported beside it.  The other
named workloads (full causal 8 x 2048 at D 128, the unequal padded rank share,
the pair-biased rows) follow as extra result blocks with the same protocol, each
with its own roofline and CPU baseline; they are not part of `value`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--extra 2,4,5]
                       [--no-cpu] [--no-ring] [--no-heads] [--no-a2a] [--recompute-dq]
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--extra", default="2,4,5",
                    help="other named workloads timed after the headline one ('' for none)")
    ap.add_argument("--extra-cpu-seconds", type=float, default=5.0)
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi clock/power samples")
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
    bs = None if bias is None else bias.cpu().numpy().astype(np.float64)
    for b, g in order:
        sub, qi, ki = W.subset(w, seqs={b})
        tq = torch.from_numpy(qi).cuda()
        tk = torch.from_numpy(ki).cuda()
        f64 = lambda t, idx: t.index_select(0, idx).float().cpu().numpy().astype(np.float64)
        qs, dos = f64(q, tq), f64(do, tq)
        ks, vs = f64(k, tk), f64(v, tk)
        t0 = time.perf_counter()
        oracle.attention(qs, ks, vs, sub.seq_offsets, sub.seq_lens, sub.chunks, w.causal, w.scale,
                         bias=bs, do=dos, select=(None, {g}))
        t_used += time.perf_counter() - t0
        done_flop += visible_pairs(sub.seq_lens, sub.chunks, w.causal) * G * 14 * w.head_dim
        samples.append((b, g))
        if t_used >= budget_s:
            break
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    return {
        "value": done_flop / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle",
        "blas_threads": int(threads), "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
        "sample": f"FP64 NumPy oracle fwd+bwd on {len(samples)} (sequence, KV-head group) pairs "
                  f"{samples[:4]}{'...' if len(samples) > 4 else ''}: {done_flop:.3e} FLOP in {t_used:.1f} s",
    }


# ---------------------------------------------------------------- clock / power samples

_SAMPLER = r"""
import json, select, subprocess, sys, time
out = []
if sys.stdin.readline().strip() == "start":
    while True:
        t = time.time()
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"],
                               capture_output=True, text=True, timeout=20)
            out.append({"t": t, "rc": r.returncode, "out": r.stdout[-20000:], "err": r.stderr[-500:]})
        except Exception as e:
            out.append({"t": t, "error": repr(e)})
        if select.select([sys.stdin], [], [], max(0.0, 0.25 - (time.time() - t)))[0]:
            break
print(json.dumps(out))
"""


class ClockSampler:
    """amd-smi clock and power readings taken while the timed steps run.  The sampler
    is a child process started before this process touches the GPU; it runs
    `amd-smi metric` between the "start" and "stop" lines it reads."""

    def __init__(self, enabled=True):
        import subprocess
        self.p = None
        if enabled:
            try:
                self.p = subprocess.Popen([sys.executable, "-c", _SAMPLER], stdin=subprocess.PIPE,
                                          stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
            except Exception:
                self.p = None

    def start(self):
        if self.p:
            self.p.stdin.write("start\n")
            self.p.stdin.flush()

    def stop(self):
        if not self.p:
            return None
        try:
            out, _ = self.p.communicate("stop\n", timeout=60)
            samples = json.loads(out.strip().splitlines()[-1])
        except Exception as e:
            try:
                self.p.kill()
            except Exception:
                pass
            return {"error": repr(e)}
        return summarize_smi(samples)


def summarize_smi(samples):
    """Min / max of every clock (MHz) and power (W) value found in the amd-smi JSON."""
    vals = {}

    def walk(x, path):
        if isinstance(x, dict):
            if "value" in x and isinstance(x["value"], (int, float)) and len(path) > 0:
                vals.setdefault("/".join(path), []).append(float(x["value"]))
                return
            for k2, v2 in x.items():
                walk(v2, path + [str(k2)])
        elif isinstance(x, list):
            for i2, v2 in enumerate(x):
                walk(v2, path + ([str(i2)] if len(x) > 1 else []))
        elif isinstance(x, (int, float)) and not isinstance(x, bool):
            vals.setdefault("/".join(path), []).append(float(x))

    n_ok = 0
    for smp in samples:
        try:
            walk(json.loads(smp["out"]), [])
            n_ok += 1
        except Exception:
            continue
    keep = {k: [min(v), max(v)] for k, v in vals.items()
            if any(t in k.lower() for t in ("gfx", "clk", "power")) and "min" not in k.lower().split("/")[-1]
            and "max" not in k.lower().split("/")[-1] and "locked" not in k.lower()}
    return {"samples": len(samples), "parsed": n_ok, "source": "amd-smi metric -g 0 -c -p", "min_max": keep}


# ---------------------------------------------------------------- one workload

def kernel_rooflines(w, per_kernel, pairs):
    """Achieved rate of each attention kernel against its bound: MFMA kernels against
    the dense BF16 peak (algorithmic FLOP: 4D forward, 8D dK/dV, 2D dQ per visible pair
    per head), and the dS-stream dQ against HBM as well."""
    D = w.head_dim
    algo = {"fwd": 4 * D, "dkdv": 8 * D, "dq": 2 * D}
    out = {}
    for n, f in algo.items():
        if n in per_kernel and per_kernel[n] > 0:
            t = pairs * f / (per_kernel[n] * 1e-3) / 1e12
            out[n] = {"tflops": round(t, 2), "frac_bf16_peak": round(t / PEAK_BF16_TFLOPS, 4)}
    return out


# The FP32 transcendental pipe: a wave64 v_exp_f32 takes four issue cycles of a 16-lane
# SIMD at a quarter of the full rate, i.e. 4 lanes per cycle per SIMD: 256 CUs x 4 SIMDs x
# 4 lanes x 2.4 GHz.
PEAK_EXP_PER_S = 256 * 4 * 4 * 2.4e9


def exp_roofline(w, per_kernel, pairs, ms):
    """The exponentials of a step against the transcendental pipe: one per visible pair
    and head in the forward, in dK/dV, and in the dBias pass that forms dS again (fp32),
    none in dQ from the stored dS."""
    per = {"fwd": pairs, "dkdv": pairs}
    if w.bias is not None or getattr(w, "bias_len", 0):
        per["dbias"] = pairs
    out = {"peak_exp_per_s": PEAK_EXP_PER_S, "exp_per_step": sum(per.values())}
    rate = out["exp_per_step"] / (ms * 1e-3)
    out["step_exp_per_s"] = round(rate, 1)
    out["step_frac"] = round(rate / PEAK_EXP_PER_S, 4)
    out["kernels"] = {}
    for n, cnt in per.items():
        if n in per_kernel and per_kernel[n] > 0:
            r = cnt / (per_kernel[n] * 1e-3)
            out["kernels"][n] = {"exp_per_s": round(r, 1), "frac": round(r / PEAK_EXP_PER_S, 4)}
    return out


def ds_store_bytes(w):
    """Stored dS: one 2 KB block per (32-query tile, head, 32-key block with a visible pair)."""
    n = 0
    for b, r0, pos0, cnt in w.chunks:
        L = int(w.seq_lens[b])
        for t in range(-(-int(cnt) // 32)):
            last = int(pos0) + min(32 * (t + 1), int(cnt)) - 1
            n += -(-min(L, last + 1 if w.causal else L) // 32)
    return n * w.hq * 2048


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_workload(cp, torch, W, cfg, args, seed, headline):
    """Warmups, then `steps` timed steps of the whole hot path on one workload."""
    w = W.make_config(cfg, materialize=False)
    progress(f"config {cfg} ({w.name}): drawing inputs")
    q, k, v, do, bias = W.draw_on_device(w, seed)
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
    # With room for it, dK/dV stores dS and dQ multiplies the stored dS.
    ws_ds = 0 if args.recompute_dq else cp.workspace_size(prob, cp.OP_BWD_DS)
    use_ds = ws_ds > 0
    ws_bytes = max(ws_ds, cp.workspace_size(prob, cp.OP_BWD), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
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
        cp.bwd_prepass(prob, lay, q, o, do, lse, ws, err)
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
            # dBias forms dS again in fp32 (as the fused backward does)
            cp.bwd_dbias(prob, lay, q, k, v, bias, lse, do, ws, dbias, err)
            mark(6)

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cp.check(err)
    # the step's device memory: inputs, outputs and the backward workspace (the library
    # allocates nothing itself)
    step_peak_gib = round(torch.cuda.max_memory_allocated() / 2 ** 30, 2)
    progress(f"config {cfg}: {args.warmup} warmup steps done; timing {args.steps}")

    n_ev = len(names) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    sampler = headline.get("sampler")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    if sampler is not None:
        sampler.start()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clocks = sampler.stop() if sampler is not None else None
    cp.check(err)
    step_ms = [events[i][0].elapsed_time(events[i][-1]) for i in range(args.steps)]
    per_kernel = {n: float(np.median([events[i][j].elapsed_time(events[i][j + 1])
                                       for i in range(args.steps)])) for j, n in enumerate(names)}
    ms = float(np.median(step_ms))

    pairs = visible_pairs(w.seq_lens, w.chunks, w.causal) * w.hq
    D = w.head_dim
    flop = pairs * 14 * D
    tflops = flop / (ms * 1e-3) / 1e12
    fwd_tflops = pairs * 4 * D / (per_kernel["fwd"] * 1e-3) / 1e12
    bwd_ms = sum(per_kernel[n] for n in names[1:])
    bwd_tflops = pairs * 10 * D / (bwd_ms * 1e-3) / 1e12
    # dominant kernel: the longest attention kernel; its algorithmic FLOP per launch
    algo = {"fwd": 4 * D, "dkdv": 8 * D, "dq": 2 * D}
    dom = max((n for n in per_kernel if n in algo), key=lambda n: per_kernel[n])
    dom_flop = pairs * algo[dom]
    achieved = dom_flop / (per_kernel[dom] * 1e-3) / 1e12
    # pre-pass: reads Q, O, dO; writes Delta and the Q^T / dO^T tiles (32 queries, zero padded)
    n_tiles = int(sum(-(-int(n) // 32) for n in w.chunks[:, 3]))
    valid_q = int(sum(int(n) for n in w.chunks[:, 3]))
    pre_bytes = 3 * valid_q * w.hq * D * 2 + 4 * valid_q * w.hq + 2 * n_tiles * w.hq * 32 * D * 2
    ds_bytes = ds_store_bytes(w) if use_ds else 0
    res = {
        "value": round(tflops, 2),
        "ms_per_step": round(ms, 4),
        "ms_per_step_wall_mean": round(wall * 1e3 / args.steps, 4),
        "ms_per_step_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "seq_len": int(w.seq_lens.max()),
                   "q_rows": w.q_rows, "kv_rows": w.kv_rows, "hq": w.hq, "hkv": w.hkv,
                   "head_dim": D, "causal": bool(w.causal), "chunks": w.num_chunks,
                   "bias": bias is not None, "visible_pairs_x_heads": pairs,
                   "flop_per_step": flop, "parallelism": "none (one GPU: one rank's share)"},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(bwd_tflops, 2),
        "kernel_ms_median": {n: round(x, 4) for n, x in per_kernel.items()},
        "kernel_rooflines": kernel_rooflines(w, per_kernel, pairs),
        "exp_roofline": exp_roofline(w, per_kernel, pairs, ms),
        "prepass_gbs": round(pre_bytes / (per_kernel["prepass"] * 1e-3) / 1e9, 1),
        "dq_path": "stored dS" if use_ds else "recompute",
        "ds_bytes_per_step": ds_bytes,
        "bwd_workspace_bytes": ws_bytes,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name, dom),
                     "algorithmic_flop_per_launch": dom_flop},
    }
    if use_ds:
        dq_gb = (ds_bytes + 2 * valid_q * w.hq * D) / (per_kernel["dq"] * 1e-3) / 1e9
        res["dq_ds_gbs_algorithmic"] = round(dq_gb, 1)
    if clocks is not None:
        res["clock_power_during_timed_steps"] = clocks
    progress(f"config {cfg}: {ms:.3f} ms per step (median), {tflops:.1f} TFLOP/s")
    if headline.get("full"):
        fl = pairs * 14 * D
        res["layout_copy"] = layout_copy_rates(cp, torch)
        res["a2a_copy"] = None if args.no_a2a else a2a_copy_rates(cp, torch)
        res["ring_step"] = None if args.no_ring else ring_step_rates(cp, torch, w, q, k, v, do, bias, lay, fl)
        res["head_groups"] = None if args.no_heads else head_group_rates(cp, torch, w, q, k, v, do, bias, lay, fl)
    res["peak_mem_gib"] = round(torch.cuda.max_memory_allocated() / 2 ** 30, 2)
    res["step_peak_mem_gib"] = step_peak_gib
    if not args.no_cpu:
        progress(f"config {cfg}: CPU baseline (oracle)")
        budget = args.cpu_seconds if headline.get("full") else args.extra_cpu_seconds
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, do, bias, budget)
    del q, k, v, do, bias, o, lse, dq, dk, dv, dbias, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is designed, not built)"}))
        sys.exit(2)
    # started before anything here touches the GPU
    sampler = ClockSampler(enabled=not args.no_clock)
    import torch
    import context_causal_gqa_cpattn_amd as cp
    import workloads as W

    cp.load()
    main_res = time_workload(cp, torch, W, args.config, args, 2000 + args.config,
                             {"full": True, "sampler": sampler})
    extra = {}
    for c in [int(x) for x in args.extra.split(",") if x.strip()]:
        if c != args.config:
            extra[f"config{c}"] = time_workload(cp, torch, W, c, args, 2000 + c, {})
    line = {
        "metric": METRIC,
        "value": main_res.pop("value"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) BF16 drawn on the device, seeded",
        "timing": "median of per-step HIP-event times over the timed steps",
    }
    line.update(main_res)
    line["other_workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
