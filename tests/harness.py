"""Shared test helpers: run the HIP path on a workload and compare it with the oracle.

Tolerances (BF16 outputs O, dQ, dK, dV and fp32 dBias, against the FP64 oracle):
  * relative L2 error of the whole compared tensor <= 1e-2;
  * per element |got - ref| <= 2e-2 wherever |ref| < 8;
  * per element |got - ref| <= one BF16 ulp of ref where |ref| >= 8: there the
    format's spacing is 2^-4 or more, so rounding even the exact value to BF16
    can cost 2^-5 = 0.031 > 2e-2 (below 8 the rounding costs at most 0.0156,
    inside the bar, so no relaxation is taken there);
  * LSE (fp32): max-abs <= 1e-3.
Every comparison prints one line (name, element count, max-abs, max-abs over
|ref| < 8, count of |ref| >= 8, rel-L2, count over the pages' own form
|err| <= 0.025 + 0.025 |ref|) so that the run's log carries the margins.

That bar is stated for the five named workloads.  Shapes outside them (the
sweeps over group sizes, head dims and chunk maps) use the full-tensor bar the
page "Optimize context parallel attention layouts and gradient accumulation"
applies in "Related optimization work" (head-partition run): per element
|err| <= 0.025 + 0.025 |ref| and relative RMS error < 0.02.
"""
from __future__ import annotations

import numpy as np

import workloads as W

ATOL = 2e-2
REL_L2 = 1e-2
LSE_ATOL = 1e-3
BIG = 8.0

# Every margin line of this process, for the end-of-run summary (tests/conftest.py).
MARGINS: list = []


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 2.0 ** (e - 7)


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, atol=ATOL, rel_l2=REL_L2,
                 bar: str = "configs"):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    assert got.shape == ref.shape, name
    assert np.isfinite(ref).all(), f"{name}: reference has non-finite values (selection bug)"
    assert np.isfinite(got).all(), f"{name}: {np.count_nonzero(~np.isfinite(got))} non-finite values"
    if got.size == 0:
        return {"n": 0}
    err = np.abs(got - ref)
    small = np.abs(ref) < BIG
    max_small = float(err[small].max()) if small.any() else 0.0
    big_bad = int(np.count_nonzero(err[~small] > np.maximum(atol, bf16_ulp(ref[~small]))))
    nrm = np.linalg.norm(ref)
    rl2 = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    info = {"n": got.size, "max_abs": float(err.max()), "max_abs_small": max_small,
            "n_big": int((~small).sum()),
            "big_over_ulp": big_bad, "rel_l2": rl2,
            "pages_form_fail": int(np.count_nonzero(err > 0.025 + 0.025 * np.abs(ref)))}
    line = (f"{name} bar={bar} n={info['n']} max_abs={info['max_abs']:.5f} "
            f"max_abs_small={max_small:.5f} n_big={info['n_big']} big_over_ulp={big_bad} "
            f"rel_l2={rl2:.5f} pages_form_fail={info['pages_form_fail']}")
    MARGINS.append((name, bar, max_small, rl2, line))
    print("[margin] " + line, flush=True)
    if bar == "pages":
        assert info["pages_form_fail"] == 0, f"{name}: elements over 0.025+0.025|ref| ({info})"
        assert rl2 < 0.02, f"{name}: relative RMS {rl2} >= 0.02 ({info})"
        return info
    assert max_small <= atol, f"{name}: max abs err {max_small} > {atol} ({info})"
    assert big_bad == 0, f"{name}: {big_bad} large-magnitude elements off by > 1 ulp ({info})"
    assert rl2 <= rel_l2, f"{name}: rel L2 {rl2} > {rel_l2} ({info})"
    return info


def assert_lse_close(name, got, ref, atol=LSE_ATOL):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    assert np.isfinite(got).all(), f"{name}: non-finite LSE"
    e = float(np.abs(got - ref).max()) if got.size else 0.0
    line = f"{name} n={got.size} lse_max_abs={e:.2e}"
    MARGINS.append((name, "lse", e, 0.0, line))
    print("[margin] " + line, flush=True)
    assert e <= atol, f"{name}: LSE max abs err {e} > {atol}"
    return e


class DeviceRun:
    """Device copies of a workload's inputs and the HIP path's outputs."""

    def __init__(self, cp, w: W.Workload, device="cuda", tensors=None):
        import torch
        self.cp, self.w, self.torch = cp, w, torch
        if tensors is not None:  # inputs already on the device (drawn there)
            self.q, self.k, self.v, self.do, self.bias = tensors
        else:
            self.q = cp.to_device_bf16(w.q, device)
            self.k = cp.to_device_bf16(w.k, device)
            self.v = cp.to_device_bf16(w.v, device)
            self.do = cp.to_device_bf16(w.do, device)
            self.bias = None if w.bias is None else torch.from_numpy(w.bias).to(device)
        self.layout = cp.make_layout(w.seq_offsets, w.seq_lens, w.chunks, device,
                                     max_chunk_len=w.max_chunk_len, max_kv_len=w.max_kv_len)

    def forward(self, **kw):
        self.o, self.lse, err = self.cp.fwd(self.q, self.k, self.v, self.layout, causal=self.w.causal,
                                            scale=self.w.scale, bias=self.bias, **kw)
        self.cp.check(err)
        return self.o, self.lse

    def backward(self, **kw):
        self.dq, self.dk, self.dv, self.dbias, err = self.cp.bwd(
            self.q, self.k, self.v, self.layout, self.o, self.lse, self.do, causal=self.w.causal,
            scale=self.w.scale, bias=self.bias, **kw)
        self.cp.check(err)
        return self.dq, self.dk, self.dv, self.dbias


def host_f64(cp, t) -> np.ndarray:
    return W.f64_from_bf16_bits(cp.to_host_bits(t))


def gather_rows_f64(cp, t, index: np.ndarray) -> np.ndarray:
    """Rows `index` of a device BF16 tensor, gathered on the GPU, as float64."""
    import torch
    idx = torch.from_numpy(np.asarray(index, np.int64)).to(t.device)
    return host_f64(cp, t.index_select(0, idx))


def oracle_inputs(w: W.Workload):
    return (W.f64_from_bf16_bits(w.q), W.f64_from_bf16_bits(w.k), W.f64_from_bf16_bits(w.v),
            W.f64_from_bf16_bits(w.do), None if w.bias is None else w.bias.astype(np.float64))


def run_oracle(w: W.Workload, kv_heads=None):
    import oracle
    q, k, v, do, bias = oracle_inputs(w)
    sel = None if kv_heads is None else (None, set(kv_heads))
    return oracle.attention(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale,
                            bias=bias, do=do, select=sel)


def rows_of(w: W.Workload, seqs=None):
    """Q rows covered by chunks of the given sequences (all if None)."""
    m = np.zeros(w.q_rows, bool)
    for s, r0, _, n in w.chunks:
        if seqs is None or s in seqs:
            m[r0:r0 + n] = True
    return m


def kv_rows_of(w: W.Workload, seqs=None):
    m = np.zeros(w.kv_rows, bool)
    for b, (o, L) in enumerate(zip(w.seq_offsets, w.seq_lens)):
        if seqs is None or b in seqs:
            m[o:o + L] = True
    return m


def compare(cp, run: DeviceRun, seqs=None, kv_heads=None, chunks=None, check_bwd=True, label="",
            bar: str = "configs"):
    """Run the oracle on a sampled sub-workload and compare the GPU rows that match it."""
    w = run.w
    sub, qi, ki = W.subset(w, seqs=seqs, chunks=chunks)
    if sub.q is None:  # inputs live on the device only: copy the sampled rows back
        import torch
        tq = torch.from_numpy(qi).to(run.q.device)
        tk = torch.from_numpy(ki).to(run.k.device)
        sub.q = cp.to_host_bits(run.q.index_select(0, tq))
        sub.do = cp.to_host_bits(run.do.index_select(0, tq))
        sub.k = cp.to_host_bits(run.k.index_select(0, tk))
        sub.v = cp.to_host_bits(run.v.index_select(0, tk))
        sub.bias = None if run.bias is None else run.bias.cpu().numpy()
    ref = run_oracle(sub, kv_heads)
    G = w.hq // w.hkv
    kvh = list(range(w.hkv)) if kv_heads is None else sorted(kv_heads)
    heads = [h for g in kvh for h in range(g * G, g * G + G)]
    out = {}
    out["o"] = assert_close(label + "O", gather_rows_f64(cp, run.o, qi)[:, heads], ref["o"][:, heads], bar=bar)
    lse = run.lse[:, __import__("torch").from_numpy(qi).to(run.lse.device)].cpu().numpy()
    out["lse"] = assert_lse_close(label + "LSE", lse[heads], ref["lse"][heads])
    if check_bwd:
        out["dq"] = assert_close(label + "dQ", gather_rows_f64(cp, run.dq, qi)[:, heads], ref["dq"][:, heads], bar=bar)
        out["dk"] = assert_close(label + "dK", gather_rows_f64(cp, run.dk, ki)[:, kvh], ref["dk"][:, kvh], bar=bar)
        out["dv"] = assert_close(label + "dV", gather_rows_f64(cp, run.dv, ki)[:, kvh], ref["dv"][:, kvh], bar=bar)
    return out, ref, sub
