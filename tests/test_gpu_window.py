"""Key-window forward, merge and key-window backward (the ring-step path) vs the FP64 oracle.

A ring step attends to one block of K/V positions.  The HIP path's partial results
over disjoint windows are checked against the window oracle, merged on the GPU
and checked against the full-attention oracle, and the window backward's shares
(dQ added over the windows, dK/dV stored per window) against the full gradients."""
import numpy as np
import pytest

import oracle
import oracle.window as OW
import workloads as W
from harness import DeviceRun, assert_close, compare, host_f64, rows_of

pytestmark = pytest.mark.gpu

BIGW = 1 << 30

CASES = [
    # (lens, hq, hkv, D, causal, bias, chunk spec, windows)
    ([300, 77], 8, 2, 128, True, False, "pair", [(0, 64), (64, 200), (200, BIGW)]),
    ([130, 257], 8, 1, 256, True, False, "pair", [(0, 100), (100, 131), (131, BIGW)]),
    ([200, 150], 8, 8, 64, False, False, None, [(0, 70), (70, 71), (71, BIGW)]),
    ([96, 33], 4, 2, 32, True, False, "three", [(0, 40), (40, BIGW)]),
    ([64, 48], 4, 4, 64, False, True, None, [(0, 30), (30, BIGW)]),
]


def _chunks(lens, spec):
    if spec is None:
        return None
    out = []
    for b, L in enumerate(lens):
        c = max(1, L // 16)
        if spec == "pair":
            out += [(b, 0, c), (b, L - c, c)]
        elif spec == "three":
            out += [(b, 0, min(L, 5)), (b, L // 3, min(L - L // 3, 37)), (b, L - 1, 1)]
    return out


def _workload(i):
    lens, hq, hkv, D, causal, bias, spec, windows = CASES[i]
    w = W.make_custom(lens=lens, hq=hq, hkv=hkv, head_dim=D, causal=causal, chunks=_chunks(lens, spec),
                      bias=bias, seed=300 + i, pad_kv_rows=5, pad_q_rows=3)
    return w, windows


def _inputs(cp, w):
    import torch
    q, k, v, do = (cp.to_device_bf16(x) for x in (w.q, w.k, w.v, w.do))
    bias = None if w.bias is None else torch.from_numpy(w.bias).cuda()
    lay = cp.make_layout(w.seq_offsets, w.seq_lens, w.chunks)
    return q, k, v, do, bias, lay


def _f64(w):
    return (W.f64_from_bf16_bits(w.q), W.f64_from_bf16_bits(w.k), W.f64_from_bf16_bits(w.v),
            W.f64_from_bf16_bits(w.do), None if w.bias is None else w.bias.astype(np.float64))


def _assert_lse(name, got, ref):
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{name}: -inf rows differ"
    e = float(np.abs(got[~inf_ref] - ref[~inf_ref]).max()) if (~inf_ref).any() else 0.0
    assert e <= 1e-3, f"{name}: LSE max abs err {e}"


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_window_forward_and_merge(gpu_lib, idx):
    import torch
    cp = gpu_lib
    w, windows = _workload(idx)
    print(f"[case] window fwd {idx} D={w.head_dim} windows={windows}", flush=True)
    q, k, v, do, bias, lay = _inputs(cp, w)
    qf, kf, vf, dof, bf = _f64(w)
    rows = w.q_valid_rows()
    run_o, run_l = None, None
    for (lo, hi) in windows:
        o, lse, err = cp.fwd_window(q, k, v, lay, lo, hi, causal=w.causal, scale=w.scale, bias=bias)
        torch.cuda.synchronize()
        cp.check(err)
        ref = OW.attention_window(qf, kf, vf, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale,
                                  (lo, hi), bias=bf)
        assert_close(f"O[{lo},{hi})", host_f64(cp, o)[rows], ref["o"][rows], bar="pages")
        _assert_lse(f"LSE[{lo},{hi})", lse.cpu().numpy()[:, rows], ref["lse"][:, rows])
        if run_o is None:
            run_o, run_l = o, lse
        else:
            prob = cp.problem(lay, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale,
                              w.bias_len)
            err = cp.new_dev_err()
            cp.merge(prob, lay, run_o, run_l, o, lse, dev_err=err)  # in place into the running result
            torch.cuda.synchronize()
            cp.check(err)
    full = oracle.attention(qf, kf, vf, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale, bias=bf)
    assert_close("merged O", host_f64(cp, run_o)[rows], full["o"][rows], bar="pages")
    _assert_lse("merged LSE", run_l.cpu().numpy()[:, rows], full["lse"][:, rows])


@pytest.mark.parametrize("store_ds", [False, True], ids=["recompute", "stored_ds"])
@pytest.mark.parametrize("idx", range(len(CASES)))
def test_window_backward_shares_sum_to_full_gradients(gpu_lib, idx, store_ds):
    import torch
    cp = gpu_lib
    w, windows = _workload(idx)
    print(f"[case] window bwd {idx} D={w.head_dim} windows={windows} store_ds={store_ds}", flush=True)
    q, k, v, do, bias, lay = _inputs(cp, w)
    o, lse, err = cp.fwd(q, k, v, lay, causal=w.causal, scale=w.scale, bias=bias)
    dq = torch.empty_like(q)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    ws = None
    for i, (lo, hi) in enumerate(windows):
        _, _, _, ws, err2 = cp.bwd_window(q, k, v, lay, o, lse, do, lo, hi, causal=w.causal, scale=w.scale,
                                          bias=bias, prepass=(i == 0), dq=dq, dq_accumulate=(i > 0),
                                          dk=dk, dv=dv, ws=ws, dev_err=err, store_ds=store_ds)
    torch.cuda.synchronize()
    cp.check(err)
    qf, kf, vf, dof, bf = _f64(w)
    full = oracle.attention(qf, kf, vf, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale, bias=bf,
                            do=dof)
    rows, kr = w.q_valid_rows(), w.kv_valid_rows()
    assert_close("dQ (sum over windows)", host_f64(cp, dq)[rows], full["dq"][rows], bar="pages")
    assert_close("dK (per window)", host_f64(cp, dk)[kr], full["dk"][kr], bar="pages")
    assert_close("dV (per window)", host_f64(cp, dv)[kr], full["dv"][kr], bar="pages")
    # rows outside every sequence are never written
    assert np.isnan(host_f64(cp, dk)[~kr]).all() and np.isnan(host_f64(cp, dv)[~kr]).all()


@pytest.mark.parametrize("store_ds", [False, True], ids=["recompute", "stored_ds"])
def test_window_backward_matches_window_oracle_shares(gpu_lib, store_ds):
    """One window's dK/dV and dQ share against the window oracle directly."""
    import torch
    cp = gpu_lib
    print(f"[case] window bwd share store_ds={store_ds}", flush=True)
    w, _ = _workload(0)
    lo, hi = 64, 200
    q, k, v, do, bias, lay = _inputs(cp, w)
    o, lse, err = cp.fwd(q, k, v, lay, causal=True, scale=w.scale)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    dq, _, _, _, err = cp.bwd_window(q, k, v, lay, o, lse, do, lo, hi, causal=True, scale=w.scale,
                                     dk=dk, dv=dv, dev_err=err, store_ds=store_ds)
    torch.cuda.synchronize()
    cp.check(err)
    qf, kf, vf, dof, _ = _f64(w)
    full = oracle.attention(qf, kf, vf, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale)
    ref = OW.backward_window(qf, kf, vf, dof, full["o"], full["lse"], w.seq_offsets, w.seq_lens, w.chunks,
                             True, w.scale, (lo, hi))
    rows = w.q_valid_rows()
    assert_close("dQ share", host_f64(cp, dq)[rows], ref["dq"][rows], bar="pages")
    m = ~np.isnan(ref["dk"][:, 0, 0])
    assert_close("dK share", host_f64(cp, dk)[m], ref["dk"][m], bar="pages")
    assert_close("dV share", host_f64(cp, dv)[m], ref["dv"][m], bar="pages")
    assert np.isnan(host_f64(cp, dk)[~m]).all()


@pytest.mark.slow
def test_config3_ring_of_eight_windows_sampled(gpu_lib):
    """The full-size rank share run as a ring of eight equal key windows: window forwards
    merged on the GPU, window backwards with the dS store and dQ added over the windows,
    checked on sampled sequences and KV heads against the full-attention oracle."""
    import torch
    cp = gpu_lib
    w = W.make_config(3, materialize=False)
    print("[case] cfg3 ring of 8 key windows", flush=True)
    run = DeviceRun(cp, w, tensors=W.draw_on_device(w, 1013))
    lay = run.layout
    n = 8
    Lmax = int(max(w.seq_lens))
    edges = [Lmax * i // n for i in range(n)] + [BIGW]
    prob = cp.problem(lay, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale, w.bias_len)
    o = torch.empty_like(run.q)
    lse = torch.empty((w.hq, w.q_rows), dtype=torch.float32, device="cuda")
    o_w, lse_w = torch.empty_like(o), torch.empty_like(lse)
    err = cp.new_dev_err()
    for i in range(n):
        first = i == 0
        cp.fwd_window(run.q, run.k, run.v, lay, edges[i], edges[i + 1], causal=True, scale=w.scale,
                      o=o if first else o_w, lse=lse if first else lse_w, dev_err=err)
        if not first:
            cp.merge(prob, lay, o, lse, o_w, lse_w, dev_err=err)
    dq, dk, dv = torch.empty_like(run.q), torch.empty_like(run.k), torch.empty_like(run.v)
    ws = None
    for i in range(n):
        _, _, _, ws, _ = cp.bwd_window(run.q, run.k, run.v, lay, o, lse, run.do, edges[i], edges[i + 1],
                                       causal=True, scale=w.scale, prepass=(i == 0), dq=dq,
                                       dq_accumulate=(i > 0), dk=dk, dv=dv, ws=ws, dev_err=err,
                                       store_ds=True)
    torch.cuda.synchronize()
    cp.check(err)
    assert ws.numel() >= cp.workspace_size(prob, cp.OP_BWD_DS)
    del ws
    run.o, run.lse, run.dq, run.dk, run.dv = o, lse, dq, dk, dv
    compare(cp, run, seqs={0, 63}, kv_heads={0, 7}, label="cfg3 ring ", bar="pages")
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    for t in (o, dq):
        assert bool(torch.isfinite(t.index_select(0, qi)).all())
    assert bool(torch.isfinite(dk).all()) and bool(torch.isfinite(dv).all())
