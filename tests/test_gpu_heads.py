"""Head-group calls on strided views (head partitioning) vs the call over all heads.

A caller that splits the heads of one layer into groups runs the forward and the
backward once per group, on views of its full-size tensors: Q, O, dO, dQ are the
group's query heads of [rows, Hq, D] tensors (row pitch Hq heads), K, V, dK, dV the
matching KV heads of [rows, Hkv, D], LSE and dBias contiguous head slices.  One
workspace, sized for a group, serves every group call.  Every head's arithmetic is
the same in both forms (dBias too: its row units do not depend on the heads of a
call), so O, LSE, dQ, dK, dV and dBias must agree bit for bit with the call over all
heads; the full call itself is checked against the FP64 oracle in the parity tests,
and once more here."""
import numpy as np
import pytest

import workloads as W
from harness import DeviceRun, compare, kv_rows_of, rows_of

pytestmark = pytest.mark.gpu

CASES = [
    # (lens, hq, hkv, D, causal, bias, chunks, head group sizes)
    ([300, 77], 16, 4, 128, True, False, [(0, 0, 40), (0, 260, 40), (1, 0, 5), (1, 72, 5)], [8, 4]),
    ([130, 257], 8, 2, 256, True, False, [(0, 0, 9), (0, 121, 9), (1, 0, 17), (1, 240, 17)], [4]),
    ([200, 150], 8, 8, 64, False, False, None, [4, 1]),
    ([96, 33], 16, 2, 32, True, False, [(0, 0, 6), (0, 90, 6), (1, 0, 3), (1, 30, 3)], [8]),
    ([64, 48], 4, 4, 32, False, True, None, [2, 1]),
]


def _workload(i):
    lens, hq, hkv, D, causal, bias, chunks, groups = CASES[i]
    w = W.make_custom(lens=lens, hq=hq, hkv=hkv, head_dim=D, causal=causal, chunks=chunks, bias=bias,
                      seed=400 + i, pad_kv_rows=7, pad_q_rows=5)
    return w, groups


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16)


def _run_groups(cp, run, Hg, ws=None):
    """Forward and backward per group of Hg query heads into NaN-filled full tensors."""
    import torch
    w = run.w
    G = w.hq // w.hkv
    nan_q = torch.full_like(run.q, float("nan"))
    nan_k = torch.full_like(run.k, float("nan"))
    o, dq, dk, dv = nan_q.clone(), nan_q.clone(), nan_k.clone(), nan_k.clone()
    lse = torch.full((w.hq, w.q_rows), float("nan"), device=run.q.device)
    dbias = None if run.bias is None else torch.full_like(run.bias, float("nan"))
    err = cp.new_dev_err()
    for h0 in range(0, w.hq, Hg):
        g0, hkv_g = h0 // G, Hg // G
        hs, gs = slice(h0, h0 + Hg), slice(g0, g0 + hkv_g)
        qv, kv, vv, dov = run.q[:, hs], run.k[:, gs], run.v[:, gs], run.do[:, hs]
        bv = None if run.bias is None else run.bias[hs]
        if Hg < w.hq:
            assert not qv.is_contiguous() and cp.head_pitch(qv) == w.hq
        cp.fwd(qv, kv, vv, run.layout, causal=w.causal, scale=w.scale, bias=bv, o=o[:, hs], lse=lse[hs],
               dev_err=err)
        _, _, _, _, err = cp.bwd(qv, kv, vv, run.layout, o[:, hs], lse[hs], dov, causal=w.causal,
                                 scale=w.scale, bias=bv, dq=dq[:, hs], dk=dk[:, gs], dv=dv[:, gs],
                                 dbias=None if dbias is None else dbias[hs], ws=ws, dev_err=err)
    torch.cuda.synchronize()
    cp.check(err)
    return o, lse, dq, dk, dv, dbias


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_head_group_views_match_the_call_over_all_heads(gpu_lib, idx):
    import torch
    cp = gpu_lib
    w, groups = _workload(idx)
    print(f"[case] heads {idx} hq={w.hq} hkv={w.hkv} D={w.head_dim} groups={groups}", flush=True)
    run = DeviceRun(cp, w)
    run.forward()
    run.backward()
    torch.cuda.synchronize()
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    ki = torch.from_numpy(np.flatnonzero(kv_rows_of(w))).cuda()
    pad_q = torch.from_numpy(np.flatnonzero(~rows_of(w))).cuda()
    pad_k = torch.from_numpy(np.flatnonzero(~kv_rows_of(w))).cuda()
    for Hg in groups:
        # one workspace for every group call, sized for a group (stored-dS backward when
        # the head dim allows it) and prefilled with NaN bytes
        G = w.hq // w.hkv
        prob_g = cp.problem(run.layout, w.q_rows, w.kv_rows, Hg, Hg // G, w.head_dim, w.causal, w.scale,
                            w.bias_len, w.hq, w.hkv)
        need = max(cp.workspace_size(prob_g, cp.OP_BWD), cp.workspace_size(prob_g, cp.OP_BWD_DS))
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        o, lse, dq, dk, dv, dbias = _run_groups(cp, run, Hg, ws)
        for name, full, part, idx_rows in (("O", run.o, o, qi), ("dQ", run.dq, dq, qi), ("dK", run.dk, dk, ki),
                                           ("dV", run.dv, dv, ki)):
            assert torch.equal(_bits(full[idx_rows]), _bits(part[idx_rows])), f"{name} differs at Hg={Hg}"
        assert torch.equal(run.lse[:, qi], lse[:, qi]), f"LSE differs at Hg={Hg}"
        # rows outside every chunk / sequence stay untouched
        assert torch.isnan(o[pad_q].float()).all() and torch.isnan(dq[pad_q].float()).all()
        assert torch.isnan(dk[pad_k].float()).all() and torch.isnan(dv[pad_k].float()).all()
        if dbias is not None:
            assert torch.equal(dbias.view(torch.int32), run.dbias.view(torch.int32)), f"dBias differs at Hg={Hg}"
    # the full call (and so every head-group form) against the oracle
    compare(cp, run, bar="pages")


def test_group_calls_write_only_their_heads(gpu_lib):
    """One group's forward and backward leave every other head of the full tensors as
    it was, and a K/V pair packed in one [rows, 2 Hkv, D] tensor works as two views."""
    import torch
    cp = gpu_lib
    w, _ = _workload(0)
    run = DeviceRun(cp, w)
    run.forward()
    run.backward()
    G = w.hq // w.hkv
    h0, Hg = 8, 4
    g0, hkv_g = h0 // G, Hg // G
    hs, gs = slice(h0, h0 + Hg), slice(g0, g0 + hkv_g)
    kv = torch.cat([run.k, run.v], dim=1)            # [rows, 2 Hkv, D]: K heads then V heads
    dkv = torch.full_like(kv, float("nan"))
    o = torch.full_like(run.q, float("nan"))
    dq = torch.full_like(run.q, float("nan"))
    lse = torch.full((w.hq, w.q_rows), float("nan"), device="cuda")
    kview, vview = kv[:, g0:g0 + hkv_g], kv[:, w.hkv + g0:w.hkv + g0 + hkv_g]
    assert cp.head_pitch(kview) == 2 * w.hkv
    cp.fwd(run.q[:, hs], kview, vview, run.layout, causal=w.causal, scale=w.scale, o=o[:, hs], lse=lse[hs])
    _, _, _, _, err = cp.bwd(run.q[:, hs], kview, vview, run.layout, o[:, hs], lse[hs], run.do[:, hs],
                             causal=w.causal, scale=w.scale, dq=dq[:, hs],
                             dk=dkv[:, g0:g0 + hkv_g], dv=dkv[:, w.hkv + g0:w.hkv + g0 + hkv_g])
    torch.cuda.synchronize()
    cp.check(err)
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    ki = torch.from_numpy(np.flatnonzero(kv_rows_of(w))).cuda()
    assert torch.equal(_bits(o[qi][:, hs]), _bits(run.o[qi][:, hs]))
    assert torch.equal(_bits(dq[qi][:, hs]), _bits(run.dq[qi][:, hs]))
    assert torch.equal(lse[hs][:, qi], run.lse[hs][:, qi])
    assert torch.equal(_bits(dkv[ki][:, g0:g0 + hkv_g]), _bits(run.dk[ki][:, gs]))
    assert torch.equal(_bits(dkv[ki][:, w.hkv + g0:w.hkv + g0 + hkv_g]), _bits(run.dv[ki][:, gs]))
    other_q = [h for h in range(w.hq) if not h0 <= h < h0 + Hg]
    other_kv = [h for h in range(2 * w.hkv) if h not in (g0, w.hkv + g0)]
    assert torch.isnan(o[:, other_q].float()).all() and torch.isnan(dq[:, other_q].float()).all()
    assert torch.isnan(lse[other_q]).all()
    assert torch.isnan(dkv[:, other_kv].float()).all()
