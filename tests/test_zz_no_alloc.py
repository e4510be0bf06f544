"""The backward without a workspace argument (cpattn_bwd_noalloc), through the C-ABI.

Its workspace is the library's static scratch array; its results must be those of
cpattn_bwd (same kernels) with a caller-provided workspace of the size it picks:
the stored-dS backward when that fits in the array, else the one that forms dS again.
Checked bit for bit on consecutive calls (a larger problem, then a smaller one, so the
second runs over what the first left in the array), on both paths and with a bias; a
problem too large for the array is rejected before anything is enqueued; the first
call is also compared with the FP64 oracle."""
import numpy as np
import pytest

import workloads as W
from harness import DeviceRun, compare, kv_rows_of, rows_of

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _noalloc_vs_bwd(cp, w, expect_path):
    import torch
    print(f"[case] noalloc {w.name} lens={list(w.seq_lens)} hq={w.hq} D={w.head_dim} "
          f"bias={w.bias is not None} expect={expect_path}", flush=True)
    run = DeviceRun(cp, w)
    run.forward()
    prob = cp.problem(run.layout, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale,
                      w.bias_len)
    need_ds = cp.workspace_size(prob, cp.OP_BWD_DS)
    need_rc = cp.workspace_size(prob, cp.OP_BWD)
    path = "stored_ds" if 0 < need_ds <= cp.NOALLOC_SCRATCH_BYTES else "recompute"
    assert path == expect_path, (need_ds, need_rc)
    ws = torch.full((need_ds if path == "stored_ds" else need_rc,), 0xFF, dtype=torch.uint8, device="cuda")
    # reference: cpattn_bwd with a workspace of the size the no-allocation call picks
    dq_r, dk_r, dv_r, db_r, err = cp.bwd(run.q, run.k, run.v, run.layout, run.o, run.lse, run.do,
                                         causal=w.causal, scale=w.scale, bias=run.bias, ws=ws)
    cp.check(err)
    dq = torch.full_like(run.q, float("nan"))
    dk = torch.full_like(run.k, float("nan"))
    dv = torch.full_like(run.v, float("nan"))
    db = None if run.bias is None else torch.full_like(run.bias, float("nan"))
    err = cp.new_dev_err()
    cp.bwd_noalloc(run.q, run.k, run.v, run.layout, run.o, run.lse, run.do, dq, dk, dv, causal=w.causal,
                   scale=w.scale, bias=run.bias, dbias=db, dev_err=err)
    torch.cuda.synchronize()
    cp.check(err)
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    ki = torch.from_numpy(np.flatnonzero(kv_rows_of(w))).cuda()
    for name, x, y in (("dq", dq_r[qi], dq[qi]), ("dk", dk_r[ki], dk[ki]), ("dv", dv_r[ki], dv[ki])):
        assert torch.equal(_bits(x), _bits(y)), name
    if db is not None:
        assert torch.equal(_bits(db_r), _bits(db)), "dbias"
    run.dq, run.dk, run.dv, run.dbias = dq, dk, dv, db
    return run


def test_noalloc_matches_bwd_on_consecutive_calls(gpu_lib):
    cp = gpu_lib
    big = W.make_custom(lens=[300, 77, 129], hq=8, hkv=2, head_dim=128, causal=True,
                        chunks=[(0, 0, 40), (0, 260, 40), (1, 0, 77), (2, 0, 9), (2, 120, 9)],
                        seed=901, pad_kv_rows=5, pad_q_rows=3)
    run = _noalloc_vs_bwd(cp, big, "stored_ds")
    compare(cp, run, label="noalloc ")  # and the first call against the oracle
    small = W.make_custom(lens=[50, 20], hq=4, hkv=4, head_dim=64, causal=True, seed=902)
    _noalloc_vs_bwd(cp, small, "stored_ds")
    # dS store beyond the array (2048 query rows x 4 heads x 8192 keys x 2 bytes), the
    # recompute path's workspace well inside it
    long = W.make_custom(lens=[8192], hq=4, hkv=1, head_dim=64, causal=True,
                         chunks=[(0, 0, 1024), (0, 7168, 1024)], seed=903)
    _noalloc_vs_bwd(cp, long, "recompute")
    biased = W.make_custom(lens=[64] * 6, hq=4, hkv=4, head_dim=32, causal=False, bias=True, seed=904)
    _noalloc_vs_bwd(cp, biased, "stored_ds")


def test_noalloc_rejects_a_problem_beyond_the_scratch(gpu_lib):
    import torch
    cp = gpu_lib
    # the recompute workspace alone (Delta and the transposed Q and dO tiles) is about
    # 2 x q_rows x hq x D x 2 bytes: 2 x 8192 x 16 x 128 x 2 = 64 MiB, plus Delta
    lens = [8192]
    w = W.make_custom(lens=lens, hq=16, hkv=4, head_dim=128, causal=True, seed=905, materialize=False)
    lay = cp.make_layout(w.seq_offsets, w.seq_lens, w.chunks, "cuda")
    prob = cp.problem(lay, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale, 0)
    assert cp.workspace_size(prob, cp.OP_BWD) > cp.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((w.q_rows, w.hq, w.head_dim), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((w.kv_rows, w.hkv, w.head_dim), dtype=torch.bfloat16, device="cuda")
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros((w.hq, w.q_rows), dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, 3.0)
    dk, dv = torch.full_like(k, 3.0), torch.full_like(k, 3.0)
    err = cp.new_dev_err()
    with pytest.raises(cp.CpattnError) as e:
        cp.bwd_noalloc(q, k, k.clone(), lay, o, lse, do, dq, dk, dv, causal=True, dev_err=err)
    assert e.value.status == cp.EUNSUPPORTED and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((dq == 3.0).all()) and bool((dk == 3.0).all()) and bool((dv == 3.0).all())
    assert int(err.item()) == 0
