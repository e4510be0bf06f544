"""Fixed-order reductions: every output is a function of the logical problem alone.

Every sum of the path runs in an order fixed by the logical problem (sequences,
positions, heads), never by scheduling, physical row numbers or the heads of a call:
  * dK/dV of a key: the group's query heads in order, then the chunks in map order,
    then each chunk's 32-query tiles in order, in fp32 registers, one rounding;
  * dQ of a query: keys ascending in 32-key blocks (from the stored dS, or formed
    again), one rounding;
  * Delta and LSE: a fixed shuffle tree per row;
  * dBias: units of consecutive chunks (a count set by the bias size and the chunk
    count), each summed in chunk order, the units' partials added in unit order.
No kernel uses atomics for arithmetic.  Tested on the GPU:
  * one logical problem at two physical placements (rows spread out with padding
    between sequences and chunks, and packed back to back) gives the same bits for
    O, LSE, dQ, dK, dV and dBias, for both dQ paths;
  * repeated calls over a workspace filled with different junk, with other GPU work
    in between, give the same bits.
Head-group calls giving the same bits as the call over all heads are tested with
the strided views."""
import numpy as np
import pytest

import workloads as W
from harness import DeviceRun, kv_rows_of, rows_of

pytestmark = pytest.mark.gpu

CASES = [
    # (lens, hq, hkv, D, causal, bias, chunks (seq, pos0, len), q_pitch, kv_pitch)
    ([300, 77, 129], 8, 2, 128, True, False,
     [(0, 0, 40), (0, 260, 40), (1, 0, 5), (1, 72, 5), (2, 0, 9), (2, 120, 9)], 200, 320),
    ([130, 257], 8, 2, 256, True, False, [(0, 0, 9), (0, 121, 9), (1, 0, 17), (1, 240, 17)], 64, 300),
    ([200, 150], 4, 4, 64, False, False, None, 256, 224),
    ([96, 33], 16, 2, 32, True, False, [(0, 0, 6), (0, 90, 6), (1, 0, 3), (1, 30, 3)], 16, 100),
    ([64] * 8, 4, 4, 32, False, True, None, 96, 80),
    ([48] * 6, 4, 2, 64, False, True, None, 64, 64),
]
PATHS = {"stored_ds": None, "recompute": False}


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16)


def _spread(i):
    lens, hq, hkv, D, causal, bias, chunks, qp, kvp = CASES[i]
    return W.make_custom(lens=lens, hq=hq, hkv=hkv, head_dim=D, causal=causal, chunks=chunks, bias=bias,
                         q_pitch=qp, kv_pitch=kvp, seed=500 + i, pad_kv_rows=13, pad_q_rows=11)


def _run(cp, w, store_ds):
    run = DeviceRun(cp, w)
    run.forward()
    run.backward(store_ds=store_ds)
    return run


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("idx", range(len(CASES)))
def test_physical_placement_does_not_change_a_bit(gpu_lib, idx, path):
    import torch
    cp = gpu_lib
    a = _spread(idx)
    b, qi, ki = W.subset(a)  # the same sequences and chunks packed back to back
    assert b.q_rows < a.q_rows and b.kv_rows < a.kv_rows
    print(f"[case] placement {idx} {path} D={a.head_dim} bias={a.bias is not None}", flush=True)
    ra, rb = _run(cp, a, PATHS[path]), _run(cp, b, PATHS[path])
    torch.cuda.synchronize()
    tq, tk = torch.from_numpy(qi).cuda(), torch.from_numpy(ki).cuda()
    for name, x, y in (("O", ra.o[tq], rb.o), ("dQ", ra.dq[tq], rb.dq), ("dK", ra.dk[tk], rb.dk),
                       ("dV", ra.dv[tk], rb.dv)):
        assert torch.equal(_bits(x), _bits(y)), f"{name} depends on the placement"
    assert torch.equal(ra.lse[:, tq], rb.lse), "LSE depends on the placement"
    if a.bias is not None:
        assert torch.equal(ra.dbias.view(torch.int32), rb.dbias.view(torch.int32)), "dBias depends on it"


@pytest.mark.parametrize("idx", [0, 4, 5])
def test_repeated_calls_over_junk_workspace_give_the_same_bits(gpu_lib, idx):
    import torch
    cp = gpu_lib
    w = _spread(idx)
    print(f"[case] repeat {idx} D={w.head_dim} bias={w.bias is not None}", flush=True)
    run = DeviceRun(cp, w)
    run.forward()
    prob = cp.problem(run.layout, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal, w.scale,
                      w.bias_len)
    need = max(cp.workspace_size(prob, cp.OP_BWD), cp.workspace_size(prob, cp.OP_BWD_DS))
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    ki = torch.from_numpy(np.flatnonzero(kv_rows_of(w))).cuda()
    gen = torch.Generator(device="cuda").manual_seed(7)
    first = None
    for fill in ("zeros", "ones", "random"):
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(0xFF)
        else:
            ws.random_(0, 256, generator=gen)
        x = torch.randn(2048, 2048, device="cuda", generator=gen)
        for _ in range(3):
            x = x @ x.T / 2048  # other work on the stream between the calls
        o, lse, err = cp.fwd(run.q, run.k, run.v, run.layout, causal=w.causal, scale=w.scale, bias=run.bias)
        dq, dk, dv, dbias, err = cp.bwd(run.q, run.k, run.v, run.layout, o, lse, run.do, causal=w.causal,
                                        scale=w.scale, bias=run.bias, ws=ws, dev_err=err)
        torch.cuda.synchronize()
        cp.check(err)
        outs = [_bits(o[qi]), lse[:, qi].clone(), _bits(dq[qi]), _bits(dk[ki]), _bits(dv[ki])]
        if dbias is not None:
            outs.append(dbias.clone())
        if first is None:
            first = outs
        else:
            for n, (p, q) in enumerate(zip(first, outs)):
                assert torch.equal(p, q), f"output {n} changed with the workspace fill {fill}"
