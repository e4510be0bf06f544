"""HIP path vs the FP64 oracle, element by element, through the C-ABI.

Small shapes are compared in full; the five named workloads at full size are
compared on oracle-computable samples (whole sequences x KV-head groups, and
for the pair-biased workload a set of dBias positions over every row)."""
import numpy as np
import pytest

import oracle
import workloads as W
from harness import (DeviceRun, assert_close, compare, gather_rows_f64, host_f64, kv_rows_of,
                     run_oracle, rows_of)

pytestmark = pytest.mark.gpu


def _run_and_compare(gpu_lib, w, seqs=None, kv_heads=None, label="", bar="configs", store_ds=None):
    print(f"[case] {label or w.name} hq={w.hq} hkv={w.hkv} D={w.head_dim} C={w.num_chunks} "
          f"store_ds={store_ds}", flush=True)
    run = DeviceRun(gpu_lib, w)
    run.forward()
    run.backward(store_ds=store_ds)
    info, ref, _ = compare(gpu_lib, run, seqs=seqs, kv_heads=kv_heads, label=label, bar=bar)
    if w.bias is not None and run.dbias is not None and seqs is None:
        info["dbias"] = assert_close(label + "dBias", run.dbias.cpu().numpy(), ref["dbias"], bar=bar)
    return run, ref, info


# ---------------------------------------------------------------- small, full comparison

# Both dQ paths: multiplying the dS that dK/dV stored, and forming S, P and dP again.
PATHS = {"stored_ds": None, "recompute": False}


@pytest.mark.parametrize("path", PATHS)
def test_config1_full(gpu_lib, path):
    _run_and_compare(gpu_lib, W.make_config(1), label=f"cfg1 {path} ", store_ds=PATHS[path])


SWEEP = [
    # (lens, hq, hkv, D, causal, chunk spec)
    ([300], 4, 4, 128, True, None),
    ([77, 200], 8, 2, 64, True, None),
    ([130, 64, 257], 8, 1, 128, True, "pair"),
    ([512, 100], 16, 2, 256, True, "pair"),
    ([96, 33], 4, 2, 32, True, "three"),
    ([1000], 6, 3, 128, True, "pair"),
    ([200, 150], 8, 8, 64, False, None),
    ([129], 2, 1, 256, False, "three"),
    ([64, 64], 4, 1, 128, True, "tail"),
    ([300, 45], 3, 3, 256, True, None),
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
        elif spec == "tail":
            out += [(b, L - 7, 7)]
    return out


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("idx", range(len(SWEEP)))
def test_small_sweep_full(gpu_lib, idx, path):
    lens, hq, hkv, D, causal, spec = SWEEP[idx]
    w = W.make_custom(lens=lens, hq=hq, hkv=hkv, head_dim=D, causal=causal, chunks=_chunks(lens, spec),
                      seed=100 + idx, pad_kv_rows=5, pad_q_rows=3)
    _run_and_compare(gpu_lib, w, label=f"sweep{idx} {path} ", bar="pages", store_ds=PATHS[path])


@pytest.mark.parametrize("scale,D", [(-0.0625, 256), (-0.1, 128), (0.0, 256), (0.05, 128)])
def test_scale_sign_and_zero(gpu_lib, scale, D):
    """Any finite scale: the forward folds a positive scale in after the row max, takes a
    negative one as |scale| with Q negated, and a zero one as uniform weights."""
    w = W.make_custom(lens=[150, 97], hq=4, hkv=2, head_dim=D, causal=True, chunks=[(0, 0, 40), (0, 110, 40),
                      (1, 0, 97)], seed=71, scale=scale, pad_kv_rows=3, pad_q_rows=2)
    _run_and_compare(gpu_lib, w, label=f"scale {scale} D{D} ", bar="pages")


@pytest.mark.parametrize("D", [32, 64, 128])
def test_bias_small_full(gpu_lib, D):
    lens = [70, 70, 70]
    w = W.make_custom(lens=lens, hq=4, hkv=4, head_dim=D, causal=False, bias=True, seed=7 + D)
    _run_and_compare(gpu_lib, w, label=f"bias D{D} ")


def test_bias_unequal_lengths_and_partial_chunks(gpu_lib):
    lens = [90, 40, 90]
    chunks = [(0, 0, 90), (1, 3, 30), (2, 50, 40)]
    w = W.make_custom(lens=lens, hq=2, hkv=2, head_dim=32, causal=False, bias=True, chunks=chunks, seed=3)
    _run_and_compare(gpu_lib, w, label="bias ragged ")


# ---------------------------------------------------------------- named workloads, sampled

@pytest.mark.parametrize("path", PATHS)
def test_config2_sampled(gpu_lib, path):
    w = W.make_config(2)
    _run_and_compare(gpu_lib, w, seqs={0, 7}, kv_heads={0, 3, 7}, label=f"cfg2 {path} ",
                     store_ds=PATHS[path])


def test_config4_sampled_with_poisoned_padding(gpu_lib):
    w = W.make_config(4)
    order = np.argsort(w.seq_lens)
    seqs = {int(order[0]), int(order[-1]), int(order[len(order) // 2])}
    run, _, _ = _run_and_compare(gpu_lib, w, seqs=seqs, kv_heads={0, 7}, label="cfg4 ")
    # every covered row of every sequence is finite (padding NaNs never read)
    qi = np.flatnonzero(rows_of(w))
    ki = np.flatnonzero(kv_rows_of(w))
    assert np.isfinite(gather_rows_f64(gpu_lib, run.o, qi)).all()
    assert np.isfinite(gather_rows_f64(gpu_lib, run.dq, qi)).all()
    assert np.isfinite(gather_rows_f64(gpu_lib, run.dk, ki)).all()
    assert np.isfinite(gather_rows_f64(gpu_lib, run.dv, ki)).all()


@pytest.mark.slow
def test_config3_sampled(gpu_lib):
    """Full-size rank share (inputs drawn on the device), sampled oracle comparison."""
    import torch
    w = W.make_config(3, materialize=False)
    print("[case] cfg3 full size", flush=True)
    run = DeviceRun(gpu_lib, w, tensors=W.draw_on_device(w, 1003))
    run.forward()
    run.backward()
    compare(gpu_lib, run, seqs={0, 37, 63}, kv_heads={0, 7}, label="cfg3 ")
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    for t in (run.o, run.dq):
        assert bool(torch.isfinite(t.index_select(0, qi)).all())
    assert bool(torch.isfinite(run.dk).all()) and bool(torch.isfinite(run.dv).all())


def test_config5_sampled_and_dbias_positions(gpu_lib):
    w = W.make_config(5)
    print("[case] cfg5", flush=True)
    run = DeviceRun(gpu_lib, w)
    run.forward()
    run.backward()
    compare(gpu_lib, run, seqs={0, 1023}, label="cfg5 ")
    # dBias at 80 query positions, summed over all 1024 rows: four runs of positions per
    # row ([0, 24), [360, 376), [600, 616), [1000, 1024)), which cover both ends, every
    # residue mod 32 (the dBias tile height) at least twice, and four of its 32 tiles
    runs = [(0, 24), (360, 16), (600, 16), (1000, 24)]
    positions = [p for p0, n in runs for p in range(p0, p0 + n)]
    assert len({p % 32 for p in positions}) == 32
    chunks = [(i, 1024 * i + p0, p0, n) for i in range(1024) for p0, n in runs]
    import workloads
    sub, _, _ = workloads.subset(w, chunks=chunks)
    ref_b = run_oracle(sub)
    got = run.dbias.cpu().numpy()
    assert_close("cfg5 dBias", got[:, positions, :], ref_b["dbias"][:, positions, :])

    assert np.isfinite(got).all()


# ---------------------------------------------------------------- contracts

def _small_case(seed=1, **kw):
    d = dict(lens=[150, 90], hq=8, hkv=2, head_dim=128, causal=True,
             chunks=[(0, 0, 20), (0, 120, 30), (1, 10, 40)], seed=seed, pad_kv_rows=9, pad_q_rows=11)
    d.update(kw)
    return W.make_custom(**d)


def test_store_mode_ignores_nan_prefill_and_padding_untouched(gpu_lib):
    import torch
    w = _small_case()
    run = DeviceRun(gpu_lib, w)
    sentinel_q = torch.full_like(run.q, float("nan"))
    o = sentinel_q.clone()
    lse = torch.full((w.hq, w.q_rows), -123.0, device="cuda")
    run.forward(o=o, lse=lse)
    dq = sentinel_q.clone()
    dk = torch.full_like(run.k, float("nan"))
    dv = torch.full_like(run.v, float("nan"))
    run.backward(dq=dq, dk=dk, dv=dv)
    compare(gpu_lib, run)
    qm = rows_of(w)
    km = kv_rows_of(w)
    assert np.isnan(host_f64(gpu_lib, o)[~qm]).all()
    assert (lse.cpu().numpy()[:, ~qm] == -123.0).all()
    assert np.isnan(host_f64(gpu_lib, dq)[~qm]).all()
    assert np.isnan(host_f64(gpu_lib, dk)[~km]).all() and np.isnan(host_f64(gpu_lib, dv)[~km]).all()


def test_first_contribution_store_then_add(gpu_lib):
    """STORE(second chunk of each sequence) then ADD(first chunk) matches the oracle's sum."""
    w = _small_case(chunks=[(0, 0, 40), (0, 110, 40), (1, 0, 30), (1, 60, 30)])
    run = DeviceRun(gpu_lib, w)
    run.forward()
    first = w.chunks[0::2]
    second = w.chunks[1::2]
    lay_first = gpu_lib.make_layout(w.seq_offsets, w.seq_lens, first)
    lay_second = gpu_lib.make_layout(w.seq_offsets, w.seq_lens, second)
    dq, dk, dv, _, err = gpu_lib.bwd(run.q, run.k, run.v, lay_second, run.o, run.lse, run.do,
                                     causal=True, scale=w.scale)
    gpu_lib.check(err)
    _, dk, dv, _, err = gpu_lib.bwd(run.q, run.k, run.v, lay_first, run.o, run.lse, run.do,
                                    causal=True, scale=w.scale, dk=dk, dv=dv, dkv_accumulate=True)
    gpu_lib.check(err)
    sub, _, ki = W.subset(w)
    ref = run_oracle(sub)
    assert_close("ADD dK", gather_rows_f64(gpu_lib, dk, ki), ref["dk"])
    assert_close("ADD dV", gather_rows_f64(gpu_lib, dv, ki), ref["dv"])


def test_sequence_without_chunks_gets_zero_dkdv(gpu_lib):
    w = _small_case(chunks=[(0, 0, 50)])
    run = DeviceRun(gpu_lib, w)
    run.forward()
    run.backward()
    off, L = w.seq_offsets[1], w.seq_lens[1]
    assert (host_f64(gpu_lib, run.dk)[off:off + L] == 0).all()
    assert (host_f64(gpu_lib, run.dv)[off:off + L] == 0).all()


def test_empty_chunk_and_zero_length_sequence(gpu_lib):
    w = _small_case(lens=[0, 90], chunks=[(1, 0, 0), (1, 10, 40)])
    _run_and_compare(gpu_lib, w, label="empty ")


def test_stored_ds_steps_match_fused_entry_over_stale_workspace(gpu_lib):
    """The step entry points (pre-pass, dK/dV storing dS, dQ from dS) give the fused
    entry point's results bit for bit, with the workspace prefilled with NaN bytes:
    no dS block that dK/dV did not write is read."""
    import torch
    w = _small_case(seed=21, lens=[300, 77], chunks=[(0, 0, 40), (0, 230, 70), (1, 5, 33)])
    run = DeviceRun(gpu_lib, w)
    run.forward()
    prob = gpu_lib.problem(run.layout, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal,
                           w.scale, 0)
    need = gpu_lib.workspace_size(prob, gpu_lib.OP_BWD_DS)
    assert need > gpu_lib.workspace_size(prob, gpu_lib.OP_BWD)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    dq_f, dk_f, dv_f, _, err = gpu_lib.bwd(run.q, run.k, run.v, run.layout, run.o, run.lse, run.do,
                                           causal=True, scale=w.scale, ws=ws)
    gpu_lib.check(err)
    ws.fill_(0xFF)
    err = gpu_lib.new_dev_err()
    dq, dk, dv = torch.empty_like(run.q), torch.empty_like(run.k), torch.empty_like(run.v)
    gpu_lib.validate(prob, run.layout, err)
    gpu_lib.bwd_prepass(prob, run.layout, run.q, run.o, run.do, run.lse, ws, err)
    gpu_lib.bwd_dkdv_ds(prob, run.layout, run.q, run.k, run.v, None, run.lse, run.do, ws, dk, dv,
                        False, err)
    gpu_lib.bwd_dq_ds(prob, run.layout, run.k, ws, dq, err)
    torch.cuda.synchronize()
    gpu_lib.check(err)
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    ki = torch.from_numpy(np.flatnonzero(kv_rows_of(w))).cuda()
    for x, y in ((dq_f[qi], dq[qi]), (dk_f[ki], dk[ki]), (dv_f[ki], dv[ki])):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    run.dq, run.dk, run.dv = dq, dk, dv
    compare(gpu_lib, run)


def test_stored_ds_dbias_steps_match_fused_entry_over_stale_workspace(gpu_lib):
    """With a bias, the step entry points (pre-pass, dK/dV storing dS, dQ from the stored
    dS, dBias forming dS again in fp32) give the fused entry point's results bit for bit
    over a workspace prefilled with NaN bytes; dBias summed from the stored dS (chunks
    starting on and off 32-position boundaries: the block-wise and the element-wise
    sums) matches the oracle."""
    import torch
    lens = [96, 70, 64]
    chunks = [(0, 0, 96), (1, 5, 40), (2, 32, 32)]
    w = W.make_custom(lens=lens, hq=4, hkv=2, head_dim=32, causal=False, bias=True, chunks=chunks, seed=33)
    run = DeviceRun(gpu_lib, w)
    run.forward()
    prob = gpu_lib.problem(run.layout, w.q_rows, w.kv_rows, w.hq, w.hkv, w.head_dim, w.causal,
                           w.scale, w.bias_len)
    need = gpu_lib.workspace_size(prob, gpu_lib.OP_BWD_DS)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    dq_f, dk_f, dv_f, dbias_f, err = gpu_lib.bwd(run.q, run.k, run.v, run.layout, run.o, run.lse, run.do,
                                                 causal=False, scale=w.scale, bias=run.bias, ws=ws)
    gpu_lib.check(err)
    ws.fill_(0xFF)
    err = gpu_lib.new_dev_err()
    dq, dk, dv = torch.empty_like(run.q), torch.empty_like(run.k), torch.empty_like(run.v)
    dbias = torch.full_like(run.bias, float("nan"))
    gpu_lib.validate(prob, run.layout, err)
    gpu_lib.bwd_prepass(prob, run.layout, run.q, run.o, run.do, run.lse, ws, err)
    gpu_lib.bwd_dkdv_ds(prob, run.layout, run.q, run.k, run.v, run.bias, run.lse, run.do, ws, dk, dv,
                        False, err)
    gpu_lib.bwd_dq_ds(prob, run.layout, run.k, ws, dq, err)
    dbias_ds = torch.full_like(run.bias, float("nan"))
    gpu_lib.bwd_dbias_ds(prob, run.layout, ws, dbias_ds, err)
    gpu_lib.bwd_dbias(prob, run.layout, run.q, run.k, run.v, run.bias, run.lse, run.do, ws, dbias, err)
    torch.cuda.synchronize()
    gpu_lib.check(err)
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    ki = torch.from_numpy(np.flatnonzero(kv_rows_of(w))).cuda()
    for x, y in ((dq_f[qi], dq[qi]), (dk_f[ki], dk[ki]), (dv_f[ki], dv[ki])):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(dbias_f.view(torch.int32), dbias.view(torch.int32))
    run.dq, run.dk, run.dv, run.dbias = dq, dk, dv, dbias
    info, ref, _ = compare(gpu_lib, run)
    assert_close("dBias", dbias.cpu().numpy(), ref["dbias"])
    assert_close("dBias from stored dS", dbias_ds.cpu().numpy(), ref["dbias"], bar="pages")


def test_run_to_run_bitwise_identical(gpu_lib):
    import torch
    w = _small_case(seed=5)
    run = DeviceRun(gpu_lib, w)
    run.forward()
    run.backward()
    qi = torch.from_numpy(np.flatnonzero(rows_of(w))).cuda()
    ki = torch.from_numpy(np.flatnonzero(kv_rows_of(w))).cuda()
    pick = lambda: [run.o[qi], run.lse[:, qi], run.dq[qi], run.dk[ki], run.dv[ki]]
    first = [t.clone() for t in pick()]
    run.forward()
    run.backward()
    for x, y in zip(first, pick()):
        bits = torch.int32 if x.dtype == torch.float32 else torch.int16
        assert torch.equal(x.view(bits), y.view(bits))


def test_changed_inputs_in_reused_buffers(gpu_lib):
    import torch
    w1 = _small_case(seed=11)
    w2 = _small_case(seed=12)
    run = DeviceRun(gpu_lib, w1)
    run.forward()
    run.backward()
    # overwrite the same device buffers with the second workload's inputs
    for name in ("q", "k", "v", "do"):
        getattr(run, name).copy_(gpu_lib.to_device_bf16(getattr(w2, name)))
    run.w = w2
    run.forward(o=run.o, lse=run.lse)
    run.backward(dq=run.dq, dk=run.dk, dv=run.dv)
    compare(gpu_lib, run)


@pytest.mark.parametrize("bad", ["chunk_past_length", "overlapping_rows", "seq_out_of_range",
                                 "decreasing_seq", "len_over_max", "offsets_overlap"])
def test_device_promise_violation_fails_closed(gpu_lib, bad):
    import torch
    w = _small_case()
    run = DeviceRun(gpu_lib, w)
    so, sl, ch = w.seq_offsets.copy(), w.seq_lens.copy(), w.chunks.copy()
    mcl, mkl = w.max_chunk_len, w.max_kv_len
    expect = {"chunk_past_length": 0x10, "overlapping_rows": 0x08, "seq_out_of_range": 0x04,
              "decreasing_seq": 0x04, "len_over_max": 0x10, "offsets_overlap": 0x02}[bad]
    if bad == "chunk_past_length":
        ch[1, 2] = sl[0] - 10          # pos0 + len > L
    elif bad == "overlapping_rows":
        ch[2, 1] = ch[1, 1] + 5
    elif bad == "seq_out_of_range":
        ch[2, 0] = 7
    elif bad == "decreasing_seq":
        ch[0, 0], ch[2, 0] = 1, 0
    elif bad == "len_over_max":
        mcl = int(ch[:, 3].max()) - 1
    elif bad == "offsets_overlap":
        so[1] = so[0] + 10
    lay = gpu_lib.make_layout(so, sl, ch, max_chunk_len=mcl, max_kv_len=mkl)
    o = torch.full_like(run.q, 7.0)
    lse = torch.full((w.hq, w.q_rows), 7.0, device="cuda")
    _, _, err = gpu_lib.fwd(run.q, run.k, run.v, lay, causal=True, scale=w.scale, o=o, lse=lse)
    torch.cuda.synchronize()
    bits = int(err.item())
    assert bits & expect, hex(bits)
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
    dk = torch.full_like(run.k, 3.0)
    dv = torch.full_like(run.v, 3.0)
    dq = torch.full_like(run.q, 3.0)
    _, _, _, _, err = gpu_lib.bwd(run.q, run.k, run.v, lay, o, lse, run.do, causal=True,
                                  scale=w.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert int(err.item()) & expect
    assert bool((dk == 3.0).all()) and bool((dv == 3.0).all()) and bool((dq == 3.0).all())
    with pytest.raises(gpu_lib.DeviceError):
        gpu_lib.check(err)


def test_ds_blocks_promise_fails_closed(gpu_lib):
    """A dS store bound below what the chunks need is a broken promise: the validation
    step reports CPATTN_DEV_EDS_BLOCKS and nothing is written (the store sized from the
    bound would be too small for the chunks)."""
    import torch
    w = _small_case()
    run = DeviceRun(gpu_lib, w)
    run.forward()
    lay = gpu_lib.make_layout(w.seq_offsets, w.seq_lens, w.chunks, max_chunk_len=w.max_chunk_len,
                              max_kv_len=w.max_kv_len)
    true_bound = gpu_lib.ds_blocks(w.chunks, w.seq_lens, True)
    # the host copy claims that the second chunk (positions 120..149) sits 64 positions
    # earlier: a bound 2 blocks per tile too small
    host = lay.host_chunks.copy()
    assert host[1, 2] == 120
    host[1, 2] -= 64
    lay.host_chunks = host
    assert gpu_lib.ds_blocks(lay.host_chunks, lay.host_seq_lens, True) < true_bound
    o = torch.full_like(run.q, 7.0)
    lse = torch.full((w.hq, w.q_rows), 7.0, device="cuda")
    dk = torch.full_like(run.k, 3.0)
    dv = torch.full_like(run.v, 3.0)
    dq = torch.full_like(run.q, 3.0)
    _, _, _, _, err = gpu_lib.bwd(run.q, run.k, run.v, lay, run.o, run.lse, run.do, causal=True,
                                  scale=w.scale, dq=dq, dk=dk, dv=dv, store_ds=True)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x80, hex(int(err.item()))
    assert bool((dk == 3.0).all()) and bool((dv == 3.0).all()) and bool((dq == 3.0).all())
    # the exact bound passes
    lay.host_chunks = w.chunks.copy()
    _, _, _, _, err = gpu_lib.bwd(run.q, run.k, run.v, lay, run.o, run.lse, run.do, causal=True,
                                  scale=w.scale, dq=dq, dk=dk, dv=dv, store_ds=True)
    gpu_lib.check(err)


# ---------------------------------------------------------------- layout copies

@pytest.mark.parametrize("D", [128, 256])
def test_pack_unpack_bit_exact(gpu_lib, D):
    import torch
    B, H, S = 5, 6, 300
    x = W.make_bhsd(B, H, S, D, seed=D)
    lens = np.array([300, 1, 0, 257, 64], np.int32)
    offs = np.array([0, 310, 320, 320, 600], np.int32)
    thd_rows = 700
    sentinel = np.full((thd_rows, H, D), 0x7FC1, np.uint16)
    so = torch.from_numpy(offs).cuda()
    sl = torch.from_numpy(lens).cuda()
    thd = gpu_lib.to_device_bf16(sentinel)
    thd, err = gpu_lib.pack(gpu_lib.to_device_bf16(x), so, sl, thd_rows, thd=thd)
    gpu_lib.check(err)
    ref = oracle.layout.pack(x, offs, lens, sentinel)
    assert np.array_equal(gpu_lib.to_host_bits(thd), ref)
    back0 = np.full_like(x, 0x1234)
    back, err = gpu_lib.unpack(thd, so, sl, B, S, bhsd=gpu_lib.to_device_bf16(back0))
    gpu_lib.check(err)
    assert np.array_equal(gpu_lib.to_host_bits(back), oracle.layout.unpack(ref, offs, lens, back0))


def test_pack_rejects_length_over_pitch(gpu_lib):
    import torch
    x = gpu_lib.to_device_bf16(W.make_bhsd(2, 2, 16, 128, seed=1))
    so = torch.tensor([0, 16], dtype=torch.int32, device="cuda")
    sl = torch.tensor([17, 4], dtype=torch.int32, device="cuda")
    thd = torch.full((40, 2, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    _, err = gpu_lib.pack(x, so, sl, 40, thd=thd)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x40
    assert bool((thd == 5.0).all())


def test_config2_pack_unpack_roundtrip(gpu_lib):
    import torch
    B, H, S, D = 8, 32, 2048, 128
    x = torch.randn(B, H, S, D, device="cuda").to(torch.bfloat16)
    so = torch.arange(B, dtype=torch.int32, device="cuda") * S
    sl = torch.full((B,), S, dtype=torch.int32, device="cuda")
    thd, err = gpu_lib.pack(x, so, sl, B * S)
    gpu_lib.check(err)
    assert torch.equal(thd.view(B, S, H, D).permute(0, 2, 1, 3), x)
    back, err = gpu_lib.unpack(thd, so, sl, B, S)
    gpu_lib.check(err)
    assert torch.equal(back, x)
