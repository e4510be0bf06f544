"""Pins for the FP64 oracle: closed forms, invariants, brute force, finite
differences and a textbook library routine.  None of these re-types the
oracle's own formula; each would catch a dropped term, a wrong sign or index,
or a transposed operand somewhere in it (see the planted-mistake tests at the
bottom, which mutate the oracle on the CPU and check that a pin fails)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle.softmax_attention as OA
from oracle import attention as run_oracle
from oracle import layout as OL
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _f64(w):
    return (W.f64_from_bf16_bits(w.q), W.f64_from_bf16_bits(w.k), W.f64_from_bf16_bits(w.v),
            W.f64_from_bf16_bits(w.do), None if w.bias is None else w.bias.astype(np.float64))


def _run(w, q=None, k=None, v=None, do=None, bias=None, chunks=None, with_grad=True):
    q0, k0, v0, do0, b0 = _f64(w)
    q = q0 if q is None else q
    k = k0 if k is None else k
    v = v0 if v is None else v
    do = do0 if do is None else do
    bias = b0 if bias is None else bias
    return run_oracle(q, k, v, w.seq_offsets, w.seq_lens, w.chunks if chunks is None else chunks,
                      w.causal, w.scale, bias=bias, do=do if with_grad else None)


def _tiny(causal=True, bias=False, chunked=True, hq=4, hkv=2, D=3, lens=(5, 7), seed=7):
    lens = list(lens)
    if chunked:
        chunks = []
        for b, L in enumerate(lens):
            chunks.append((b, 0, 2))
            chunks.append((b, L - 2, 2))
    else:
        chunks = None
    return W.make_custom(lens=lens, hq=hq, hkv=hkv, head_dim=D, causal=causal, chunks=chunks,
                         bias=bias, seed=seed, pad_kv_rows=2, pad_q_rows=1, poison_padding=False)


# ---------------------------------------------------------------- golden

def test_golden_hand_worked():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q = np.asarray(c["q"], np.float64)[:, None, :]
        k = np.asarray(c["k"], np.float64)[:, None, :]
        v = np.asarray(c["v"], np.float64)[:, None, :]
        do = np.asarray(c["do"], np.float64)[:, None, :]
        n = q.shape[0]
        bias = np.asarray(c["bias"], np.float64)[None] if "bias" in c else None
        r = run_oracle(q, k, v, np.array([0]), np.array([n]), np.array([[0, 0, 0, n]]),
                       c["causal"], c["scale"], bias=bias, do=do)
        np.testing.assert_allclose(r["lse"][0], c["lse"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["o"][:, 0], c["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["delta"][0], c["delta"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["dq"][:, 0], c["dq"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["dk"][:, 0], c["dk"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["dv"][:, 0], c["dv"], rtol=0, atol=1e-14)
        if bias is not None:
            np.testing.assert_allclose(r["dbias"][0], c["dbias"], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("causal,bias", [(True, False), (False, False), (False, True)])
def test_softmax_rows_sum_to_one_and_lse_bruteforce(causal, bias):
    w = _tiny(causal=causal, bias=bias)
    q, k, v, do, bb = _f64(w)
    G = w.hq // w.hkv
    for (b, r0, p0, n) in w.chunks:
        off, L = w.seq_offsets[b], w.seq_lens[b]
        for h in range(w.hq):
            g = h // G
            t = OA.block_terms(q[r0:r0 + n, h], k[off:off + L, g], v[off:off + L, g], None,
                               w.scale, np.arange(p0, p0 + n), causal,
                               None if bb is None else bb[h])
            np.testing.assert_allclose(t["p"].sum(1), 1.0, rtol=0, atol=1e-12)
            for r in range(n):
                p = p0 + r
                # brute force: explicit loop over keys, independent of the oracle's masking
                row = []
                for j in range(L):
                    if causal and j > p:
                        continue
                    s = w.scale * sum(q[r0 + r, h, d] * k[off + j, g, d] for d in range(w.head_dim))
                    if bb is not None:
                        s += bb[h, p, j]
                    row.append(s)
                assert abs(t["lse"][r] - scipy.special.logsumexp(row)) < 1e-12


def test_closed_form_zero_query():
    """q = 0: every visible score is 0, so LSE = ln(#visible) and O is the mean of visible values."""
    w = _tiny(causal=True)
    q = np.zeros((w.q_rows, w.hq, w.head_dim))
    r = _run(w, q=q, with_grad=False)
    _, k, v, _, _ = _f64(w)
    G = w.hq // w.hkv
    for (b, r0, p0, n) in w.chunks:
        off = w.seq_offsets[b]
        for i in range(n):
            p = p0 + i
            for h in range(w.hq):
                assert abs(r["lse"][h, r0 + i] - math.log(p + 1)) < 1e-14
                np.testing.assert_allclose(r["o"][r0 + i, h], v[off:off + p + 1, h // G].mean(0),
                                           rtol=0, atol=1e-14)


def test_single_visible_key():
    """The query at position 0 sees only key 0: LSE = s_00 and O = v_0."""
    w = _tiny(causal=True)
    q, k, v, _, _ = _f64(w)
    r = _run(w, with_grad=False)
    G = w.hq // w.hkv
    for (b, r0, p0, n) in w.chunks:
        if p0 != 0:
            continue
        off = w.seq_offsets[b]
        for h in range(w.hq):
            s00 = w.scale * float(np.dot(q[r0, h], k[off, h // G]))
            assert abs(r["lse"][h, r0] - s00) < 1e-14
            np.testing.assert_array_equal(r["o"][r0, h], v[off, h // G])


def test_causal_perturbation_leaves_earlier_rows_bit_identical():
    w = _tiny(causal=True)
    q, k, v, _, _ = _f64(w)
    base = _run(w, with_grad=False)
    rng = np.random.default_rng(3)
    for (b, r0, p0, n) in w.chunks:
        off, L = w.seq_offsets[b], w.seq_lens[b]
        p = p0  # first row of the chunk
        k2, v2 = k.copy(), v.copy()
        k2[off + p + 1:off + L] += rng.standard_normal(k2[off + p + 1:off + L].shape)
        v2[off + p + 1:off + L] += rng.standard_normal(v2[off + p + 1:off + L].shape)
        pert = _run(w, k=k2, v=v2, with_grad=False)
        np.testing.assert_array_equal(pert["o"][r0], base["o"][r0])
        np.testing.assert_array_equal(pert["lse"][:, r0], base["lse"][:, r0])
        if p + 1 < L and n > 1:
            # a later row that sees a perturbed key must change
            assert not np.array_equal(pert["o"][r0 + n - 1], base["o"][r0 + n - 1]) or p0 + n - 1 <= p


def test_constant_values_give_constant_output_and_zero_qk_grads():
    w = _tiny(causal=True)
    v = np.full((w.kv_rows, w.hkv, w.head_dim), 0.0)
    v[:, :, :] = np.array([1.5, -2.0, 0.25])[: w.head_dim]
    r = _run(w, v=v)
    cov = w.q_valid_rows()
    np.testing.assert_allclose(r["o"][cov], np.broadcast_to(v[0, 0], r["o"][cov].shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["dq"][cov], 0.0, atol=1e-13)
    kvv = w.kv_valid_rows()
    np.testing.assert_allclose(r["dk"][kvv], 0.0, atol=1e-13)


# ---------------------------------------------------------------- rank share

def test_rank_share_equals_full_sequence_rows():
    """Chunked O/LSE/dQ equal the full-sequence rows; chunked dK/dV equal the
    full-sequence gradient with dO zeroed outside the local rows."""
    lens = [16, 12]
    full = W.make_custom(lens=lens, hq=4, hkv=2, head_dim=3, seed=11, poison_padding=False)
    q, k, v, do, _ = _f64(full)
    # share: chunks (0..3) and (12..15) of seq 0, (0..2) and (9..11) of seq 1
    share_chunks = [(0, 0, 4), (0, 12, 4), (1, 0, 3), (1, 9, 3)]
    full_rows = []
    share = W.make_custom(lens=lens, hq=4, hkv=2, head_dim=3, chunks=share_chunks, seed=11,
                          materialize=False)
    for (s, r0, p0, n) in share.chunks:
        full_rows.append(full.chunks[s][1] + p0 + np.arange(n))
    idx = np.concatenate(full_rows)
    qs, dos = q[idx], do[idx]
    rs = run_oracle(qs, k, v, share.seq_offsets, share.seq_lens, share.chunks, True, full.scale, do=dos)
    do_masked = np.zeros_like(do)
    do_masked[idx] = do[idx]
    rf = run_oracle(q, k, v, full.seq_offsets, full.seq_lens, full.chunks, True, full.scale, do=do_masked)
    np.testing.assert_allclose(rs["o"], rf["o"][idx], rtol=0, atol=1e-13)
    np.testing.assert_allclose(rs["lse"], rf["lse"][:, idx], rtol=0, atol=1e-13)
    np.testing.assert_allclose(rs["dq"], rf["dq"][idx], rtol=0, atol=1e-13)
    np.testing.assert_allclose(rs["dk"], rf["dk"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(rs["dv"], rf["dv"], rtol=0, atol=1e-13)


def test_first_contribution_then_addition_equals_one_call():
    """dK/dV of the chunk-pair share = STORE(second chunk) + ADD(first chunk)."""
    w = _tiny(causal=True, chunked=True)
    both = _run(w)
    first = _run(w, chunks=w.chunks[0::2])
    second = _run(w, chunks=w.chunks[1::2])
    kvv = w.kv_valid_rows()
    np.testing.assert_allclose(second["dk"][kvv] + first["dk"][kvv], both["dk"][kvv], rtol=0, atol=1e-13)
    np.testing.assert_allclose(second["dv"][kvv] + first["dv"][kvv], both["dv"][kvv], rtol=0, atol=1e-13)
    assert np.isnan(both["dk"][~kvv]).all()


# ---------------------------------------------------------------- gradients

def _objective(w, q, k, v, do, bias):
    r = run_oracle(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale, bias=bias)
    cov = w.q_valid_rows()
    return float(np.sum(r["o"][cov] * do[cov]))


def _fd_check(w, tol=1e-6):
    q, k, v, do, bias = _f64(w)
    r = run_oracle(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale, bias=bias, do=do)
    eps = 1e-6
    cov = w.q_valid_rows()
    kvv = w.kv_valid_rows()
    targets = [("q", q, r["dq"], cov), ("k", k, r["dk"], kvv), ("v", v, r["dv"], kvv)]
    if bias is not None:
        targets.append(("bias", bias, r["dbias"], None))
    for name, arr, grad, rowmask in targets:
        num = np.zeros_like(arr)
        it = np.ndindex(arr.shape)
        for ix in it:
            if rowmask is not None and not rowmask[ix[0]]:
                continue
            old = arr[ix]
            arr[ix] = old + eps
            fp = _objective(w, q, k, v, do, bias)
            arr[ix] = old - eps
            fm = _objective(w, q, k, v, do, bias)
            arr[ix] = old
            num[ix] = (fp - fm) / (2 * eps)
        sel = (slice(None),) if rowmask is None else (rowmask,)
        a, n = grad[sel], num[sel]
        err = np.linalg.norm(a - n) / max(np.linalg.norm(n), 1e-30)
        assert err <= tol, f"{name}: rel err {err}"


@pytest.mark.parametrize("chunked", [False, True])
@pytest.mark.parametrize("causal,bias", [(True, False), (False, False), (False, True)])
def test_finite_differences(chunked, causal, bias):
    _fd_check(_tiny(causal=causal, bias=bias, chunked=chunked))


def test_ds_rows_sum_to_zero_and_delta_is_do_dot_o():
    w = _tiny(causal=True)
    q, k, v, do, _ = _f64(w)
    G = w.hq // w.hkv
    for (b, r0, p0, n) in w.chunks:
        off, L = w.seq_offsets[b], w.seq_lens[b]
        for h in range(w.hq):
            t = OA.block_terms(q[r0:r0 + n, h], k[off:off + L, h // G], v[off:off + L, h // G],
                               do[r0:r0 + n, h], w.scale, np.arange(p0, p0 + n), True)
            np.testing.assert_allclose(t["ds"].sum(1), 0.0, atol=1e-13)
            np.testing.assert_allclose(t["delta"], np.sum(do[r0:r0 + n, h] * t["o"], 1), atol=1e-13)


def test_gqa_equals_mha_on_repeated_kv():
    w = _tiny(causal=True, hq=4, hkv=2)
    q, k, v, do, _ = _f64(w)
    G = 2
    k_rep = np.repeat(k, G, axis=1)
    v_rep = np.repeat(v, G, axis=1)
    g = run_oracle(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale, do=do)
    m = run_oracle(q, k_rep, v_rep, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale, do=do)
    np.testing.assert_allclose(g["o"], m["o"], atol=1e-14)
    np.testing.assert_allclose(g["dq"], m["dq"], atol=1e-14)
    kvv = w.kv_valid_rows()
    summed_k = m["dk"][kvv].reshape(-1, 2, G, w.head_dim).sum(2)
    summed_v = m["dv"][kvv].reshape(-1, 2, G, w.head_dim).sum(2)
    np.testing.assert_allclose(g["dk"][kvv], summed_k, atol=1e-13)
    np.testing.assert_allclose(g["dv"][kvv], summed_v, atol=1e-13)


# ---------------------------------------------------------------- textbook routine

@pytest.mark.parametrize("causal,bias", [(True, False), (False, True)])
def test_matches_torch_sdpa_float64(causal, bias):
    torch = pytest.importorskip("torch")
    B, L, hq, hkv, D = 2, 9, 4, 2, 8
    w = W.make_custom(lens=[L] * B, hq=hq, hkv=hkv, head_dim=D, causal=causal, bias=bias, seed=5,
                      poison_padding=False)
    q, k, v, do, bb = _f64(w)
    r = _run(w)
    G = hq // hkv
    tq = torch.tensor(q.reshape(B, L, hq, D).transpose(0, 2, 1, 3).copy(), requires_grad=True)
    tk = torch.tensor(k.reshape(B, L, hkv, D).transpose(0, 2, 1, 3).copy(), requires_grad=True)
    tv = torch.tensor(v.reshape(B, L, hkv, D).transpose(0, 2, 1, 3).copy(), requires_grad=True)
    mask = None
    if bias:
        tb = torch.tensor(bb, requires_grad=True)
        mask = tb.unsqueeze(0).expand(B, hq, L, L)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1),
        attn_mask=mask, is_causal=causal, scale=w.scale)
    tdo = torch.tensor(do.reshape(B, L, hq, D).transpose(0, 2, 1, 3).copy())
    (o * tdo).sum().backward()
    back = lambda t, H: t.detach().numpy().transpose(0, 2, 1, 3).reshape(B * L, H, D)
    np.testing.assert_allclose(r["o"], back(o, hq), rtol=0, atol=1e-10)
    np.testing.assert_allclose(r["dq"], back(tq.grad, hq), rtol=0, atol=1e-10)
    np.testing.assert_allclose(r["dk"], back(tk.grad, hkv), rtol=0, atol=1e-10)
    np.testing.assert_allclose(r["dv"], back(tv.grad, hkv), rtol=0, atol=1e-10)
    if bias:
        np.testing.assert_allclose(r["dbias"], tb.grad.numpy(), rtol=0, atol=1e-10)


# ---------------------------------------------------------------- bias pins

def test_dbias_rows_sum_to_zero_and_shift_invariance():
    w = _tiny(causal=False, bias=True, chunked=False)
    q, k, v, do, bias = _f64(w)
    r = _run(w)
    np.testing.assert_allclose(r["dbias"].sum(-1), 0.0, atol=1e-12)
    shift = np.random.default_rng(1).standard_normal(bias.shape[:2])
    r2 = _run(w, bias=bias + shift[:, :, None])
    np.testing.assert_allclose(r2["o"], r["o"], atol=1e-13)
    for (b, r0, p0, n) in w.chunks:
        for h in range(w.hq):
            np.testing.assert_allclose(r2["lse"][h, r0:r0 + n] - r["lse"][h, r0:r0 + n],
                                       shift[h, p0:p0 + n], atol=1e-13)


# ---------------------------------------------------------------- layout copies

def test_pack_unpack_roundtrip_and_index_map():
    B, H, S, D = 3, 2, 6, 4
    x = W.make_bhsd(B, H, S, D, seed=9)
    lens = np.array([6, 2, 5], np.int32)
    offs = np.array([0, 8, 10], np.int32)
    sentinel = np.full((16, H, D), 0xABCD, np.uint16)
    thd = OL.pack(x, offs, lens, sentinel)
    for b in range(B):
        for h in range(H):
            for s in range(S):
                if s < lens[b]:
                    assert (thd[offs[b] + s, h] == x[b, h, s]).all()
    written = np.zeros(16, bool)
    for o, L in zip(offs, lens):
        written[o:o + L] = True
    assert (thd[~written] == 0xABCD).all()
    back = OL.unpack(thd, offs, lens, np.full_like(x, 0x1234))
    for b in range(B):
        assert (back[b, :, :lens[b]] == x[b, :, :lens[b]]).all()
        assert (back[b, :, lens[b]:] == 0x1234).all()


# ---------------------------------------------------------------- workloads

def test_named_workload_shapes_and_pair_counts():
    w3 = W.make_config(3, materialize=False)
    assert w3.q_rows == 65536 and w3.kv_rows == 524288 and w3.num_chunks == 128
    assert OA.visible_pairs(w3.seq_lens, w3.chunks, True) == 64 * 512 * 8193
    w1 = W.make_config(1, materialize=False)
    assert OA.visible_pairs(w1.seq_lens, w1.chunks, True) * w1.hq == 525312
    w4 = W.make_config(4, materialize=False)
    assert (w4.seq_lens % 64 == 0).all() and w4.seq_lens.min() >= 1024 and w4.seq_lens.max() <= 8192
    w5 = W.make_config(5, materialize=False)
    assert OA.visible_pairs(w5.seq_lens, w5.chunks, False) * w5.hq == 4294967296


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -3.1415927, 65504.0], np.float32)
    b = W.bf16_bits_from_f32(x)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1 + 3*2^-9 rounds up
    assert list(W.f32_from_bf16_bits(b)[:4]) == [1.0, 1.0, 1.0078125, 1.0078125]
    assert abs(W.f32_from_bf16_bits(b)[4] - (-3.140625)) < 1e-7


# ---------------------------------------------------------------- planted mistakes

def _mutant(kind):
    orig = OA.block_terms

    def mutated(qc, kb, vb, doc, scale, pos, causal, bias_h=None):
        t = orig(qc, kb, vb, doc, scale, pos, causal, bias_h)
        if doc is None:
            return t
        if kind == "dk_without_scale":
            t["dk"] = t["dk"] / scale
        elif kind == "delta_dropped":
            ds = t["p"] * t["dp"]
            t["dq"] = scale * ds @ kb
            t["dk"] = scale * ds.T @ qc
        elif kind == "dv_wrong_row_index":
            t["dv"] = t["p"].T @ doc[::-1]
        elif kind == "dq_sign":
            t["dq"] = -t["dq"]
        return t
    return mutated


@pytest.mark.parametrize("kind", ["dk_without_scale", "delta_dropped", "dv_wrong_row_index", "dq_sign"])
def test_planted_gradient_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(OA, "block_terms", _mutant(kind))
    with pytest.raises(AssertionError):
        _fd_check(_tiny(causal=True, chunked=True, D=2, lens=(3, 4)))


def test_planted_mask_mistake_is_caught(monkeypatch):
    orig = OA.visible_mask
    monkeypatch.setattr(OA, "visible_mask", lambda pos, L, causal: orig(pos - 1, L, causal) | (np.arange(L)[None, :] == 0))
    with pytest.raises(AssertionError):
        test_matches_torch_sdpa_float64(True, False)
