"""Pins of the key-window oracle and the merge of partial results (CPU only).

They tie oracle/window.py to things fixed outside it: the full-attention oracle
(itself pinned in test_oracle_pins.py), PyTorch's float64 scaled-dot-product
attention with an explicit mask, and the algebra of the merge (identity element,
order independence)."""
import numpy as np
import pytest

import oracle
import oracle.window as OW
import workloads as W


def _f64(w):
    return (W.f64_from_bf16_bits(w.q), W.f64_from_bf16_bits(w.k), W.f64_from_bf16_bits(w.v),
            W.f64_from_bf16_bits(w.do), None if w.bias is None else w.bias.astype(np.float64))


def _case(causal=True, bias=False, lens=(9, 14), hq=4, hkv=2, D=5, seed=3):
    chunks = []
    for b, L in enumerate(lens):
        chunks += [(b, 0, 3), (b, L - 4, 4)]
    return W.make_custom(lens=list(lens), hq=hq, hkv=hkv, head_dim=D, causal=causal,
                         chunks=None if bias else chunks, bias=bias, seed=seed, pad_kv_rows=2,
                         pad_q_rows=1, poison_padding=False)


def _rows(w):
    return w.q_valid_rows()


CASES = [dict(causal=True), dict(causal=False), dict(causal=False, bias=True)]


@pytest.mark.parametrize("kw", CASES)
@pytest.mark.parametrize("cuts", [(4,), (1, 6), (0, 5, 11), (3, 100)])
def test_window_partials_merge_to_full_attention(kw, cuts):
    w = _case(**kw)
    q, k, v, do, bias = _f64(w)
    full = oracle.attention(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale, bias=bias)
    edges = [0, *cuts, 10**6]
    parts = [OW.attention_window(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale,
                                 (lo, hi), bias=bias) for lo, hi in zip(edges[:-1], edges[1:])]
    rows = _rows(w)
    # left to right, and right to left: the merge does not depend on the order
    o, lse = parts[0]["o"], parts[0]["lse"]
    for p in parts[1:]:
        o, lse = OW.merge(o, lse, p["o"], p["lse"])
    o2, lse2 = parts[-1]["o"], parts[-1]["lse"]
    for p in parts[-2::-1]:
        o2, lse2 = OW.merge(p["o"], p["lse"], o2, lse2)
    for oo, ll in ((o, lse), (o2, lse2)):
        np.testing.assert_allclose(oo[rows], full["o"][rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ll[:, rows], full["lse"][:, rows], rtol=0, atol=1e-12)


def test_whole_sequence_window_is_the_full_forward():
    w = _case()
    q, k, v, do, bias = _f64(w)
    full = oracle.attention(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale)
    part = OW.attention_window(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale, (0, 10**6))
    rows = _rows(w)
    np.testing.assert_allclose(part["o"][rows], full["o"][rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(part["lse"][:, rows], full["lse"][:, rows], rtol=0, atol=1e-14)


def test_rows_without_a_visible_key_and_merge_identity():
    w = _case()
    q, k, v, do, bias = _f64(w)
    # causal rows at positions 0..2 see no key in [5, 9)
    part = OW.attention_window(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale, (5, 9))
    early = np.array([r for (b, r0, p0, n) in w.chunks for r in range(r0, r0 + n) if p0 == 0])
    assert np.all(part["lse"][:, early] == -np.inf)
    assert np.all(part["o"][early] == 0.0)
    # merging with an empty partial changes nothing
    empty_o = np.zeros_like(part["o"])
    empty_l = np.full_like(part["lse"], -np.inf)
    rows = _rows(w)
    full = OW.attention_window(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale, (0, 10**6))
    o, lse = OW.merge(full["o"], full["lse"], empty_o, empty_l)
    np.testing.assert_allclose(o[rows], full["o"][rows], rtol=0, atol=0)
    np.testing.assert_allclose(lse[:, rows], full["lse"][:, rows], rtol=0, atol=0)
    o, lse = OW.merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(lse == -np.inf) and np.all(o == 0.0)


@pytest.mark.parametrize("kw", CASES)
def test_window_backward_shares_add_up_to_the_full_gradients(kw):
    w = _case(**kw)
    q, k, v, do, bias = _f64(w)
    full = oracle.attention(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, w.causal, w.scale, bias=bias,
                            do=do)
    edges = [0, 2, 7, 10**6]
    dq = np.zeros_like(q)
    dk = np.full_like(k, np.nan)
    dv = np.full_like(v, np.nan)
    for lo, hi in zip(edges[:-1], edges[1:]):
        g = OW.backward_window(q, k, v, do, full["o"], full["lse"], w.seq_offsets, w.seq_lens, w.chunks,
                               w.causal, w.scale, (lo, hi), bias=bias)
        rows = _rows(w)
        dq[rows] += g["dq"][rows]
        m = ~np.isnan(g["dk"][:, 0, 0])
        assert np.all(np.isnan(dk[m, 0, 0])), "windows overlap"
        dk[m] = g["dk"][m]
        dv[m] = g["dv"][m]
    rows = _rows(w)
    kr = w.kv_valid_rows()
    np.testing.assert_allclose(dq[rows], full["dq"][rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk[kr], full["dk"][kr], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv[kr], full["dv"][kr], rtol=0, atol=1e-12)


def test_window_forward_matches_torch_sdpa_with_an_explicit_mask():
    torch = pytest.importorskip("torch")
    B, L, hq, hkv, D = 2, 10, 4, 2, 6
    w = W.make_custom(lens=[L] * B, hq=hq, hkv=hkv, head_dim=D, causal=True, seed=9, poison_padding=False)
    q, k, v, do, _ = _f64(w)
    lo, hi = 0, 6  # every causal row keeps key 0, so no row of the mask is empty
    part = OW.attention_window(q, k, v, w.seq_offsets, w.seq_lens, w.chunks, True, w.scale, (lo, hi))
    G = hq // hkv
    tq = torch.tensor(q.reshape(B, L, hq, D).transpose(0, 2, 1, 3).copy())
    tk = torch.tensor(k.reshape(B, L, hkv, D).transpose(0, 2, 1, 3).copy()).repeat_interleave(G, dim=1)
    tv = torch.tensor(v.reshape(B, L, hkv, D).transpose(0, 2, 1, 3).copy()).repeat_interleave(G, dim=1)
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    mask = (j <= i) & (j >= lo) & (j < hi)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=w.scale)
    got = part["o"].reshape(B, L, hq, D).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(got, o.numpy(), rtol=0, atol=1e-12)
    s = torch.einsum("bhid,bhjd->bhij", tq, tk) * w.scale
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(part["lse"].reshape(hq, B, L).transpose(1, 0, 2), lse.numpy(), rtol=0,
                               atol=1e-12)
