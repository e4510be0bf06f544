"""FP64 CPU oracle for attention over one key window and the merge of partial results.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The product path never calls it and shares
no code with it.

Sources (page titles and sections):
  * "Optimize context parallel attention layouts and gradient accumulation",
    "Private C++ FROST P2P": context parallelism over point-to-point exchanges,
    where each step attends to one block of the gathered K/V;
  * "Support and performance optimization for Hopper (H200) architecture?"
    (boltz-cp issue 1): the asynchronous P2P ring communications of the folding
    model's context parallelism.

What it computes, from the plain definition (readings listed in the design notes):
  * A key window W = [lo, hi) of sequence positions narrows the visible keys of
    every query to V(p) intersected with W.  The partial forward over W is the
    softmax over those keys: LSE_W = log sum_{j in V(p) & W} exp(s_j) and
    O_W = sum_j exp(s_j - LSE_W) v_j.  A row with no visible key in W has
    LSE_W = -inf and O_W = 0.
  * For disjoint key sets A and B, e^(LSE_X - LSE) is the share of the total
    softmax mass that lies on X, so LSE = log(e^LSE_A + e^LSE_B) and
    O = e^(LSE_A - LSE) O_A + e^(LSE_B - LSE) O_B is the result over A and B.
  * The backward over W uses the complete O and LSE: P_j = exp(s_j - LSE) for
    j in W (0 elsewhere), dP_j = dO.v_j, Delta = dO.O, dS_j = P_j (dP_j - Delta);
    the window's shares are dQ_W = scale dS K, and dK, dV of the keys in W.  The
    shares over disjoint windows covering every key add up to the full gradients.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

from .softmax_attention import scores


def _window_scores(qc, kb, scale, pos, causal, bias_h, lo: int, hi: int) -> np.ndarray:
    """Scores with the keys outside [lo, hi) masked as well (-inf)."""
    s = scores(qc, kb, scale, pos, causal, bias_h)
    j = np.arange(kb.shape[0])[None, :]
    return np.where((j >= lo) & (j < hi), s, -np.inf)


def _lse_or_minus_inf(s: np.ndarray) -> np.ndarray:
    """Row-wise log-sum-exp; -inf for a row without a finite score."""
    m = np.max(s, axis=1)
    out = np.full(s.shape[0], -np.inf)
    ok = np.isfinite(m)
    if ok.any():
        out[ok] = m[ok] + np.log(np.sum(np.exp(s[ok] - m[ok, None]), axis=1))
    return out


def attention_window(q, k, v, seq_offsets, seq_lens, chunks, causal: bool, scale: float,
                     window: Tuple[int, int], bias=None) -> Dict[str, np.ndarray]:
    """Partial forward over the key window: o [q_rows, hq, D], lse [hq, q_rows] (NaN off chunks)."""
    lo, hi = window
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_rows, hq, D = q.shape
    G = hq // k.shape[1]
    o = np.full((q_rows, hq, D), np.nan)
    lse = np.full((hq, q_rows), np.nan)
    for (b, r0, p0, n) in np.asarray(chunks):
        if n == 0:
            continue
        off, L = int(seq_offsets[b]), int(seq_lens[b])
        pos = np.arange(p0, p0 + n)
        rows = slice(r0, r0 + n)
        for h in range(hq):
            g = h // G
            s = _window_scores(q[rows, h], k[off:off + L, g], scale, pos, causal,
                               None if bias is None else np.asarray(bias[h], np.float64), lo, hi)
            l = _lse_or_minus_inf(s)
            p = np.exp(s - np.where(np.isfinite(l), l, 0.0)[:, None])
            p[~np.isfinite(l)] = 0.0
            o[rows, h] = p @ v[off:off + L, g]
            lse[h, rows] = l
    return {"o": o, "lse": lse}


def merge(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Result over the union of two disjoint key sets from the two partial results.

    o_*: [rows, hq, D]; lse_*: [hq, rows].  Rows where both LSEs are -inf give
    O = 0 and LSE = -inf.
    """
    o_a = np.asarray(o_a, np.float64)
    o_b = np.asarray(o_b, np.float64)
    la = np.asarray(lse_a, np.float64).T  # [rows, hq]
    lb = np.asarray(lse_b, np.float64).T
    m = np.maximum(la, lb)
    fin = np.isfinite(m)
    ms = np.where(fin, m, 0.0)
    wa = np.where(fin, np.exp(la - ms), 0.0)
    wb = np.where(fin, np.exp(lb - ms), 0.0)
    tot = wa + wb
    lse = np.where(fin, ms + np.log(np.where(fin, tot, 1.0)), -np.inf)
    ra = np.where(fin, wa / np.where(fin, tot, 1.0), 0.0)
    rb = np.where(fin, wb / np.where(fin, tot, 1.0), 0.0)
    o = ra[..., None] * o_a + rb[..., None] * o_b
    return o, lse.T


def backward_window(q, k, v, do, o, lse, seq_offsets, seq_lens, chunks, causal: bool, scale: float,
                    window: Tuple[int, int], bias=None) -> Dict[str, np.ndarray]:
    """The window's gradient shares, given the complete forward results o and lse.

    Returns dq [q_rows, hq, D] (NaN off chunk rows), and dk, dv [kv_rows, hkv, D]
    holding the window's keys' gradients on every valid key row inside the window of
    every sequence (0 where no query attends) and NaN elsewhere.
    """
    lo, hi = window
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    q_rows, hq, D = q.shape
    kv_rows, hkv, _ = k.shape
    G = hq // hkv
    dq = np.full((q_rows, hq, D), np.nan)
    dk = np.full((kv_rows, hkv, D), np.nan)
    dv = np.full((kv_rows, hkv, D), np.nan)
    for b, (off, L) in enumerate(zip(seq_offsets, seq_lens)):
        a, e = off + max(0, min(lo, L)), off + max(0, min(hi, L))
        dk[a:e] = 0.0
        dv[a:e] = 0.0
    for (b, r0, p0, n) in np.asarray(chunks):
        if n == 0:
            continue
        off, L = int(seq_offsets[b]), int(seq_lens[b])
        pos = np.arange(p0, p0 + n)
        rows = slice(r0, r0 + n)
        for h in range(hq):
            g = h // G
            kb, vb = k[off:off + L, g], v[off:off + L, g]
            s = _window_scores(q[rows, h], kb, scale, pos, causal,
                               None if bias is None else np.asarray(bias[h], np.float64), lo, hi)
            p = np.exp(s - lse[h, rows][:, None])
            dp = do[rows, h] @ vb.T
            delta = np.sum(do[rows, h] * o[rows, h], axis=1)
            ds = p * (dp - delta[:, None])
            dq[rows, h] = scale * (ds @ kb)
            w = slice(max(0, min(lo, L)), max(0, min(hi, L)))
            dk[off + w.start:off + w.stop, g] += (scale * (ds.T @ q[rows, h]))[w]
            dv[off + w.start:off + w.stop, g] += (p.T @ do[rows, h])[w]
    return {"dq": dq, "dk": dk, "dv": dv}
