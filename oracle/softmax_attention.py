"""FP64 CPU oracle for blockwise causal GQA attention on one context-parallel rank's share.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The product path (the HIP library and its
binding) never calls it and shares no code with it.

What it computes is the plain definition of softmax attention, written out in
float64 with NumPy matrix products and no blocking, fusion or reordering.  The
blockwise (flash-style) algorithm the GPU runs is an exact reformulation of the
same result in real arithmetic, so the plain definition is the oracle.

Sources (page titles and sections):
  * "Optimize context parallel attention layouts and gradient accumulation"
    (TransformerEngine PR 3683):
      - "Description" / "Changes": causal attention on packed THD inputs with
        physical sequence offsets and pitches, separate Q/K/V, grouped-query
        heads (GQA), head dims 128 and 256, the softmax statistics (Stats = the
        log-sum-exp per query row and head) kept as an output of the forward;
      - "CP8 first-gradient accumulator reuse": the AllGather backward sums the
        per-chunk dK/dV contributions; the first contribution is the initial
        value of the accumulator and the later one is added to it;
      - "CP8 AllGather: composition with first-gradient reuse": the backward's
        pre-pass takes the row dot product of dO and O;
      - "Independent-node complete-CP evidence": the B64/S8192/Hq32/Hkv8/D256
        coordinate and the independent CPU FP64 checks this oracle mirrors.
  * "Support and performance optimization for Hopper (H200) architecture?"
    (boltz-cp issue 1, maintainer reply): triangle attention, i.e. row
    attention over a pair tensor with an additive pair bias shared by all rows.

Readings where the pages are silent (all listed in the design notes):
  * A query at position p of its sequence sees key j iff 0 <= j < L and, when
    causal, j <= p.  Positions come from the chunk map, so no top-left or
    bottom-right alignment choice remains.
  * GQA maps query head h to KV head h // G with G = Hq / Hkv.
  * LSE is the natural-log log-sum-exp of the scaled (and biased) scores.
  * The pair bias enters after scaling: s = scale * q.k + bias[h, p, j].
  * dBias is the plain sum of dS over every query row that uses it.

Inputs are float64 arrays holding the BF16 input values exactly.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# One (chunk, query head) block: the definition, row by row, with matrix products.
# ----------------------------------------------------------------------------

def visible_mask(pos: np.ndarray, L: int, causal: bool) -> np.ndarray:
    """[n, L] boolean: key j is visible to the query at position pos[r].

    Causal masking by position within the sequence ("Changes": causal THD with
    physical offsets; chunk positions per the rank-share chunk map).
    """
    j = np.arange(L)[None, :]
    if causal:
        return j <= pos[:, None]
    return np.ones((pos.shape[0], L), dtype=bool)


def scores(qc: np.ndarray, kb: np.ndarray, scale: float, pos: np.ndarray, causal: bool,
           bias_h: Optional[np.ndarray]) -> np.ndarray:
    """s[r, j] = scale * <q_r, k_j> (+ bias[h, p_r, j]); masked keys are -inf."""
    L = kb.shape[0]
    s = scale * (qc @ kb.T)
    if bias_h is not None:
        s = s + bias_h[pos][:, :L]
    return np.where(visible_mask(pos, L, causal), s, -np.inf)


def log_sum_exp(s: np.ndarray) -> np.ndarray:
    """Row-wise log(sum_j exp(s_j)) with the usual max shift; rows need >= 1 finite entry."""
    m = np.max(s, axis=1)
    return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))


def probs(s: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """P = exp(s - LSE): the softmax of each row (masked entries give 0)."""
    return np.exp(s - lse[:, None])


def block_terms(qc, kb, vb, doc, scale, pos, causal, bias_h=None) -> Dict[str, np.ndarray]:
    """Every intermediate of one (chunk, query head) block.

    Forward: S, LSE, P, O = P V.  Backward (given dO): dP = dO V^T,
    Delta = rowsum(P * dP) (equal to rowsum(dO * O), the pre-pass dot of the
    composition section), dS = P * (dP - Delta), dQ = scale dS K,
    dK = scale dS^T Q, dV = P^T dO, dBias = dS.
    """
    s = scores(qc, kb, scale, pos, causal, bias_h)
    lse = log_sum_exp(s)
    p = probs(s, lse)
    out = {"s": s, "lse": lse, "p": p, "o": p @ vb}
    if doc is not None:
        dp = doc @ vb.T
        delta = np.sum(p * dp, axis=1)
        ds = p * (dp - delta[:, None])
        out.update(dp=dp, delta=delta, ds=ds, dq=scale * (ds @ kb),
                   dk=scale * (ds.T @ qc), dv=p.T @ doc)
    return out


# ----------------------------------------------------------------------------
# The whole rank share.
# ----------------------------------------------------------------------------

def _selected(select, b: int, g: int) -> bool:
    if select is None:
        return True
    seqs, kv_heads = select
    return (seqs is None or b in seqs) and (kv_heads is None or g in kv_heads)


def attention(q, k, v, seq_offsets, seq_lens, chunks, causal: bool, scale: float,
              bias=None, do=None, select: Optional[Tuple[Optional[Iterable[int]], Optional[Iterable[int]]]] = None):
    """Forward (and backward when dO is given) of the rank share.

    q, do: [q_rows, hq, D]; k, v: [kv_rows, hkv, D]; bias: [hq, Lb, Lb] or None.
    chunks: [C, 4] rows {seq, q_row, pos0, len}.
    select: optional (sequences, kv heads) to restrict the work to; outputs
    outside the selection stay NaN.

    Returns a dict with
      o [q_rows, hq, D], lse [hq, q_rows], delta [hq, q_rows]: NaN on rows no
        (selected) chunk covers;
      dq [q_rows, hq, D]: likewise;
      dk, dv [kv_rows, hkv, D]: the GQA- and chunk-summed gradient on every
        valid row of every selected sequence (0 where no query attends), NaN
        on padding rows;
      dbias [hq, Lb, Lb]: summed over all query rows (only when bias is given).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_rows, hq, D = q.shape
    kv_rows, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    G = hq // hkv
    nan = np.nan
    o = np.full((q_rows, hq, D), nan)
    lse = np.full((hq, q_rows), nan)
    res = {"o": o, "lse": lse}
    if do is not None:
        do = np.asarray(do, np.float64)
        dq = np.full((q_rows, hq, D), nan)
        delta = np.full((hq, q_rows), nan)
        dk = np.full((kv_rows, hkv, D), nan)
        dv = np.full((kv_rows, hkv, D), nan)
        # the first contribution of every valid row of every sequence: zero
        for b, (off, L) in enumerate(zip(seq_offsets, seq_lens)):
            for g in range(hkv):
                if _selected(select, b, g):
                    dk[off:off + L, g] = 0.0
                    dv[off:off + L, g] = 0.0
        res.update(dq=dq, delta=delta, dk=dk, dv=dv)
        if bias is not None:
            res["dbias"] = np.zeros(np.shape(bias))
    for (b, r0, p0, n) in np.asarray(chunks):
        if n == 0:
            continue
        off, L = int(seq_offsets[b]), int(seq_lens[b])
        pos = np.arange(p0, p0 + n)
        rows = slice(r0, r0 + n)
        for h in range(hq):
            g = h // G
            if not _selected(select, int(b), g):
                continue
            kb = k[off:off + L, g]
            vb = v[off:off + L, g]
            t = block_terms(q[rows, h], kb, vb, None if do is None else do[rows, h], scale, pos,
                            causal, None if bias is None else np.asarray(bias[h], np.float64))
            o[rows, h] = t["o"]
            lse[h, rows] = t["lse"]
            if do is not None:
                dq[rows, h] = t["dq"]
                delta[h, rows] = t["delta"]
                dk[off:off + L, g] += t["dk"]
                dv[off:off + L, g] += t["dv"]
                if bias is not None:
                    res["dbias"][h, p0:p0 + n, :L] += t["ds"]
    return res


def visible_pairs(seq_lens, chunks, causal: bool) -> int:
    """Number of visible (query, key) pairs per query head, summed over chunks."""
    total = 0
    for (b, _, p0, n) in np.asarray(chunks):
        L = int(seq_lens[b])
        if causal:
            total += sum(min(p + 1, L) for p in range(int(p0), int(p0) + int(n)))
        else:
            total += int(n) * L
    return total
