"""Oracle for the BHSD <-> THD layout copies.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.

Source: page "Optimize context parallel attention layouts and gradient
accumulation", "Changes" (vectorised BF16 pack/unpack layout copies, physical
sequence origins and pitches preserved).  The copy is a pure re-indexing of
head-dim rows: thd[off_b + s, h, :] = bhsd[b, h, s, :] for s < L_b.  Rows the
copy does not cover keep whatever the destination held.
"""
from __future__ import annotations

import numpy as np


def pack(bhsd: np.ndarray, seq_offsets, seq_lens, thd_out: np.ndarray) -> np.ndarray:
    """Return a copy of thd_out with every valid BHSD row written into it."""
    B, H, S, D = bhsd.shape
    thd = thd_out.copy()
    for b in range(B):
        off, L = int(seq_offsets[b]), int(seq_lens[b])
        for h in range(H):
            for s in range(L):
                thd[off + s, h, :] = bhsd[b, h, s, :]
    return thd


def unpack(thd: np.ndarray, seq_offsets, seq_lens, bhsd_out: np.ndarray) -> np.ndarray:
    """Return a copy of bhsd_out with every valid THD row written back into it."""
    B, H, S, D = bhsd_out.shape
    bhsd = bhsd_out.copy()
    for b in range(B):
        off, L = int(seq_offsets[b]), int(seq_lens[b])
        for h in range(H):
            for s in range(L):
                bhsd[b, h, s, :] = thd[off + s, h, :]
    return bhsd
