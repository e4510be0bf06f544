"""Oracle for the copies around the all-to-all (A2A) head <-> sequence swap.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The product path never calls it and shares
no code with it.

Sources (page titles and sections):
  * "Optimize context parallel attention layouts and gradient accumulation":
    "Description" and "Changes" (vectorised BF16 A2A pack/unpack copies inside the
    existing head/sequence swap, used by both attention backends), "Validation and
    performance" (the CP4/A2A B64/S8192/Hq32/Hkv8/D128 run that those copies sped up).

What the swap does (the pages name it; the steps are the plain reading):
context parallelism over cp ranks keeps, on rank r, the THD rows of its chunks of
every sequence with all H heads: local [rows_per_rank, H, D].  Attention needs whole
sequences, so an all-to-all gives every rank all rows of H / cp heads.  Four copies
surround the two all-to-alls (Hc = H / cp):

  sequence -> head (before attention):
    split_heads   send[j, t, h, :] = local[t, j Hc + h, :]; block j goes to rank j.
    scatter_rows  the received block s holds rank s's rows: row q_row + i of chunk
                  {seq, q_row, pos0, len} of rank s lands on row
                  seq_offsets[seq] + pos0 + i of the sequence-ordered tensor.
  head -> sequence (after attention):
    gather_rows   the inverse of scatter_rows: block s collects rank s's rows.
    merge_heads   the inverse of split_heads.

Rows that no chunk names keep whatever the destination held.
"""
from __future__ import annotations

import numpy as np


def split_heads(local: np.ndarray, cp: int) -> np.ndarray:
    """[rows, H, D] -> [cp, rows, H / cp, D]: block j holds heads [j Hc, (j + 1) Hc)."""
    rows, H, D = local.shape
    Hc = H // cp
    send = np.empty((cp, rows, Hc, D), dtype=local.dtype)
    for j in range(cp):
        for h in range(Hc):
            send[j, :, h, :] = local[:, j * Hc + h, :]
    return send


def merge_heads(recv: np.ndarray) -> np.ndarray:
    """[cp, rows, Hc, D] -> [rows, cp Hc, D]: block j becomes heads [j Hc, (j + 1) Hc)."""
    cp, rows, Hc, D = recv.shape
    out = np.empty((rows, cp * Hc, D), dtype=recv.dtype)
    for j in range(cp):
        for h in range(Hc):
            out[:, j * Hc + h, :] = recv[j, :, h, :]
    return out


def scatter_rows(recv: np.ndarray, chunk_maps, seq_offsets, full_out: np.ndarray) -> np.ndarray:
    """Blocks [cp, rows_per_rank, Hc, D] into a copy of the sequence-ordered full_out."""
    full = full_out.copy()
    for s in range(recv.shape[0]):
        for (seq, q_row, pos0, n) in np.asarray(chunk_maps[s]).reshape(-1, 4):
            for i in range(int(n)):
                full[int(seq_offsets[seq]) + int(pos0) + i] = recv[s, int(q_row) + i]
    return full


def gather_rows(full: np.ndarray, chunk_maps, seq_offsets, send_out: np.ndarray) -> np.ndarray:
    """Rank s's rows of the sequence-ordered `full` into block s of a copy of send_out."""
    send = send_out.copy()
    for s in range(send.shape[0]):
        for (seq, q_row, pos0, n) in np.asarray(chunk_maps[s]).reshape(-1, 4):
            for i in range(int(n)):
                send[s, int(q_row) + i] = full[int(seq_offsets[seq]) + int(pos0) + i]
    return send
