"""Seeded synthetic inputs for the context-parallel causal GQA attention path.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  Both the FP64 oracle and the HIP path receive exactly the arrays
made here, so parity compares the two on identical bits.

Layouts (all row-major, head dim innermost):
  Q, dO        [q_rows,  hq,  D]   BF16 bit patterns (uint16)
  K, V         [kv_rows, hkv, D]   BF16 bit patterns (uint16)
  bias         [hq, bias_len, bias_len] float32 (pair-biased variant only)
  seq_offsets  int32 [B]   physical K/V row of position 0 of sequence b
  seq_lens     int32 [B]   valid length of sequence b
  chunks       int32 [C,4] {seq, q_row, pos0, len}: Q rows [q_row, q_row+len)
               hold positions [pos0, pos0+len) of sequence `seq`.

The five named workloads follow the shapes of the pages' measurements:
the context-parallel coordinate B64/S8192/Hq32/Hkv8/D256 (page "Optimize
context parallel attention layouts and gradient accumulation", section
"Independent-node complete-CP evidence") cut to one rank's chunk-pair share,
the unequal padded THD coverage named in its "Changes" list, and the
triangle-attention computation of page "Support and performance optimization
for Hopper (H200) architecture?" (maintainer reply on the TriAttn kernel).
Values are N(0,1) drawn with NumPy PCG64 and rounded to BF16 with
round-to-nearest-even; padding rows are filled with NaN so that any read of
padding shows up in the results.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
_BLOCK = 1 << 24  # elements drawn per block (bounds host memory on big shapes)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (round-to-nearest-even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def f32_from_bf16_bits(u: np.ndarray) -> np.ndarray:
    """Exact decode of BF16 bit patterns to float32."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_from_bf16_bits(u: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(u).astype(np.float64)


def draw_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to BF16, drawn block by block in C order."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = bf16_bits_from_f32(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def draw_f32(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


@dataclasses.dataclass
class Workload:
    name: str
    hq: int
    hkv: int
    head_dim: int
    q_rows: int
    kv_rows: int
    causal: bool
    scale: float
    seq_offsets: np.ndarray
    seq_lens: np.ndarray
    chunks: np.ndarray
    bias_len: int = 0
    seed: Optional[int] = None
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    do: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.seq_offsets.shape[0])

    @property
    def num_chunks(self) -> int:
        return int(self.chunks.shape[0])

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def max_chunk_len(self) -> int:
        return int(self.chunks[:, 3].max()) if self.num_chunks else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    def q_valid_rows(self) -> np.ndarray:
        """Boolean mask over Q rows that some chunk covers."""
        m = np.zeros(self.q_rows, dtype=bool)
        for _, r0, _, n in self.chunks:
            m[r0:r0 + n] = True
        return m

    def kv_valid_rows(self) -> np.ndarray:
        m = np.zeros(self.kv_rows, dtype=bool)
        for o, n in zip(self.seq_offsets, self.seq_lens):
            m[o:o + n] = True
        return m


def _finish(w: Workload, materialize: bool, poison_padding: bool) -> Workload:
    if not materialize:
        return w
    rng = np.random.Generator(np.random.PCG64(w.seed))
    w.q = draw_bf16(rng, (w.q_rows, w.hq, w.head_dim))
    w.k = draw_bf16(rng, (w.kv_rows, w.hkv, w.head_dim))
    w.v = draw_bf16(rng, (w.kv_rows, w.hkv, w.head_dim))
    w.do = draw_bf16(rng, (w.q_rows, w.hq, w.head_dim))
    if w.bias_len:
        w.bias = draw_f32(rng, (w.hq, w.bias_len, w.bias_len))
    if poison_padding:
        qpad = ~w.q_valid_rows()
        kvpad = ~w.kv_valid_rows()
        if qpad.any():
            w.q[qpad] = BF16_NAN
            w.do[qpad] = BF16_NAN
        if kvpad.any():
            w.k[kvpad] = BF16_NAN
            w.v[kvpad] = BF16_NAN
    return w


def _rank_share_chunks(lens, q_pitch, n_chunks=16, first=0, second=15):
    """Chunk pair {first, second} of every sequence, packed at a fixed Q pitch."""
    rows = []
    for b, L in enumerate(lens):
        c = int(L) // n_chunks
        rows.append((b, q_pitch * b, first * c, c))
        rows.append((b, q_pitch * b + c, second * c, c))
    return np.asarray(rows, dtype=np.int32).reshape(-1, 4)


CONFIG_NAMES = {
    1: "causal_gqa_b1_s512_hq4_hkv1_d128",
    2: "thd_equal_b8_s2048_hq32_hkv8_d128",
    3: "cp_rank_share_b64_s8192_chunks0_15_hq32_hkv8_d256",
    4: "thd_unequal_padded_b16_pitch8192_chunks0_15_hq32_hkv8_d128",
    5: "pair_bias_rows1024_len1024_h4_d32",
}


def make_config(cfg: int, materialize: bool = True, seed: Optional[int] = None,
                poison_padding: bool = True) -> Workload:
    """One of the five named workloads, seeded with 1000+cfg unless given."""
    seed = 1000 + cfg if seed is None else seed
    if cfg == 1:
        S, D = 512, 128
        w = Workload(CONFIG_NAMES[1], 4, 1, D, S, S, True, 1 / math.sqrt(D),
                     np.array([0], np.int32), np.array([S], np.int32),
                     np.array([[0, 0, 0, S]], np.int32), seed=seed)
    elif cfg == 2:
        B, S, D = 8, 2048, 128
        off = (np.arange(B) * S).astype(np.int32)
        w = Workload(CONFIG_NAMES[2], 32, 8, D, B * S, B * S, True, 1 / math.sqrt(D),
                     off, np.full(B, S, np.int32),
                     np.stack([np.arange(B), off, np.zeros(B), np.full(B, S)], 1).astype(np.int32),
                     seed=seed)
    elif cfg == 3:
        B, S, D = 64, 8192, 256
        lens = np.full(B, S, np.int32)
        w = Workload(CONFIG_NAMES[3], 32, 8, D, B * 1024, B * S, True, 1 / math.sqrt(D),
                     (np.arange(B) * S).astype(np.int32), lens,
                     _rank_share_chunks(lens, 1024), seed=seed)
    elif cfg == 4:
        B, pitch, D = 16, 8192, 128
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = (64 * rng.integers(16, 129, size=B)).astype(np.int32)
        w = Workload(CONFIG_NAMES[4], 32, 8, D, B * 1024, B * pitch, True, 1 / math.sqrt(D),
                     (np.arange(B) * pitch).astype(np.int32), lens,
                     _rank_share_chunks(lens, 1024), seed=seed)
        # the length draw advanced a separate generator; tensors use the main seed stream
    elif cfg == 5:
        N, L, H, D = 1024, 1024, 4, 32
        off = (np.arange(N) * L).astype(np.int32)
        w = Workload(CONFIG_NAMES[5], H, H, D, N * L, N * L, False, 1 / math.sqrt(D),
                     off, np.full(N, L, np.int32),
                     np.stack([np.arange(N), off, np.zeros(N), np.full(N, L)], 1).astype(np.int32),
                     bias_len=L, seed=seed)
    else:
        raise ValueError(f"unknown config {cfg}")
    return _finish(w, materialize, poison_padding)


def make_custom(*, lens, hq, hkv, head_dim, causal=True, chunks=None, kv_pitch=None,
                q_pitch=None, bias=False, seed=0, scale=None, pad_kv_rows=0, pad_q_rows=0,
                materialize=True, poison_padding=True) -> Workload:
    """A small workload for sweeps.

    lens: sequence lengths.  K/V rows of sequence b start at b*kv_pitch
    (default: packed back to back).  chunks: list of (seq, pos0, len) triples;
    their Q rows are packed in order, each sequence's chunks starting at
    b*q_pitch when q_pitch is given.  Default: one full-length chunk per
    sequence.
    """
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    if kv_pitch is None:
        off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
        kv_rows = int(lens.sum()) + pad_kv_rows
    else:
        off = (np.arange(B) * kv_pitch).astype(np.int32)
        kv_rows = B * kv_pitch + pad_kv_rows
    if chunks is None:
        chunks = [(b, 0, int(lens[b])) for b in range(B)]
    rows = []
    r = 0
    last_seq = -1
    for (s, p0, n) in chunks:
        if q_pitch is not None and s != last_seq:
            r = max(r, s * q_pitch)
        rows.append((s, r, p0, n))
        r += n
        last_seq = s
    q_rows = (max(r, B * q_pitch) if q_pitch is not None else r) + pad_q_rows
    blen = int(lens.max()) if bias else 0
    w = Workload("custom", hq, hkv, head_dim, q_rows, kv_rows, causal,
                 (1 / math.sqrt(head_dim)) if scale is None else scale,
                 off, lens, np.asarray(rows, np.int32).reshape(-1, 4), bias_len=blen, seed=seed)
    return _finish(w, materialize, poison_padding)


def bhsd_shape(B: int, H: int, S_pitch: int, D: int):
    return (B, H, S_pitch, D)


def make_bhsd(B: int, H: int, S_pitch: int, D: int, seed: int) -> np.ndarray:
    """BF16 bits of a [B, H, S_pitch, D] tensor for the layout-copy path."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return draw_bf16(rng, (B, H, S_pitch, D))


def subset(w: Workload, seqs=None, chunks=None):
    """A compact copy of part of a workload (pure re-indexing, no arithmetic).

    Keeps the given sequences with all their chunks, or the sequences named by an
    explicit chunk list.  Returns (sub, q_index, kv_index): sub's Q row i is row
    q_index[i] of w, and its K/V row j is row kv_index[j] of w.
    """
    if chunks is None:
        keep = set(range(w.num_seqs)) if seqs is None else set(int(s) for s in seqs)
        chunks = [tuple(int(x) for x in c) for c in w.chunks if int(c[0]) in keep]
        seq_ids = sorted(keep)
    else:
        chunks = [tuple(int(x) for x in c) for c in chunks]
        seq_ids = sorted(set(c[0] for c in chunks)) if seqs is None else sorted(set(int(s) for s in seqs))
    seq_map = {s: i for i, s in enumerate(seq_ids)}
    kv_parts, offs, lens = [], [], []
    n = 0
    for s in seq_ids:
        o, L = int(w.seq_offsets[s]), int(w.seq_lens[s])
        offs.append(n)
        lens.append(L)
        kv_parts.append(np.arange(o, o + L, dtype=np.int64))
        n += L
    kv_index = np.concatenate(kv_parts) if kv_parts else np.zeros(0, np.int64)
    chunks = sorted(chunks, key=lambda c: (seq_map[c[0]], c[1]))
    q_parts, new_chunks = [], []
    r = 0
    for (s, r0, p0, ln) in chunks:
        new_chunks.append((seq_map[s], r, p0, ln))
        q_parts.append(np.arange(r0, r0 + ln, dtype=np.int64))
        r += ln
    q_index = np.concatenate(q_parts) if q_parts else np.zeros(0, np.int64)
    sub = Workload(w.name + "[subset]", w.hq, w.hkv, w.head_dim, len(q_index), len(kv_index),
                   w.causal, w.scale, np.asarray(offs, np.int32), np.asarray(lens, np.int32),
                   np.asarray(new_chunks, np.int32).reshape(-1, 4), bias_len=w.bias_len, seed=w.seed)
    if w.q is not None:
        sub.q, sub.do = w.q[q_index], w.do[q_index]
        sub.k, sub.v = w.k[kv_index], w.v[kv_index]
        sub.bias = w.bias
    return sub, q_index, kv_index


def draw_on_device(w: Workload, seed: int, device="cuda", poison_padding: bool = True):
    """Full-size inputs drawn on the GPU: N(0,1) float32 from a seeded torch
    generator, rounded to BF16 (round to nearest even), NaN in padding rows.

    Same shapes and distribution as the host draws, for workloads too large to
    draw on the host quickly.  Returns torch tensors (q, k, v, do, bias)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = out.view(-1)
        step = 1 << 26
        for s in range(0, flat.numel(), step):
            e = min(flat.numel(), s + step)
            flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        return out

    q = draw((w.q_rows, w.hq, w.head_dim))
    k = draw((w.kv_rows, w.hkv, w.head_dim))
    v = draw((w.kv_rows, w.hkv, w.head_dim))
    do = draw((w.q_rows, w.hq, w.head_dim))
    bias = None
    if w.bias_len:
        bias = torch.randn((w.hq, w.bias_len, w.bias_len), generator=g, device=device)
    if poison_padding:
        qpad = torch.from_numpy(~w.q_valid_rows()).to(device)
        kpad = torch.from_numpy(~w.kv_valid_rows()).to(device)
        for t, m in ((q, qpad), (do, qpad), (k, kpad), (v, kpad)):
            if bool(m.any()):
                t[m] = float("nan")
    return q, k, v, do, bias


def a2a_rank_maps(seq_lens, cp: int, pad_rows: int = 0):
    """Chunk maps of the load-balanced rank shares of an all-to-all (A2A) swap.

    Every sequence is cut into 2 cp chunks, chunk k covering positions
    [floor(k L / 2cp), floor((k + 1) L / 2cp)); rank r holds chunks r and
    2cp - 1 - r of every sequence, packed back to back in sequence order from row 0
    of its block.  Returns (maps, rows_per_rank): maps[r] is int32 [2 B, 4] of
    {seq, q_row, pos0, len} and rows_per_rank the longest rank's row count plus
    `pad_rows` (every block of the exchange has that many rows)."""
    lens = np.asarray(seq_lens, np.int64)
    n = 2 * cp
    maps, most = [], 0
    for r in range(cp):
        rows, q = [], 0
        for b, L in enumerate(lens):
            for k in (r, n - 1 - r):
                p0, p1 = (k * L) // n, ((k + 1) * L) // n
                rows.append((b, q, p0, p1 - p0))
                q += p1 - p0
        maps.append(np.asarray(rows, np.int32).reshape(-1, 4))
        most = max(most, q)
    return maps, most + pad_rows


def make_a2a(lens, H: int, D: int, cp: int, seed: int, kv_pitch=None, pad_rows: int = 0,
             pad_block_rows: int = 0):
    """A sequence-ordered THD tensor [rows, H, D] (BF16 bits, NaN padding) and the A2A
    rank maps over it: dict(full, seq_offsets, seq_lens, maps, rows_per_rank)."""
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    if kv_pitch is None:
        off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
        rows = int(lens.sum()) + pad_rows
    else:
        off = (np.arange(B) * kv_pitch).astype(np.int32)
        rows = B * kv_pitch + pad_rows
    rng = np.random.Generator(np.random.PCG64(seed))
    full = draw_bf16(rng, (rows, H, D))
    valid = np.zeros(rows, bool)
    for o, L in zip(off, lens):
        valid[o:o + L] = True
    full[~valid] = BF16_NAN
    maps, rpr = a2a_rank_maps(lens, cp, pad_block_rows)
    return dict(full=full, seq_offsets=off, seq_lens=lens, maps=maps, rows_per_rank=rpr, valid=valid)
