"""Pins of the A2A swap-copy oracle (CPU only).

The pins tie oracle/a2a.py to what the head <-> sequence swap must achieve,
written without the oracle's per-row loops: after split_heads, the exchange and
scatter_rows, rank j holds every row of every sequence for its head slice
[j H/cp, (j+1) H/cp) of the sequence-ordered tensor (NumPy slicing of the global
tensor, ranks built by concatenating slices); the way back returns each rank's
own rows with all heads.  Round trips, untouched rows, cp = 1, and planted
mistakes complete them."""
import numpy as np
import pytest

import oracle.a2a as A
import workloads as W

CASES = [
    dict(lens=[16, 10], H=4, D=8, cp=2),
    dict(lens=[24, 7, 33], H=8, D=16, cp=4, kv_pitch=40, pad_rows=3),
    dict(lens=[12], H=6, D=8, cp=3, pad_block_rows=2),
    dict(lens=[9, 30, 5, 16], H=8, D=8, cp=8),
]


def _setup(c, seed=11):
    kw = {k: c[k] for k in ("kv_pitch", "pad_rows", "pad_block_rows") if k in c}
    return W.make_a2a(c["lens"], c["H"], c["D"], c["cp"], seed, **kw)


def _rank_positions(L, cp, r):
    """Positions rank r holds of a sequence of length L: chunks r and 2cp-1-r of 2cp."""
    n = 2 * cp
    cut = [(k * L) // n for k in range(n + 1)]
    return list(range(cut[r], cut[r + 1])) + list(range(cut[n - 1 - r], cut[n - r]))


def _local(a, r, H):
    """Rank r's rows with all heads, built from the global tensor by slicing."""
    parts = [a["full"][o + np.asarray(_rank_positions(int(L), len(a["maps"]), r), np.int64)]
             for o, L in zip(a["seq_offsets"], a["seq_lens"])]
    loc = np.concatenate(parts, 0) if parts else np.zeros((0, H, a["full"].shape[2]), np.uint16)
    pad = np.full((a["rows_per_rank"] - loc.shape[0],) + loc.shape[1:], W.BF16_NAN, np.uint16)
    return np.concatenate([loc, pad], 0)


def _exchange(sends):
    """The all-to-all: block j of rank s's send buffer becomes block s of rank j's."""
    cp = len(sends)
    return [np.stack([sends[s][j] for s in range(cp)], 0) for j in range(cp)]


@pytest.mark.parametrize("c", CASES)
def test_sequence_to_head_swap_gives_every_rank_whole_sequences_of_its_heads(c):
    a = _setup(c)
    cp, H = c["cp"], c["H"]
    Hc = H // cp
    sends = [A.split_heads(_local(a, r, H), cp) for r in range(cp)]
    recvs = _exchange(sends)
    valid = a["valid"]
    for j in range(cp):
        sentinel = np.full(a["full"][:, :Hc].shape, 0x1234, np.uint16)
        got = A.scatter_rows(recvs[j], a["maps"], a["seq_offsets"], sentinel)
        np.testing.assert_array_equal(got[valid], a["full"][valid][:, j * Hc:(j + 1) * Hc])
        assert np.all(got[~valid] == 0x1234), "rows outside every sequence were written"


@pytest.mark.parametrize("c", CASES)
def test_head_to_sequence_swap_returns_each_rank_its_rows_with_all_heads(c):
    a = _setup(c, seed=12)
    cp, H = c["cp"], c["H"]
    Hc = H // cp
    blank = np.full((cp, a["rows_per_rank"], Hc, c["D"]), 0x1234, np.uint16)
    sends = [A.gather_rows(a["full"][:, j * Hc:(j + 1) * Hc], a["maps"], a["seq_offsets"], blank)
             for j in range(cp)]
    recvs = _exchange(sends)
    for r in range(cp):
        got = A.merge_heads(recvs[r])
        n = int(a["maps"][r][:, 3].sum())
        np.testing.assert_array_equal(got[:n], _local(a, r, H)[:n])
        assert np.all(got[n:] == 0x1234), "padding rows of a block were written"


@pytest.mark.parametrize("c", CASES)
def test_round_trips(c):
    a = _setup(c, seed=13)
    cp, H = c["cp"], c["H"]
    x = a["full"]
    np.testing.assert_array_equal(A.merge_heads(A.split_heads(x, cp)), x)
    Hc = H // cp
    blocks = np.random.Generator(np.random.PCG64(5)).integers(0, 1 << 16, (cp, a["rows_per_rank"], Hc, c["D"]),
                                                              dtype=np.uint16)
    full = A.scatter_rows(blocks, a["maps"], a["seq_offsets"], np.zeros(x[:, :Hc].shape, np.uint16))
    back = A.gather_rows(full, a["maps"], a["seq_offsets"], np.zeros_like(blocks))
    for r in range(cp):
        n = int(a["maps"][r][:, 3].sum())  # rank r's rows are packed from row 0
        np.testing.assert_array_equal(back[r, :n], blocks[r, :n])


def test_one_rank_is_a_plain_copy():
    a = _setup(dict(lens=[10, 6], H=4, D=8, cp=1))
    np.testing.assert_array_equal(A.split_heads(a["full"], 1)[0], a["full"])
    loc = _local(a, 0, 4)
    got = A.scatter_rows(loc[None], a["maps"], a["seq_offsets"], np.zeros_like(a["full"]))
    np.testing.assert_array_equal(got[a["valid"]], a["full"][a["valid"]])


def test_planted_mistakes_are_caught():
    """Plausible slips in the copies break the swap pin."""
    c = CASES[1]
    a = _setup(c)
    cp, H = c["cp"], c["H"]
    Hc = H // cp

    def swap_ok(split, scatter):
        recvs = _exchange([split(_local(a, r, H), cp) for r in range(cp)])
        for j in range(cp):
            got = scatter(recvs[j], a["maps"], a["seq_offsets"], np.zeros(a["full"][:, :Hc].shape, np.uint16))
            if not np.array_equal(got[a["valid"]], a["full"][a["valid"]][:, j * Hc:(j + 1) * Hc]):
                return False
        return True

    def split_strided(local, cp):  # heads dealt round-robin instead of in blocks
        rows, H, D = local.shape
        return np.stack([local[:, j::cp] for j in range(cp)], 0)

    def scatter_off_by_one(recv, maps, offs, out):
        shifted = [m.copy() for m in maps]
        for m in shifted:
            m[:, 2] += 1
            m[:, 3] = np.maximum(0, m[:, 3] - 1)
        return A.scatter_rows(recv, shifted, offs, out)

    def scatter_ranks_swapped(recv, maps, offs, out):
        return A.scatter_rows(recv[::-1], maps, offs, out)

    assert swap_ok(A.split_heads, A.scatter_rows)
    assert not swap_ok(split_strided, A.scatter_rows)
    assert not swap_ok(A.split_heads, scatter_off_by_one)
    assert not swap_ok(A.split_heads, scatter_ranks_swapped)
