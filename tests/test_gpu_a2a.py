"""The A2A swap copies through the C-ABI vs the oracle (bit-exact; GPU).

Every case checks the four copies against oracle/a2a.py on the same bits, with the
destinations prefilled with a sentinel so that rows no chunk names are seen to keep
it; the emulated exchange (torch copies between the ranks' buffers) must give every
rank whole sequences of its head slice and back; broken rank maps fail closed; and
the copies at the CP4/A2A B64/S8192/Hq32/Hkv8/D128 rank share are checked on
sampled rows."""
import numpy as np
import pytest

import oracle.a2a as A
import workloads as W

pytestmark = pytest.mark.gpu

SENT = 0x1234  # a finite BF16 bit pattern

CASES = [
    dict(lens=[16, 10], H=4, D=8, cp=2),
    dict(lens=[24, 7, 33], H=8, D=16, cp=4, kv_pitch=40, pad_rows=3),
    dict(lens=[12], H=6, D=8, cp=3, pad_block_rows=2),
    dict(lens=[9, 30, 5, 16], H=8, D=8, cp=8),
    dict(lens=[300, 77, 129], H=32, D=128, cp=4, pad_rows=5, pad_block_rows=3),
    dict(lens=[260, 64], H=8, D=256, cp=4, kv_pitch=300),
    dict(lens=[1000, 24], H=8, D=128, cp=2),
]


def _setup(c, seed=21):
    kw = {k: c[k] for k in ("kv_pitch", "pad_rows", "pad_block_rows") if k in c}
    return W.make_a2a(c["lens"], c["H"], c["D"], c["cp"], seed, **kw)


def _local(a, r):
    """Rank r's block rows (all heads) taken from the global tensor by the oracle."""
    cp, rpr = len(a["maps"]), a["rows_per_rank"]
    H, D = a["full"].shape[1:]
    blank = np.full((cp, rpr, H, D), SENT, np.uint16)
    return A.gather_rows(a["full"], a["maps"], a["seq_offsets"], blank)[r]


def _dev(cp, bits):
    return cp.to_device_bf16(bits)


def _host(cp, t):
    return cp.to_host_bits(t)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_head_copies_match_the_oracle(gpu_lib, i):
    import torch
    cp, c = gpu_lib, CASES[i]
    a = _setup(c)
    x = a["full"]
    print(f"[case] a2a heads {i} rows={x.shape[0]} H={c['H']} D={c['D']} cp={c['cp']}", flush=True)
    send = cp.a2a_split_heads(_dev(cp, x), c["cp"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(cp, send), A.split_heads(x, c["cp"]))
    back = cp.a2a_merge_heads(send)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(cp, back), A.merge_heads(A.split_heads(x, c["cp"])))
    np.testing.assert_array_equal(_host(cp, back), x)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_row_copies_match_the_oracle(gpu_lib, i):
    import torch
    cp, c = gpu_lib, CASES[i]
    a = _setup(c, seed=22)
    Hc = c["H"] // c["cp"]
    print(f"[case] a2a rows {i} lens={c['lens']} Hc={Hc} D={c['D']} cp={c['cp']}", flush=True)
    lay = cp.make_a2a_layout(a["maps"], a["seq_offsets"], a["seq_lens"])
    rng = np.random.Generator(np.random.PCG64(9))
    blocks = rng.integers(0, 0x7F00, (c["cp"], a["rows_per_rank"], Hc, c["D"]), dtype=np.uint16)
    full0 = np.full((a["full"].shape[0], Hc, c["D"]), SENT, np.uint16)
    full, err = cp.a2a_scatter_rows(_dev(cp, blocks), lay, full0.shape[0], full=_dev(cp, full0))
    torch.cuda.synchronize()
    cp.check(err)
    np.testing.assert_array_equal(_host(cp, full), A.scatter_rows(blocks, a["maps"], a["seq_offsets"], full0))
    src = a["full"][:, :Hc].copy()
    blk0 = np.full(blocks.shape, SENT, np.uint16)
    got, err = cp.a2a_gather_rows(_dev(cp, src), lay, a["rows_per_rank"], blocks=_dev(cp, blk0))
    torch.cuda.synchronize()
    cp.check(err)
    np.testing.assert_array_equal(_host(cp, got), A.gather_rows(src, a["maps"], a["seq_offsets"], blk0))


@pytest.mark.parametrize("i", [1, 4, 5])
def test_emulated_swap_gives_whole_sequences_and_back(gpu_lib, i):
    import torch
    cp, c = gpu_lib, CASES[i]
    a = _setup(c, seed=23)
    n, H, D = c["cp"], c["H"], c["D"]
    Hc = H // n
    lay = cp.make_a2a_layout(a["maps"], a["seq_offsets"], a["seq_lens"])
    full = _dev(cp, a["full"])
    locals_ = [_dev(cp, _local(a, r)) for r in range(n)]
    sends = [cp.a2a_split_heads(x, n) for x in locals_]
    recvs = [torch.stack([sends[s][j] for s in range(n)]) for j in range(n)]  # the all-to-all
    valid = torch.from_numpy(np.flatnonzero(a["valid"])).cuda()
    outs = []
    for j in range(n):
        out, err = cp.a2a_scatter_rows(recvs[j], lay, full.shape[0])
        cp.check(err)
        assert torch.equal(out[valid].view(torch.int16), full[valid][:, j * Hc:(j + 1) * Hc].view(torch.int16))
        outs.append(out)
    # and back: each rank's head slice of whole sequences -> its own rows with all heads
    sends = [cp.a2a_gather_rows(outs[j], lay, a["rows_per_rank"])[0] for j in range(n)]
    recvs = [torch.stack([sends[j][r] for j in range(n)]) for r in range(n)]
    for r in range(n):
        got = cp.a2a_merge_heads(recvs[r])
        rows = int(a["maps"][r][:, 3].sum())
        assert torch.equal(got[:rows].view(torch.int16), locals_[r][:rows].view(torch.int16))


def test_broken_rank_maps_fail_closed(gpu_lib):
    import torch
    cp, c = gpu_lib, CASES[1]
    a = _setup(c, seed=24)
    Hc = c["H"] // c["cp"]
    blocks = _dev(cp, np.zeros((c["cp"], a["rows_per_rank"], Hc, c["D"]), np.uint16))
    bad_cases = [
        ("chunk past its block", lambda m: m[1].__setitem__((0, 1), a["rows_per_rank"] - 1), 0x08),
        ("chunk past its sequence", lambda m: m[2].__setitem__((1, 2), 10_000), 0x10),
        ("unknown sequence", lambda m: m[0].__setitem__((0, 0), 7), 0x04),
    ]
    for name, spoil, bit in bad_cases:
        maps = [m.copy() for m in a["maps"]]
        spoil(maps)
        lay = cp.make_a2a_layout(maps, a["seq_offsets"], a["seq_lens"])
        lay.max_chunk_len = max(lay.max_chunk_len, 1)
        full = torch.full((a["full"].shape[0], Hc, c["D"]), 3.0, dtype=torch.bfloat16, device="cuda")
        _, err = cp.a2a_scatter_rows(blocks, lay, full.shape[0], full=full)
        torch.cuda.synchronize()
        assert int(err.item()) & bit, name
        assert bool((full == 3.0).all()), f"{name}: rows were written"
    # sequences outside the full tensor
    lay = cp.make_a2a_layout(a["maps"], a["seq_offsets"] + 10_000, a["seq_lens"])
    full = torch.full((a["full"].shape[0], Hc, c["D"]), 3.0, dtype=torch.bfloat16, device="cuda")
    _, err = cp.a2a_scatter_rows(blocks, lay, full.shape[0], full=full)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x02 and bool((full == 3.0).all())


def test_cp4_rank_share_at_full_size_on_sampled_rows(gpu_lib):
    """CP4/A2A at B64/S8192/Hq32/Hkv8/D128: one rank's Q share [131072, 32, 128] split
    into 4 head groups, and 4 received blocks scattered into [524288, 8, 128]."""
    import torch
    cp = gpu_lib
    B, S, H, D, n = 64, 8192, 32, 128, 4
    lens = np.full(B, S, np.int32)
    offs = (np.arange(B) * S).astype(np.int32)
    maps, rpr = W.a2a_rank_maps(lens, n)
    assert rpr == B * S // n
    g = torch.Generator(device="cuda").manual_seed(31)
    x = torch.randn((rpr, H, D), generator=g, device="cuda").to(torch.bfloat16)
    send = cp.a2a_split_heads(x, n)
    torch.cuda.synchronize()
    rows = np.sort(np.random.Generator(np.random.PCG64(3)).choice(rpr, 512, replace=False))
    ti = torch.from_numpy(rows).cuda()
    np.testing.assert_array_equal(_host(cp, send[:, ti]), A.split_heads(_host(cp, x[ti]), n))
    # scatter: the received blocks of one rank (Hc = 8 heads) into whole sequences
    blocks = torch.randn((n, rpr, H // n, D), generator=g, device="cuda").to(torch.bfloat16)
    lay = cp.make_a2a_layout(maps, offs, lens)
    full, err = cp.a2a_scatter_rows(blocks, lay, B * S)
    torch.cuda.synchronize()
    cp.check(err)
    for b in (0, 17, 63):  # whole sequences, by the oracle on their rows only
        sub_maps = [m[m[:, 0] == b].copy() for m in maps]
        for m in sub_maps:
            m[:, 0] = 0
        rows_b = [np.concatenate([np.arange(q, q + ln) for (_, q, _, ln) in m]) for m in sub_maps]
        blk_b = np.stack([_host(cp, blocks[s][torch.from_numpy(r).cuda()]) for s, r in enumerate(rows_b)])
        for m in sub_maps:  # the sequence's rows of each block, packed from row 0
            m[:, 1] = np.concatenate([[0], np.cumsum(m[:-1, 3])])
        ref = A.scatter_rows(blk_b, sub_maps, [0], np.zeros((S, H // n, D), np.uint16))
        np.testing.assert_array_equal(_host(cp, full[b * S:(b + 1) * S]), ref)
