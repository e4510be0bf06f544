"""C-ABI checks that need no GPU: the library loads, exports every declared symbol,
and rejects host-detectable contract violations before touching the device.

Every call below fails a host check, so no kernel is ever launched with the fake
addresses used here."""
import ctypes
import os
import re

import pytest

import context_causal_gqa_cpattn_amd as cp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(cp.LIB_PATH), reason="library not built")


def declared_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(cpattn_\w+)\s*\(", txt, re.M)))


def test_header_declares_what_the_binding_expects():
    assert declared_symbols() == sorted(cp.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = cp.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.cpattn_version() == 10100
    assert lib.cpattn_status_str(0) == b"CPATTN_OK"


A = 0x7f0000000000  # fake, 256-aligned base addresses: never dereferenced


def _prob(**kw):
    d = dict(num_seqs=2, hq=8, hkv=2, head_dim=128, q_rows=64, kv_rows=128, num_chunks=2,
             max_chunk_len=32, max_kv_len=64, causal=1, scale=0.088, bias_len=0)
    d.update(kw)
    return cp.Problem(**d)


def _fwd(prob, q=A, k=A + (1 << 24), v=A + (2 << 24), so=A + (3 << 24), sl=A + (3 << 24) + 256,
         cm=A + (3 << 24) + 512, bias=None, o=A + (4 << 24), lse=A + (5 << 24), err=A + (6 << 24)):
    lib = cp.load()
    return lib.cpattn_fwd(ctypes.byref(prob), q, k, v, so, sl, cm, bias, o, lse, None, 0, err, None)


def _err():
    return cp.load().cpattn_last_error().decode()


def test_rejects_bad_problems():
    assert _fwd(_prob(hq=6, hkv=4)) == cp.EINVAL and "multiple" in _err()
    assert _fwd(_prob(head_dim=96)) == cp.EUNSUPPORTED
    assert _fwd(_prob(head_dim=256, bias_len=64, causal=0)) == cp.EUNSUPPORTED
    assert _fwd(_prob(bias_len=64, causal=1)) == cp.EUNSUPPORTED
    assert _fwd(_prob(num_seqs=-1)) == cp.EINVAL
    assert _fwd(_prob(scale=float("nan"))) == cp.EINVAL
    assert _fwd(_prob(causal=2)) == cp.EINVAL
    lib = cp.load()
    assert lib.cpattn_fwd(None, A, A, A, A, A, A, None, A, A, None, 0, A, None) == cp.EINVAL


def test_rejects_null_and_misaligned_pointers():
    assert _fwd(_prob(), q=None) == cp.EINVAL and "q is NULL" in _err()
    assert _fwd(_prob(), o=A + (4 << 24) + 2) == cp.EINVAL and "aligned" in _err()
    assert _fwd(_prob(), cm=A + (3 << 24) + 520) == cp.EINVAL  # chunk map needs 16 bytes
    assert _fwd(_prob(), err=None) == cp.EINVAL
    assert _fwd(_prob(), bias=A + (7 << 24)) == cp.EINVAL and "bias_len is 0" in _err()


def test_alias_audit_rejects_overlapping_outputs():
    # O overlapping Q
    assert _fwd(_prob(), o=A + 4096) == cp.EINVAL and "alias" in _err()
    # LSE overlapping O
    assert _fwd(_prob(), lse=A + (4 << 24) + 256) == cp.EINVAL and "alias" in _err()
    # dev_err inside the chunk map
    assert _fwd(_prob(), err=A + (3 << 24) + 512 + 16) == cp.EINVAL and "alias" in _err()


def test_bwd_rejects_small_workspace_and_aliases():
    lib = cp.load()
    p = _prob()
    need = lib.cpattn_workspace_size(ctypes.byref(p), cp.OP_BWD)
    assert need >= 8 * 64 * 4 and need % 256 == 0
    base = [ctypes.byref(p), A, A + (1 << 24), A + (2 << 24), A + (3 << 24), A + (3 << 24) + 256,
            A + (3 << 24) + 512, None, A + (4 << 24), A + (5 << 24), A + (8 << 24),
            A + (9 << 24), A + (10 << 24), A + (11 << 24), None, 0]
    tail = [A + (12 << 24), need - 4, A + (6 << 24), None]
    assert lib.cpattn_bwd(*base, *tail) == cp.EINVAL and "workspace" in _err()
    bad = list(base)
    bad[12] = A + (1 << 24)  # dk == k
    assert lib.cpattn_bwd(*bad, A + (12 << 24), need, A + (6 << 24), None) == cp.EINVAL
    assert "alias" in _err()
    bad = list(base)
    bad[15] = 2  # dkv_accumulate must be 0/1
    assert lib.cpattn_bwd(*bad, A + (12 << 24), need, A + (6 << 24), None) == cp.EINVAL


def _ws_layout(hq, q_rows, num_chunks, head_dim):
    """Backward workspace bytes without dBias partials, from the layout the header states."""
    r256 = lambda x: (x + 255) // 256 * 256
    tiles = -(-q_rows // 32) + num_chunks
    return (r256(hq * q_rows * 4) + 2 * r256(tiles * hq * head_dim * 32 * 2)
            + r256(tiles * hq * 64 * 4))


def test_workspace_sizes():
    lib = cp.load()
    p = _prob()
    assert lib.cpattn_workspace_size(ctypes.byref(p), cp.OP_FWD) == 0
    assert lib.cpattn_workspace_size(ctypes.byref(p), cp.OP_BWD) == _ws_layout(8, 64, 2, 128)
    p3 = _prob(num_seqs=64, hq=32, hkv=8, head_dim=256, q_rows=64 * 1024, kv_rows=64 * 8192,
               num_chunks=128, max_chunk_len=512, max_kv_len=8192)
    assert lib.cpattn_workspace_size(ctypes.byref(p3), cp.OP_BWD) == _ws_layout(32, 64 * 1024, 128, 256)
    pb = _prob(head_dim=32, bias_len=1024, causal=0, hq=4, hkv=4, num_chunks=1024, q_rows=1 << 20,
               kv_rows=1 << 20)
    ws = lib.cpattn_workspace_size(ctypes.byref(pb), cp.OP_BWD)
    assert ws >= _ws_layout(4, 1 << 20, 1024, 32) + 4 * 1024 * 1024 * 4  # + one partial slab
    assert lib.cpattn_workspace_size(ctypes.byref(_prob(hq=3)), cp.OP_BWD) == 0


def test_backward_steps_check_workspace():
    lib = cp.load()
    p = _prob()
    core = _ws_layout(8, 64, 2, 128)
    q, k, v = A, A + (1 << 24), A + (2 << 24)
    so, sl, cm = A + (3 << 24), A + (3 << 24) + 256, A + (3 << 24) + 512
    o, lse, do, err, ws = A + (4 << 24), A + (5 << 24), A + (8 << 24), A + (6 << 24), A + (12 << 24)
    dk, dv, dq = A + (9 << 24), A + (10 << 24), A + (11 << 24)
    assert lib.cpattn_bwd_prepass(ctypes.byref(p), q, cm, o, do, lse, ws, core - 256, err, None) == cp.EINVAL
    assert "workspace" in _err()
    assert lib.cpattn_bwd_prepass(ctypes.byref(p), q, cm, o, do, lse, ws + 16, core, err, None) == cp.EINVAL
    assert lib.cpattn_bwd_prepass(ctypes.byref(p), q, cm, o, do, lse, o, core, err, None) == cp.EINVAL
    assert "alias" in _err()
    args = [ctypes.byref(p), q, k, v, so, sl, cm, None, lse, do]
    assert lib.cpattn_bwd_dkdv(*args, ws, core - 1, dk, dv, 0, err, None) == cp.EINVAL
    assert lib.cpattn_bwd_dkdv(*args, ws, core, ws + 4096, dv, 0, err, None) == cp.EINVAL
    assert "alias" in _err()
    assert lib.cpattn_bwd_dkdv(*args, ws, core, dk, dv, 3, err, None) == cp.EINVAL
    assert lib.cpattn_bwd_dq(*args, ws, core - 1, dq, err, None) == cp.EINVAL
    assert lib.cpattn_bwd_dq(*args, ws, core, do, err, None) == cp.EINVAL and "alias" in _err()
    assert lib.cpattn_bwd_dbias(*args, ws, core, A + (13 << 24), err, None) == cp.EINVAL
    assert "bias" in _err()


def test_layout_copy_host_checks():
    lib = cp.load()
    assert lib.cpattn_pack(A, A + (1 << 24), 2, 4, 64, 12, 128, A + (2 << 24), A + (2 << 24) + 256,
                           A + (3 << 24), None) == cp.EUNSUPPORTED  # D % 8
    assert lib.cpattn_pack(A, A + 64, 2, 4, 64, 128, 128, A + (2 << 24), A + (2 << 24) + 256,
                           A + (3 << 24), None) == cp.EINVAL  # dst overlaps src
    assert lib.cpattn_unpack(None, A, 2, 4, 64, 128, 128, A + (2 << 24), A + (2 << 24) + 256,
                             A + (3 << 24), None) == cp.EINVAL


def _ds_bytes(hq, q_rows, num_chunks, max_kv_len, ds_blocks=0):
    """dS store bytes from the layout the header states: the chunks' int64 offsets, then
    2 KB per (chunk tile, head, 32-key block), ds_blocks blocks per head when given, else
    every tile slot sized for max_kv_len."""
    r256 = lambda x: (x + 255) // 256 * 256
    tiles = -(-q_rows // 32) + num_chunks
    blocks = ds_blocks if ds_blocks else tiles * (-(-max_kv_len // 32))
    return r256(num_chunks * 8) + 2048 + r256(blocks * hq * 2048)


def test_stored_ds_workspace_size():
    lib = cp.load()
    p = _prob()
    assert lib.cpattn_workspace_size(ctypes.byref(p), cp.OP_BWD_DS) == \
        _ws_layout(8, 64, 2, 128) + _ds_bytes(8, 64, 2, 64)
    p3 = _prob(num_seqs=64, hq=32, hkv=8, head_dim=256, q_rows=64 * 1024, kv_rows=64 * 8192,
               num_chunks=128, max_chunk_len=512, max_kv_len=8192)
    ds3 = _ds_bytes(32, 64 * 1024, 128, 8192)
    assert ds3 == 36_507_222_016 + 1024 + 2048  # the figure the header quotes (+ offsets, zeros)
    assert lib.cpattn_workspace_size(ctypes.byref(p3), cp.OP_BWD_DS) == \
        _ws_layout(32, 64 * 1024, 128, 256) + ds3
    # with the chunks' bound: two 512-row chunks per 8192-key sequence, at its start
    # (16 key blocks) and end (256 key blocks), 16 tiles each
    chunks = [(b, 1024 * b + 512 * j, 7680 * j, 512) for b in range(64) for j in range(2)]
    dsb = cp.ds_blocks(chunks, [8192] * 64, causal=True)
    assert dsb == 64 * (16 * 16 + 16 * 256)
    p3.ds_blocks = dsb
    ds3b = _ds_bytes(32, 64 * 1024, 128, 8192, dsb)
    assert ds3b == 18_253_614_080  # the figure the header quotes
    assert lib.cpattn_workspace_size(ctypes.byref(p3), cp.OP_BWD_DS) == \
        _ws_layout(32, 64 * 1024, 128, 256) + ds3b
    # without causal masking every chunk keeps all of its sequence's key blocks
    assert cp.ds_blocks(chunks, [8192] * 64, causal=False) == 128 * 16 * 256
    p3.ds_blocks = -1
    assert lib.cpattn_workspace_size(ctypes.byref(p3), cp.OP_BWD_DS) == 0
    # after the dBias partial sums when there is a bias
    pb = _prob(head_dim=64, bias_len=256, causal=0, hq=4, hkv=4, num_chunks=64, q_rows=1 << 14,
               kv_rows=1 << 14, max_chunk_len=256, max_kv_len=256)
    assert lib.cpattn_workspace_size(ctypes.byref(pb), cp.OP_BWD_DS) == \
        lib.cpattn_workspace_size(ctypes.byref(pb), cp.OP_BWD) + _ds_bytes(4, 1 << 14, 64, 256)
    # head_dim 32 too (the pair-bias rows); not for an invalid problem
    assert lib.cpattn_workspace_size(ctypes.byref(_prob(head_dim=32)), cp.OP_BWD_DS) == \
        _ws_layout(8, 64, 2, 32) + _ds_bytes(8, 64, 2, 64)
    assert lib.cpattn_workspace_size(ctypes.byref(_prob(hq=3)), cp.OP_BWD_DS) == 0


def test_stored_ds_steps_check_workspace_and_aliases():
    lib = cp.load()
    p = _prob()
    core = _ws_layout(8, 64, 2, 128)
    full = lib.cpattn_workspace_size(ctypes.byref(p), cp.OP_BWD_DS)
    q, k, v = A, A + (1 << 24), A + (2 << 24)
    so, sl, cm = A + (3 << 24), A + (3 << 24) + 256, A + (3 << 24) + 512
    lse, do, err, ws = A + (5 << 24), A + (8 << 24), A + (6 << 24), A + (12 << 24)
    dk, dv, dq = A + (9 << 24), A + (10 << 24), A + (11 << 24)
    args = [ctypes.byref(p), q, k, v, so, sl, cm, None, lse, do]
    assert lib.cpattn_bwd_dkdv_ds(*args, ws, full - 1, dk, dv, 0, err, None) == cp.EINVAL
    assert "workspace" in _err()
    assert lib.cpattn_bwd_dkdv_ds(*args, ws, full, ws + core + 4096, dv, 0, err, None) == cp.EINVAL
    assert "alias" in _err()  # dK inside the dS store
    assert lib.cpattn_bwd_dkdv_ds(*args, ws, full, dk, dv, 2, err, None) == cp.EINVAL
    assert lib.cpattn_bwd_dq_ds(ctypes.byref(p), k, so, sl, cm, ws, full - 1, dq, err, None) == cp.EINVAL
    assert "workspace" in _err()
    assert lib.cpattn_bwd_dq_ds(ctypes.byref(p), k, so, sl, cm, ws, full, ws + core + 512, err,
                                None) == cp.EINVAL
    assert "alias" in _err()  # dQ over the dS it reads
    assert lib.cpattn_bwd_dq_ds(ctypes.byref(p), k, so, sl, cm, ws + 16, full, dq, err, None) == cp.EINVAL
    # head_dim 32 has a dS store as well: its size is checked the same way
    p32 = _prob(head_dim=32)
    full32 = lib.cpattn_workspace_size(ctypes.byref(p32), cp.OP_BWD_DS)
    args32 = [ctypes.byref(p32)] + args[1:]
    assert lib.cpattn_bwd_dkdv_ds(*args32, ws, full32 - 1, dk, dv, 0, err, None) == cp.EINVAL
    assert "workspace" in _err()
    assert lib.cpattn_bwd_dq_ds(ctypes.byref(p32), k, so, sl, cm, ws, full32 - 1, dq, err, None) == cp.EINVAL
    assert "workspace" in _err()


def test_window_and_merge_host_checks():
    lib = cp.load()
    p = _prob()
    q, k, v = A, A + (1 << 24), A + (2 << 24)
    so, sl, cm = A + (3 << 24), A + (3 << 24) + 256, A + (3 << 24) + 512
    o, lse, do, err, ws = A + (4 << 24), A + (5 << 24), A + (8 << 24), A + (6 << 24), A + (12 << 24)
    dk, dv, dq = A + (9 << 24), A + (10 << 24), A + (11 << 24)
    fa = [ctypes.byref(p), q, k, v, so, sl, cm, None]
    assert lib.cpattn_fwd_window(*fa, -1, 10, o, lse, err, None) == cp.EINVAL and "window" in _err()
    assert lib.cpattn_fwd_window(*fa, 10, 5, o, lse, err, None) == cp.EINVAL and "window" in _err()
    assert lib.cpattn_fwd_window(*fa, 0, 10, q + 4096, lse, err, None) == cp.EINVAL and "alias" in _err()
    # merge: in place on (o_a, lse_a) is allowed by the host checks; other overlaps are not
    o2, l2 = A + (13 << 24), A + (14 << 24)
    assert lib.cpattn_merge(ctypes.byref(p), cm, o, lse, o2, l2, o2 + 4096, lse, err, None) == cp.EINVAL
    assert "alias" in _err()
    assert lib.cpattn_merge(ctypes.byref(p), cm, o, lse, o2, l2, o, l2, err, None) == cp.EINVAL
    assert "alias" in _err()
    assert lib.cpattn_merge(ctypes.byref(p), cm, o, lse, None, l2, o, lse, err, None) == cp.EINVAL
    core = _ws_layout(8, 64, 2, 128)
    ba = [ctypes.byref(p), q, k, v, so, sl, cm, None, o, lse, do]
    assert lib.cpattn_bwd_window(*ba, 5, 1, 1, dq, 0, dk, dv, 0, ws, core, err, None) == cp.EINVAL
    assert lib.cpattn_bwd_window(*ba, 0, 8, 2, dq, 0, dk, dv, 0, ws, core, err, None) == cp.EINVAL
    assert lib.cpattn_bwd_window(*ba, 0, 8, 1, dq, 0, dk, dv, 0, ws, core - 1, err, None) == cp.EINVAL
    assert "workspace" in _err()
    assert lib.cpattn_bwd_window(*ba, 0, 8, 1, dk + 64, 0, dk, dv, 0, ws, core, err, None) == cp.EINVAL
    assert "alias" in _err()


def test_head_pitch_bounds():
    assert _fwd(_prob(q_head_pitch=4)) == cp.EINVAL and "pitch" in _err()
    assert _fwd(_prob(kv_head_pitch=1)) == cp.EINVAL and "pitch" in _err()
    assert _fwd(_prob(q_head_pitch=-1)) == cp.EINVAL
    assert _fwd(_prob(q_head_pitch=4097)) == cp.EUNSUPPORTED and "4096" in _err()
    # a head slice's span: rows 0..q_rows-1 at pitch 16 heads end 8 heads into the last row
    hd = 128 * 2
    span = (63 * 16 + 8) * hd
    assert _fwd(_prob(q_head_pitch=16), o=A + span - 16) == cp.EINVAL and "alias" in _err()


def _bwd_alias_msg(prob, q, k, v, dq, dk, dv):
    """The alias error of a backward call whose workspace overlaps seq_offsets on purpose
    (so the call never gets past its host checks): it names the first overlapping
    output in the order dq, dk, dv, ws."""
    lib = cp.load()
    need = lib.cpattn_workspace_size(ctypes.byref(prob), cp.OP_BWD)
    so, sl, cm = A + (3 << 24), A + (3 << 24) + 256, A + (3 << 24) + 512
    o, lse, do, err = A + (4 << 24), A + (5 << 24), A + (8 << 24), A + (6 << 24)
    r = lib.cpattn_bwd(ctypes.byref(prob), q, k, v, so, sl, cm, None, o, lse, do, dq, dk, dv, None, 0, so,
                       need, err, None)
    assert r == cp.EINVAL
    return _err()


def test_alias_audit_is_exact_for_head_slices_of_one_tensor():
    hd = 128 * 2
    p = _prob(q_head_pitch=16, kv_head_pitch=4)
    q, k = A, A + (1 << 24)
    dk, dv = A + (9 << 24), A + (10 << 24)
    last = "output ws overlaps input seq_offsets"
    # dQ as the other 8 heads of Q's 16-head tensor shares no byte with Q
    for dq in (q + 8 * hd, q + 24 * hd):
        msg = _bwd_alias_msg(p, q, k, k + 2 * hd, dq, dk, dv)
        assert last in msg, msg
    # interleaved slices that do share heads or rows are found
    for dq in (q + 4 * hd, q + 16 * hd, q + 31 * hd):
        msg = _bwd_alias_msg(p, q, k, k + 2 * hd, dq, dk, dv)
        assert "output dq overlaps input q" in msg, msg
    # K and V as the two halves of one packed [rows, 2 hkv, D] tensor, and dK, dV the same
    msg = _bwd_alias_msg(p, q, k, k + 2 * hd, A + (11 << 24), dk, dk + 2 * hd)
    assert last in msg, msg
    msg = _bwd_alias_msg(p, q, k, k + 2 * hd, A + (11 << 24), dk, dk + 1 * hd)
    assert "output dk overlaps output dv" in msg, msg


def test_a2a_copy_host_checks():
    lib = cp.load()
    src, dst = A, A + (1 << 24)
    assert lib.cpattn_a2a_split_heads(src, dst, 64, 6, 128, 4, None) == cp.EINVAL and "multiple" in _err()
    assert lib.cpattn_a2a_split_heads(src, dst, 64, 8, 100, 4, None) == cp.EUNSUPPORTED
    assert lib.cpattn_a2a_split_heads(src, src + 4096, 64, 8, 128, 4, None) == cp.EINVAL and "alias" in _err()
    assert lib.cpattn_a2a_merge_heads(None, dst, 64, 8, 128, 4, None) == cp.EINVAL and "NULL" in _err()
    assert lib.cpattn_a2a_merge_heads(src + 8, dst, 64, 8, 128, 4, None) == cp.EINVAL and "aligned" in _err()
    assert lib.cpattn_a2a_split_heads(src, dst, -1, 8, 128, 4, None) == cp.EINVAL
    p = cp.A2aRows(cp=4, chunks_per_rank=2, num_seqs=1, max_chunk_len=8, rows_per_rank=16, full_rows=64,
                   heads=2, head_dim=128)
    maps, so, sl, err = A + (2 << 24), A + (3 << 24), A + (3 << 24) + 256, A + (6 << 24)
    f = lib.cpattn_a2a_scatter_rows
    assert f(ctypes.byref(p), src, src + 4096, maps, so, sl, err, None) == cp.EINVAL and "alias" in _err()
    assert f(ctypes.byref(p), src, dst, maps + 4, so, sl, err, None) == cp.EINVAL and "rank_maps" in _err()
    assert f(ctypes.byref(p), src, dst, maps, so, sl, maps + 16, None) == cp.EINVAL and "alias" in _err()
    assert f(ctypes.byref(p), src, dst, maps, so, sl, None, None) == cp.EINVAL
    assert f(None, src, dst, maps, so, sl, err, None) == cp.EINVAL
    bad = cp.A2aRows(cp=4, chunks_per_rank=2, num_seqs=1, max_chunk_len=8, rows_per_rank=16, full_rows=64,
                     heads=2, head_dim=12)
    assert f(ctypes.byref(bad), src, dst, maps, so, sl, err, None) == cp.EUNSUPPORTED
    bad.head_dim, bad.rows_per_rank = 128, -1
    assert lib.cpattn_a2a_gather_rows(ctypes.byref(bad), src, dst, maps, so, sl, err, None) == cp.EINVAL
