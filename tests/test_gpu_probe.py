"""The access-pattern probe moves the bytes it claims to (ep_probe_pattern).

The probe is a measurement reference, not a step of the method, so it has
no oracle: its results are checked against numpy definitions of each mode
(copy: xor of the named source rows; scatter: each source row at its named
output rows; fill: the pattern each wave writes; read: dst written only
where a lane's data xors to the key).
"""
import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep

pytestmark = pytest.mark.gpu

ROW = 14336      # one bf16 row of the decode hidden size
KEY = 0x9E3779B9


def rand_rows(rng, n, row=ROW):
    return rng.integers(0, 256, size=(n, row), dtype=np.uint8)


def run(dst, src, table, rows, indexed_rows, piece, fan_in=1, mode=ep.EP_PROBE_COPY, flags=0,
        waves=0, row=ROW, in_flight=0):
    ep.probe_pattern(dst, src, table, rows, indexed_rows, row, piece, fan_in=fan_in,
                     in_flight=in_flight, mode=mode, flags=flags, waves=waves)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


def xor_rows(a, idx):
    out = a[idx[:, 0]].copy()
    for j in range(1, idx.shape[1]):
        out ^= a[idx[:, j]]
    return out


@pytest.mark.parametrize("piece", [1024, 2048, 7168, 14336])
@pytest.mark.parametrize("flags,waves", [(0, 0), (ep.EP_PROBE_NT_LOADS, 0),
                                         (ep.EP_PROBE_XCD, 0), (0, 24),
                                         (ep.EP_PROBE_ONE_WAVE, 0),
                                         (ep.EP_PROBE_ONE_WAVE | ep.EP_PROBE_XCD, 0),
                                         (ep.EP_PROBE_ONE_WAVE | ep.EP_PROBE_NT_LOADS, 24)])
def test_linear_copy(piece, flags, waves):
    rng = np.random.default_rng(piece + flags + waves)
    rows = 37
    a = rand_rows(rng, rows)
    src = torch.from_numpy(a).cuda()
    dst = torch.zeros_like(src)
    got = run(dst, src, None, rows, rows, piece, flags=flags, waves=waves)
    assert np.array_equal(got, a)


@pytest.mark.parametrize("fan_in,in_flight,piece", [
    (1, 1, 1024), (2, 2, 7168), (4, 4, 2048), (8, 8, 1024), (8, 8, 2048), (8, 8, 14336),
    (8, 2, 7168), (8, 1, 14336), (4, 2, 2048)])
def test_table_copy_and_mix(fan_in, in_flight, piece):
    rng = np.random.default_rng(fan_in * 100 + in_flight * 10 + piece)
    rows, src_rows = 29, 53
    a = rand_rows(rng, src_rows)
    idx = rng.integers(0, src_rows, size=(rows, fan_in)).astype(np.int32)
    idx[3, 0] = src_rows + 5     # outside the source: row 0 is read
    idx[7, -1] = -2
    want_idx = np.where((idx >= 0) & (idx < src_rows), idx, 0)
    src = torch.from_numpy(a).cuda()
    table = torch.from_numpy(idx).cuda()
    dst = torch.zeros((rows, ROW), dtype=torch.uint8, device="cuda")
    got = run(dst, src, table, rows, src_rows, piece, fan_in, flags=ep.EP_PROBE_XCD,
              in_flight=in_flight)
    assert np.array_equal(got, xor_rows(a, want_idx))
    dst.zero_()
    got = run(dst, src, table, rows, src_rows, piece, fan_in,
              flags=ep.EP_PROBE_ONE_WAVE | ep.EP_PROBE_NT_LOADS, in_flight=in_flight)
    assert np.array_equal(got, xor_rows(a, want_idx))


def test_linear_mix_of_eight_regions():
    rng = np.random.default_rng(8)
    rows = 41
    a = rand_rows(rng, 8 * rows)
    src = torch.from_numpy(a).cuda()
    dst = torch.zeros((rows, ROW), dtype=torch.uint8, device="cuda")
    got = run(dst, src, None, rows, 8 * rows, 7168, 8, flags=ep.EP_PROBE_NT_LOADS, in_flight=2)
    want = xor_rows(a, np.arange(rows)[:, None] + rows * np.arange(8)[None, :])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("piece,flags", [(1024, ep.EP_PROBE_NT_LOADS), (14336, 0),
                                         (2048, ep.EP_PROBE_XCD)])
def test_scatter(piece, flags):
    rng = np.random.default_rng(piece + 7 * flags)
    rows, fan, out_rows = 23, 8, 23 * 8
    a = rand_rows(rng, rows)
    # Every output row named once (a send order), two of them out of range.
    idx = rng.permutation(out_rows).astype(np.int32).reshape(rows, fan)
    src = torch.from_numpy(a).cuda()
    dst = torch.zeros((out_rows, ROW), dtype=torch.uint8, device="cuda")
    got = run(dst, src, torch.from_numpy(idx).cuda(), rows, out_rows, piece, fan,
              mode=ep.EP_PROBE_SCATTER, flags=flags)
    want = np.zeros_like(got)
    for i in range(rows):
        for k in range(fan):
            want[idx[i, k]] = a[i]
    assert np.array_equal(got, want)
    # Without a table, row i goes to rows i * fan .. i * fan + fan - 1; an
    # entry outside the output (row 0 stands in) lands on row 0.
    dst.zero_()
    got = run(dst, src, None, rows, out_rows, piece, fan, mode=ep.EP_PROBE_SCATTER, flags=flags)
    assert np.array_equal(got, np.repeat(a, fan, axis=0))
    idx2 = np.arange(out_rows, dtype=np.int32).reshape(rows, fan)
    idx2[5, 3] = out_rows + 9
    dst.zero_()
    got = run(dst, src, torch.from_numpy(idx2).cuda(), rows, out_rows, piece, fan,
              mode=ep.EP_PROBE_SCATTER, flags=flags)
    want = np.repeat(a, fan, axis=0)
    want[5 * fan + 3] = 0
    assert np.array_equal(got[1:], want[1:])
    # Row 0 is written by two sources; each piece holds one of them.
    assert np.all((got[0] == a[0]) | (got[0] == a[5]))


@pytest.mark.parametrize("piece,flags", [(1024, 0), (7168, ep.EP_PROBE_NT_LOADS)])
def test_scatter_wide(piece, flags):
    """Source rows twice as long: output chunk c = source chunk 2c xor 2c + 1."""
    rng = np.random.default_rng(piece + 3)
    rows, fan, out_rows, row = 19, 8, 19 * 8, 7168
    a = rand_rows(rng, rows, 2 * row)
    idx = rng.permutation(out_rows).astype(np.int32).reshape(rows, fan)
    src = torch.from_numpy(a).cuda()
    dst = torch.zeros((out_rows, row), dtype=torch.uint8, device="cuda")
    got = run(dst, src, torch.from_numpy(idx).cuda(), rows, out_rows, piece, fan,
              mode=ep.EP_PROBE_SCATTER_WIDE, flags=flags, row=row)
    c = a.reshape(rows, -1, 2, 16)
    narrow = (c[:, :, 0] ^ c[:, :, 1]).reshape(rows, row)
    want = np.zeros_like(got)
    for i in range(rows):
        for k in range(fan):
            want[idx[i, k]] = narrow[i]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("flags", [0, ep.EP_PROBE_ONE_WAVE])
@pytest.mark.parametrize("piece,waves", [(1024, 0), (4096, 0), (65536, 0), (1024, 40)])
def test_fill_pattern(piece, waves, flags):
    row = 65536
    rows = 5
    dst = torch.zeros((rows, row), dtype=torch.uint8, device="cuda")
    got = run(dst, None, None, rows, 0, piece, mode=ep.EP_PROBE_FILL, waves=waves,
              row=row, flags=flags).view(np.uint32).reshape(-1, 4)
    chunk = np.arange(rows * row // 16)
    per_piece = piece // 16
    w = chunk // per_piece
    lane = (chunk % per_piece) % 64
    want = np.stack([w, lane, np.full_like(w, 0x5A5A5A5A), np.zeros_like(w)], 1)
    assert np.array_equal(got, want.astype(np.uint32))


def test_read_writes_only_for_the_key():
    rows = 9
    a = np.zeros((rows, ROW), np.uint8)
    src = torch.from_numpy(a).cuda()
    dst = torch.zeros(64, dtype=torch.int32, device="cuda")
    got = run(dst, src, None, rows, rows, 1024, mode=ep.EP_PROBE_READ)
    assert not got.any()
    # Lane 5 of the wave on row 2's piece 3 sees the key in its chunk.
    words = a.view(np.uint32).reshape(rows, -1, 4)
    words[2, 3 * 64 + 5, 1] = KEY
    src = torch.from_numpy(a).cuda()
    table = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    got = run(dst, src, table, 3, rows, 1024, mode=ep.EP_PROBE_READ,
              flags=ep.EP_PROBE_NT_LOADS)
    want = np.zeros(64, np.uint32)
    want[5] = KEY
    assert np.array_equal(got.view(np.uint32), want)


def test_zero_rows_is_a_no_op():
    dst = torch.zeros(256, dtype=torch.uint8, device="cuda")
    ep.probe_pattern(dst, None, None, 0, 0, ROW, 1024)
    torch.cuda.synchronize()
    assert not dst.any()
