"""C ABI checks that need no GPU: exports, descriptor validation, sizes.

None of these calls reaches a HIP runtime function that needs a device:
descriptor checks fail before the device is looked up, and the size and
view helpers are host-only.
"""
import ctypes
import os
import re
import subprocess

import pytest

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^EP_API\s+[\w\s\*]*?\b(ep_\w+)\s*\(", text, re.M)))


def test_header_declares_every_binding():
    assert header_functions() == sorted(ep.EXPORTS)


def test_library_exports_exactly_the_header():
    out = subprocess.run(["nm", "-D", "--defined-only", ep.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("ep_")})
    assert exported == header_functions()
    for name in header_functions():
        assert getattr(ep.lib(), name) is not None


def test_library_is_gfx950():
    """The embedded device code object targets gfx950 only."""
    blob = open(ep.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob
    for other in (b"--gfx942", b"--gfx90a", b"--gfx1100"):
        assert other not in blob


def _desc(**kw):
    base = dict(n_ranks=4, tokens=16, hidden=256, n_experts=16, topk=2, payload=0, cap_rows=0)
    base.update(kw)
    return ep.make_desc(**base)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_bound_matches_oracle_and_page_formula(name):
    sh = W.CONFIGS[name]
    d = ep.make_desc(sh.n_ranks, sh.tokens, sh.hidden, sh.n_experts, sh.topk, sh.payload)
    assert ep.recv_bound(d) == oracle.recv_bound(sh.n_ranks, sh.tokens, sh.n_experts, sh.topk)
    assert ep.capacity(d) == ep.recv_bound(d)
    d.cap_rows = 1000
    assert ep.capacity(d) == 1000


def test_row_bytes_and_planes():
    d = _desc()
    assert ep.num_planes(d) == 1 and ep.row_bytes(d, 0) == 512 and ep.row_bytes(d, 1) == 0
    d = _desc(hidden=7168, payload=ep.EP_PAYLOAD_FP8_B128)
    assert ep.num_planes(d) == 2
    assert ep.row_bytes(d, 0) == 7168 and ep.row_bytes(d, 1) == 224


@pytest.mark.parametrize("bad,code", [
    (dict(n_ranks=0), ep.EP_ERR_INVALID_ARG),
    (dict(n_experts=15), ep.EP_ERR_INVALID_ARG),           # E % N != 0
    (dict(hidden=250), ep.EP_ERR_INVALID_ARG),             # 16-byte bf16 rows
    (dict(hidden=200, payload=1), ep.EP_ERR_INVALID_ARG),  # fp8 blocks of 128
    (dict(payload=7), ep.EP_ERR_INVALID_ARG),
    (dict(cap_rows=-1), ep.EP_ERR_INVALID_ARG),
    (dict(topk=0), ep.EP_ERR_INVALID_ARG),
    (dict(tokens=-1), ep.EP_ERR_INVALID_ARG),
    (dict(n_experts=4096, n_ranks=4), ep.EP_ERR_UNSUPPORTED),
    (dict(topk=65, n_experts=128), ep.EP_ERR_UNSUPPORTED),
    (dict(n_ranks=64, tokens=1 << 20, topk=8, n_experts=512), ep.EP_ERR_UNSUPPORTED),
    # 2^23 slots of 14 KB rows: 14 pieces each, over 2^26 waves in one copy
    (dict(n_ranks=64, tokens=8192, topk=16, n_experts=256, hidden=7168),
     ep.EP_ERR_UNSUPPORTED),
])
def test_invalid_descriptors_fail_fast(bad, code):
    d = _desc(**bad)
    assert ep.recv_bound(d) == -1
    assert ep.plan_bytes(d) == 0
    fake = 0x10000
    for fn, args in [
        (ep.lib().ep_plan, (ctypes.byref(d), fake, fake, fake, None)),
        (ep.lib().ep_dispatch_pack, (ctypes.byref(d), None, fake, None, None)),
        (ep.lib().ep_dispatch_recv, (ctypes.byref(d), None, fake, None, None)),
        (ep.lib().ep_dispatch_transfer, (ctypes.byref(d), None, fake, None, None)),
        (ep.lib().ep_dispatch_unpack, (ctypes.byref(d), None, fake, None, None)),
        (ep.lib().ep_expert_stub, (ctypes.byref(d), None, None, fake, fake, None)),
        (ep.lib().ep_combine, (ctypes.byref(d), fake, fake, fake, fake, None)),
    ]:
        assert fn(*args) == code
        assert ep.last_error() != ""


# ep_probe_pattern's argument checks, all taken before the device lookup:
# (rows, indexed_rows, row_bytes, piece_bytes, fan_in, in_flight, mode, flags, waves).
@pytest.mark.parametrize("args,code", [
    ((4, 4, 14336, 1024, 1, 1, 5, 0, 0), ep.EP_ERR_INVALID_ARG),          # unknown mode
    ((4, 4, 14336, 1024, 1, 1, 0, 8, 0), ep.EP_ERR_INVALID_ARG),          # unknown flag
    ((-1, 4, 14336, 1024, 1, 1, 0, 0, 0), ep.EP_ERR_INVALID_ARG),         # negative rows
    ((4, 4, 14336, 1000, 1, 1, 0, 0, 0), ep.EP_ERR_INVALID_ARG),          # piece not 1 KB steps
    ((4, 4, 14336, 4096, 1, 1, 0, 0, 0), ep.EP_ERR_INVALID_ARG),          # piece does not divide row
    ((4, 12, 14336, 1024, 3, 1, 0, 0, 0), ep.EP_ERR_INVALID_ARG),         # fan_in 3
    ((4, 32, 14336, 1024, 8, 3, 0, 0, 0), ep.EP_ERR_INVALID_ARG),         # in_flight 3
    ((4, 32, 14336, 1024, 2, 4, 0, 0, 0), ep.EP_ERR_INVALID_ARG),         # in_flight > fan_in
    ((4, 4, 14336, 1024, 2, 2, 1, 0, 0), ep.EP_ERR_INVALID_ARG),          # fan_in on a fill
    ((4, 4, 14336, 1024, 1, 1, 0, 2, 64), ep.EP_ERR_INVALID_ARG),         # XCD order + grid-stride
    ((4, 7, 14336, 1024, 2, 2, 0, 0, 0), ep.EP_ERR_INVALID_ARG),          # linear inputs short
    ((4, 32, 14336, 1024, 8, 2, 3, 0, 0), ep.EP_ERR_INVALID_ARG),         # scatter in_flight 2
    ((4, 31, 14336, 1024, 8, 1, 3, 0, 0), ep.EP_ERR_INVALID_ARG),         # scatter targets short
    ((1 << 22, 4, 1 << 20, 1024, 1, 1, 1, 0, 0), ep.EP_ERR_UNSUPPORTED),  # 2^32 pieces
])
def test_probe_pattern_rejects_bad_shapes(args, code):
    fake = 0x10000
    assert ep.lib().ep_probe_pattern(fake, fake, None, *args, None) == code
    assert ep.last_error() != ""


def test_null_descriptor():
    assert ep.lib().ep_plan(None, None, None, None, None) == ep.EP_ERR_INVALID_ARG
    assert ep.lib().ep_recv_bound(None) == -1


def test_plan_views_layout():
    d = _desc(n_ranks=8, tokens=4096, hidden=7168, n_experts=256, topk=8)
    base = 1 << 20
    v = ep.plan_views(d, base)
    N, E, L, NTR = 8, 256, 32, 8 * 4096 * 8
    names = ["cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos", "src_off",
             "comb_row", "grp_slot", "send_slot", "recv_rows", "send_seg"]
    sizes = [N * E, N * (E + 1), NTR, N * (N + 1), N * (L + 1), NTR, N * E, NTR, NTR, NTR,
             2 * NTR, NTR]
    ptrs = [getattr(v, n) for n in names]
    assert ptrs[0] == base
    for p, q, n in zip(ptrs, ptrs[1:], sizes):
        assert (p - base) % 256 == 0
        assert q - p >= 4 * n                      # no overlap
    assert ep.plan_bytes(d) >= ptrs[-1] - base + 4 * NTR


def test_status_strings():
    for c in [0, -1, -2, -3, -4, 1, 2, 3, 4, 99]:
        assert isinstance(ep.status_string(c), str) and ep.status_string(c)


def test_oracle_and_library_share_nothing():
    """The oracle builds from its own sources and never names the library."""
    osrc = open(os.path.join(ROOT, "oracle", "ep_oracle.c")).read()
    assert "ep.h" not in osrc and "combine_ep_plan_amd" not in osrc
    for f in os.listdir(os.path.join(ROOT, "combine_ep_plan_amd", "csrc")):
        text = open(os.path.join(ROOT, "combine_ep_plan_amd", "csrc", f)).read()
        assert "oracle" not in text.lower(), f
    pkg = open(os.path.join(ROOT, "combine_ep_plan_amd", "__init__.py")).read()
    assert "import oracle" not in pkg and "from oracle" not in pkg


# (N, T, H, R, payload) -> (W, nwin) by the rule the header states for the
# windowed sender: more than 4 and at most 32 MiB of token rows per source,
# all send buffers at most 2 GiB, W the largest power of two whose rows fit
# 4 MiB. bf16 H = 2048 gives 4 KiB rows.
WINDOW_CASES = [
    ((2, 1024, 2048, 2, 0), (0, 0)),          # exactly 4 MiB per source
    ((2, 1025, 2048, 2, 0), (1024, 2)),       # one row more
    ((2, 8192, 2048, 2, 0), (1024, 8)),       # exactly 32 MiB
    ((2, 8193, 2048, 2, 0), (0, 0)),          # one row more
    ((63, 1025, 2048, 8, 0), (1024, 2)),      # send buffers just under 2 GiB
    ((64, 1025, 2048, 8, 0), (0, 0)),         # just over
    ((2, 600, 7168, 8, 1), (512, 2)),         # fp8: 7168 + 224 bytes per token
]


@pytest.mark.parametrize("args,want", WINDOW_CASES)
def test_window_list_view_follows_the_stated_rule(args, want):
    N, T, H, R, payload = args
    d = ep.make_desc(N, T, H, 16 * N, R, payload)
    base = 1 << 30
    v = ep.plan_views(d, base)
    W_, nwin = want
    if W_ == 0:
        assert not v.win_list
        return
    assert v.win_list and (v.win_list - base) % 256 == 0
    NTR = N * T * R
    assert v.win_list >= v.send_seg + 4 * NTR           # after the last table
    assert ep.plan_bytes(d) >= v.win_list - base + 8 * N * nwin * W_ * R


def test_binding_rejects_strided_views():
    """The library reads every buffer as dense row-major bytes, so the binding
    refuses a strided view before anything reaches the C ABI."""
    import torch

    a = torch.zeros((8, 16), dtype=torch.int16)
    assert ep._addr(a) == a.data_ptr()
    assert ep._addr(a[2:5]) == a[2:5].data_ptr()          # a row slice stays dense
    assert ep._addr(None) is None and ep._addr(0x1000) == 0x1000
    for view in (a.t(), a[:, ::2], a[:, 3:7]):
        with pytest.raises(ValueError, match="not contiguous"):
            ep._addr(view)
    with pytest.raises(ValueError, match="not contiguous"):
        ep._planes([a, a.t()])


def test_copy_grid_bound_counts_1kb_pieces():
    """The copies launch one wave per 1 KB piece of every slot's row, so the
    accepted sizes keep N T R times the pieces per row under 2^26 (one
    launch under 2^32 work-items)."""
    ok = _desc(n_ranks=64, tokens=4096, topk=16, n_experts=256, hidden=7168)   # 2^22 x 14
    assert ep.plan_bytes(ok) > 0 and ep.recv_bound(ok) > 0
    fp8 = _desc(n_ranks=64, tokens=8192, topk=16, n_experts=256, hidden=7168, payload=1)
    assert ep.plan_bytes(fp8) == 0            # 2^23 x (7 + 1) pieces
    narrow = _desc(n_ranks=64, tokens=8192, topk=7, n_experts=256, hidden=256)
    assert ep.plan_bytes(narrow) > 0          # 512-byte rows: one piece each
