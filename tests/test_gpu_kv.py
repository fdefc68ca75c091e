"""KV-block push on the GPU: planner regions copied by the device push and
by the staged relay, against the CPU oracle (byte exact), with completion
counting. Full-size requests are checked on the device against a
token-by-token gather with torch indexing."""
import gc

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _pool_bytes(sh, side):
    if side == "src":
        return sh.src_pool_blocks * sh.src_block_tokens * sh.token_bytes
    return sh.dst_pool_blocks * sh.dst_block_tokens * sh.token_bytes


def push(sh, reg, src, dst, mode="direct", slots=64, host_bounce=False):
    """Run one push; returns (notify, status)."""
    ranks = sh.ranks
    reg_dev = torch.from_numpy(np.ascontiguousarray(reg, dtype=np.int64)).cuda()
    total = int(reg[:, 2].sum()) if len(reg) else 0
    notify = torch.zeros(1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sb, db = src.shape[1], dst.shape[1]
    if mode == "direct":
        ep.kv_push(ranks, reg_dev, len(reg), total, src, sb, dst, db, notify, status)
    else:
        bounce = torch.empty(slots * 32768, dtype=torch.uint8,
                             pin_memory=host_bounce, device="cpu" if host_bounce else "cuda")
        ep.kv_push_staged(ranks, reg_dev, len(reg), total, src, sb, dst, db, bounce, slots,
                          notify, status)
    torch.cuda.synchronize()
    return int(notify.item()), int(status.item())


def _small_case(sh, merge=True):
    src_t, dst_t = W.make_kv_tables(sh)
    reg = ep.kv_plan(sh.tokens, sh.token_bytes, sh.src_block_tokens, src_t, sh.dst_block_tokens,
                     dst_t, merge=merge)
    g = torch.Generator().manual_seed(sh.seed + 1)
    src = torch.randint(0, 256, (sh.ranks, _pool_bytes(sh, "src")), dtype=torch.uint8, generator=g)
    dst = torch.randint(0, 256, (sh.ranks, _pool_bytes(sh, "dst")), dtype=torch.uint8, generator=g)
    want = oracle.kv_copy(oracle.kv_regions(sh.tokens, sh.token_bytes, sh.src_block_tokens, src_t,
                                            sh.dst_block_tokens, dst_t), src.numpy(), dst.numpy())
    return reg, src.cuda(), dst.cuda(), want


SMALL = [
    W.KV_CONFIGS["kv_tiny"],
    W.KvShape("kv_mixed_blocks", 3, 500, 32, 16, 4, 64, 300, 3.0, 2.0, seed=2),
    W.KvShape("kv_tiny_tokens_fragmented", 2, 3000, 16, 1, 1, 4000, 4000, 1.0, 1.0, seed=3),
    W.KvShape("kv_big_tokens", 4, 200, 40960, 1, 1, 300, 300, 16.0, 4.0, seed=4),
    W.KvShape("kv_odd_blocks", 1, 77, 48, 3, 5, 60, 40, 2.0, 2.0, seed=5),
]
MODES = [("direct", 64, False), ("staged", 64, False), ("staged", 1, False), ("staged", 4, True)]


@pytest.mark.parametrize("sh", SMALL, ids=[s.name for s in SMALL])
@pytest.mark.parametrize("mode,slots,host", MODES, ids=["direct", "staged64", "staged1", "host4"])
def test_kv_push_matches_oracle(sh, mode, slots, host):
    note(f"kv {sh.name} {mode} slots={slots} host={host}")
    reg, src, dst, want = _small_case(sh)
    notify, status = push(sh, reg, src, dst, mode, slots, host)
    assert (notify, status) == (sh.ranks, 0)
    np.testing.assert_array_equal(dst.cpu().numpy(), want)


def test_kv_push_unmerged_descriptors_same_bytes():
    sh = SMALL[1]
    reg, src, dst, want = _small_case(sh, merge=False)
    assert push(sh, reg, src, dst) == (sh.ranks, 0)
    np.testing.assert_array_equal(dst.cpu().numpy(), want)


def test_kv_push_bad_region_is_skipped_and_flagged():
    sh = W.KV_CONFIGS["kv_tiny"]
    reg, src, dst, _ = _small_case(sh)
    before = dst.cpu().numpy()
    bad = reg.copy()
    bad[0, 1] = _pool_bytes(sh, "dst") - 16            # runs past the end of the pool
    notify, status = push(sh, bad, src, dst)
    assert status == ep.EP_STATUS_BAD_REGION and notify == sh.ranks
    good = oracle.kv_copy(reg[1:, :3], src.cpu().numpy(), before)
    np.testing.assert_array_equal(dst.cpu().numpy(), good)


def test_kv_push_empty_request_notifies():
    sh = W.KV_CONFIGS["kv_tiny"]
    src = torch.zeros((2, 64), dtype=torch.uint8, device="cuda")
    dst = torch.zeros((2, 64), dtype=torch.uint8, device="cuda")
    reg = np.zeros((0, 4), np.int64)
    assert push(sh, reg, src, dst) == (2, 0)
    assert push(sh, reg, src, dst, "staged", 2) == (2, 0)


def test_kv_push_rejects_bad_arguments():
    sh = W.KV_CONFIGS["kv_tiny"]
    reg, src, dst, _ = _small_case(sh)
    reg_dev = torch.from_numpy(reg).cuda()
    z = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(ep.EPError):
        ep.kv_push(0, reg_dev, len(reg), 64, src, src.shape[1], dst, dst.shape[1], z, z)
    with pytest.raises(ep.EPError):
        ep.kv_push(2, reg_dev, len(reg), 24, src, src.shape[1], dst, dst.shape[1], z, z)
    with pytest.raises(ep.EPError):
        ep.kv_push_staged(2, reg_dev, len(reg), 64, src, src.shape[1], dst, dst.shape[1],
                          torch.empty(32768, dtype=torch.uint8, device="cuda"), 65, z, z)
    with pytest.raises(ep.EPError):                     # pageable host bounce
        ep.kv_push_staged(2, reg_dev, len(reg), 64, src, src.shape[1], dst, dst.shape[1],
                          torch.empty(32768, dtype=torch.uint8), 1, z, z)


@pytest.mark.parametrize("name,mode", [("kv_qwen32b_16k", "direct"), ("kv_qwen32b_16k", "staged"),
                                       ("kv_page1_4k", "direct")])
def test_kv_push_full_size(name, mode):
    """Whole request on the device: every token's block slot on the
    destination holds its source bytes (torch gather), nothing else is
    written; the planner's regions equal the oracle's."""
    sh = W.KV_CONFIGS[name]
    note(f"kv full-size {sh.name} {mode}")
    src_t, dst_t = W.make_kv_tables(sh)
    bs, bd, tok = sh.src_block_tokens, sh.dst_block_tokens, sh.token_bytes
    reg = ep.kv_plan(sh.tokens, tok, bs, src_t, bd, dst_t)
    np.testing.assert_array_equal(reg[:, :3], oracle.kv_regions(sh.tokens, tok, bs, src_t, bd,
                                                                dst_t))
    src = torch.randint(0, 256, (sh.ranks, _pool_bytes(sh, "src")), dtype=torch.uint8,
                        device="cuda")
    dst = torch.zeros((sh.ranks, _pool_bytes(sh, "dst")), dtype=torch.uint8, device="cuda")
    assert push(sh, reg, src, dst, mode) == (sh.ranks, 0)
    i = torch.arange(sh.tokens, device="cuda")
    st = torch.from_numpy(src_t.astype(np.int64)).cuda()[i // bs] * bs + i % bs
    dt = torch.from_numpy(dst_t.astype(np.int64)).cuda()[i // bd] * bd + i % bd
    sv = src.view(sh.ranks, -1, tok)
    dv = dst.view(sh.ranks, -1, tok)
    assert torch.equal(dv[:, dt], sv[:, st])
    untouched = torch.ones(dv.shape[1], dtype=torch.bool, device="cuda")
    untouched[dt] = False
    assert not dv[:, untouched].any()
