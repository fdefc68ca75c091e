"""The relay that allocates nothing: ep_kv_push_staged_static (bounce slots
in the library's static device array) against ep_kv_push_staged with a
caller-allocated device bounce buffer. Destination pools must be byte
identical, with the same completion count and status, over two calls in a
row on one GPU, the second on a smaller request (the static slots still
hold the first call's bytes)."""
import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
import oracle
from gpu_util import note

pytestmark = pytest.mark.gpu


def _case(sh):
    src_t, dst_t = W.make_kv_tables(sh)
    reg = ep.kv_plan(sh.tokens, sh.token_bytes, sh.src_block_tokens, src_t, sh.dst_block_tokens,
                     dst_t)
    sb = sh.src_pool_blocks * sh.src_block_tokens * sh.token_bytes
    db = sh.dst_pool_blocks * sh.dst_block_tokens * sh.token_bytes
    g = torch.Generator().manual_seed(sh.seed + 7)
    src = torch.randint(0, 256, (sh.ranks, sb), dtype=torch.uint8, generator=g)
    dst = torch.randint(0, 256, (sh.ranks, db), dtype=torch.uint8, generator=g)
    want = oracle.kv_copy(oracle.kv_regions(sh.tokens, sh.token_bytes, sh.src_block_tokens,
                                            src_t, sh.dst_block_tokens, dst_t),
                          src.numpy(), dst.numpy())
    return reg, src.cuda(), dst.cuda(), want


def _push(sh, reg, src, dst, slots, static):
    reg_dev = torch.from_numpy(np.ascontiguousarray(reg, dtype=np.int64)).cuda()
    total = int(reg[:, 2].sum())
    notify = torch.zeros(1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if static:
        ep.kv_push_staged_static(sh.ranks, reg_dev, len(reg), total, src, src.shape[1], dst,
                                 dst.shape[1], slots, notify, status)
    else:
        bounce = torch.empty(slots * 32768, dtype=torch.uint8, device="cuda")
        ep.kv_push_staged(sh.ranks, reg_dev, len(reg), total, src, src.shape[1], dst,
                          dst.shape[1], bounce, slots, notify, status)
    torch.cuda.synchronize()
    return int(notify.item()), int(status.item())


# First a request of 8 MiB per rank (four rounds of 64 slots), then a small
# one through a single slot.
CALLS = [
    (W.KvShape("kv_big_tokens", 4, 200, 40960, 1, 1, 300, 300, 16.0, 4.0, seed=4), 64),
    (W.KV_CONFIGS["kv_tiny"], 1),
]


def test_static_relay_matches_caller_bounce_two_calls():
    for sh, slots in CALLS:
        note(f"static relay {sh.name} ranks={sh.ranks} tokens={sh.tokens} slots={slots}")
        reg, src, dst, want = _case(sh)
        dst_ref = dst.clone()
        got = _push(sh, reg, src, dst, slots, static=True)
        ref = _push(sh, reg, src, dst_ref, slots, static=False)
        assert got == ref == (sh.ranks, 0)
        assert torch.equal(dst, dst_ref)
        np.testing.assert_array_equal(dst.cpu().numpy(), want)


def test_static_relay_rejects_more_slots_than_it_holds():
    sh = W.KV_CONFIGS["kv_tiny"]
    reg, src, dst, _ = _case(sh)
    reg_dev = torch.from_numpy(reg).cuda()
    z = torch.zeros(2, dtype=torch.int32, device="cuda")
    total = int(reg[:, 2].sum())
    for slots in (0, ep.EP_KV_STATIC_SLOTS + 1):
        with pytest.raises(ep.EPError) as e:
            ep.kv_push_staged_static(2, reg_dev, len(reg), total, src, src.shape[1], dst,
                                     dst.shape[1], slots, z[:1], z[1:])
        assert e.value.code == ep.EP_ERR_INVALID_ARG and "64" in str(e.value)
    torch.cuda.synchronize()
    assert int(z.sum().item()) == 0          # nothing was enqueued
