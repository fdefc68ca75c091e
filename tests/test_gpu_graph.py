"""The dispatch + combine step captured into a HIP graph (torch.cuda.CUDAGraph)
and replayed several times, with eager work and synchronisations between
replays: every replay must equal the eager result. The library enqueues
only kernels (no memset or copy nodes), so the captured step is the same
launches."""
import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import ep_workloads as W
from gpu_util import plan_fields, desc_of, note, plan_arrays, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_zipf", "decode"])
def test_graph_replays_equal_eager(name):
    sh = W.CONFIGS[name]
    wl = W.make_workload(sh)
    d = desc_of(sh)
    note(f"graph {name}")
    b = ep.Buffers(d)
    upload(b, wl)
    alpha = torch.from_numpy(wl.alpha).cuda() if wl.alpha is not None else None
    b.status.zero_()
    ep.dispatch(d, b.idx, b.x, b.plan_ws, b.send, b.grouped, b.status)
    ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out)
    ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out)
    torch.cuda.synchronize()
    want_tables = plan_arrays(d, b)
    want_out = b.out.clone()
    want_grouped = [g.clone() for g in b.grouped] if name == "tiny_zipf" else None

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ep.dispatch(d, b.idx, b.x, b.plan_ws, b.send, b.grouped, b.status)
        ep.expert_stub(d, b.grouped, alpha, b.plan_ws, b.expert_out)
        ep.combine(d, b.expert_out, b.weights, b.plan_ws, b.out)
    for rep in range(4):
        # eager work between replays: scramble every output
        b.plan_ws.fill_(rep + 1)
        b.out.fill_(rep)
        for t in b.grouped:
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(b.status.item()) == 0
        got = plan_arrays(d, b)
        for f in plan_fields(d):
            np.testing.assert_array_equal(got[f], want_tables[f], err_msg=f"{f} replay {rep}")
        assert torch.equal(b.out, want_out), f"replay {rep}"
        if want_grouped is not None:
            totals = want_tables["recv_off"][:, d.n_ranks]
            for t, wt in zip(b.grouped, want_grouped):
                for dd in range(d.n_ranks):
                    n = int(totals[dd])
                    assert torch.equal(t[dd, :n], wt[dd, :n])
