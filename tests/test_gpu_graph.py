"""The layer forward captured in a HIP graph (torch.cuda.graph) and replayed:
every replay must give exactly the eager result (all kernels are
deterministic), with other GPU work and synchronisations between replays.
The forward enqueues kernels only (no memset or copy nodes)."""
import pytest
import torch

from group_limited_top_amd import synth

from gpu_helpers import DEV, L, make_layer

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)


def _outputs(d, dt):
    return dict(y=torch.empty(d.T, d.H, dtype=dt, device=DEV),
                idx=torch.empty(d.T, d.top_k, dtype=torch.int32, device=DEV),
                w=torch.empty(d.T, d.top_k, dtype=torch.float32, device=DEV),
                counts=torch.empty(d.E, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("name", ["full_t512", "full_t16k_bias"])
def test_graph_replay_matches_eager(name):
    shape = synth.WORKLOADS[name]
    say("graph replay", name)
    Lb = L()
    dev = make_layer(shape)
    d = Lb.desc_from_shape(shape)
    weights = {k: dev[k] for k in ("w_router", "expert_bias", "w_gate", "w_up", "w_down",
                                   "ws_gate", "ws_up", "ws_down")}
    ws = Lb.alloc_workspace(d, DEV)
    ref = _outputs(d, dev["x"].dtype)
    Lb.moe_layer_forward(d, dev["x"], weights, ref["y"], ref["idx"], ref["w"], None,
                         ref["counts"], None, ws)
    torch.cuda.synchronize()

    got = _outputs(d, dev["x"].dtype)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Lb.moe_layer_forward(d, dev["x"], weights, got["y"], got["idx"], got["w"], None,
                             got["counts"], None, ws)
    other = _outputs(d, dev["x"].dtype)
    for r in range(3):
        for t in got.values():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (name, r, k)
        # eager work on the same workspace between replays
        Lb.moe_layer_forward(d, dev["x"], weights, other["y"], other["idx"], other["w"], None,
                             other["counts"], None, ws)
        torch.cuda.synchronize()
        assert torch.equal(other["y"], ref["y"])
    assert Lb.moe_status(ws) == 0
