"""moe_layer_forward_noalloc (the layer forward with the library's static
per-device scratch buffer, for callers that cannot allocate) against
moe_layer_forward with a caller's workspace: the same kernels, so every
output must be bit-identical.  Two calls in a row, the second with fewer
tokens (the buffer keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from group_limited_top_amd import synth

from gpu_helpers import DEV, L, make_layer

pytestmark = pytest.mark.gpu


def _outputs(shape):
    T, H, E, K = shape.T, shape.H, shape.E, shape.top_k
    return dict(y=torch.full((T, H), float("nan"), dtype=shape.torch_dtype, device=DEV),
                idx=torch.full((T, K), -7, dtype=torch.int32, device=DEV),
                w=torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV),
                logits=torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV),
                counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
                tracking=torch.zeros(E, dtype=torch.int64, device=DEV))


def _weights(dev):
    return {k: dev[k] for k in ("w_router", "expert_bias", "w_gate", "w_up", "w_down",
                                "ws_gate", "ws_up", "ws_down")}


@pytest.mark.parametrize("name", ["full_t512", "tiny_f32"])
def test_noalloc_matches_workspace_entry_point(name):
    Lb = L()
    base = synth.WORKLOADS[name]
    # the workload's size, then a smaller batch of the same layer
    for T in (base.T, 200):
        shape = synth.LayerShape(base.name, T=T, H=base.H, I=base.I, I_shared=base.I_shared,
                                 dtype=base.dtype, bias="normal", seed=base.seed + T)
        print("[gpu-case] noalloc", name, "T", T, flush=True)
        dev = make_layer(shape)
        d = Lb.desc_from_shape(shape, flags=Lb.MOE_F_WRITE_LOGITS)
        assert Lb.workspace_size(d) <= Lb.MOE_NOALLOC_SCRATCH_BYTES
        ref = _outputs(shape)
        ws = Lb.alloc_workspace(d, DEV)
        Lb.moe_layer_forward(d, dev["x"], _weights(dev), ref["y"], ref["idx"], ref["w"],
                             ref["logits"], ref["counts"], ref["tracking"], ws)
        got = _outputs(shape)
        Lb.moe_layer_forward_noalloc(d, dev["x"], _weights(dev), got["y"], got["idx"], got["w"],
                                     got["logits"], got["counts"], got["tracking"])
        torch.cuda.synchronize()
        for k in ("y", "idx", "w", "logits", "counts", "tracking"):
            a, b = ref[k], got[k]
            if a.dtype.is_floating_point:
                a, b = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32), \
                    b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
            assert torch.equal(a, b), (name, T, k)
        assert Lb.moe_status(ws) == 0
        np.testing.assert_array_equal(got["counts"].cpu().numpy(),
                                      np.bincount(got["idx"].cpu().numpy().ravel(),
                                                  minlength=shape.E))
