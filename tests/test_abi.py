"""libmoe's C ABI on the host: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments before any HIP call (so
these run without a GPU; no test here launches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    from group_limited_top_amd import _lib
    return _lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["moe_workspace_size", "moe_route", "moe_permute", "moe_experts",
              "moe_layer_forward", "moe_status", "moe_strerror"]:
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L.LIB, n), n
    assert set(declared_functions()) == set(L.EXPORTS)


def full_desc(L, **kw):
    base = dict(T=512, H=2048)
    base.update(kw)
    T, H = base.pop("T"), base.pop("H")
    return L.make_desc(T, H, **base)


def test_workspace_size(L):
    d = full_desc(L)
    n = L.LIB.moe_workspace_size(ctypes.byref(d))
    T, H, E, K, I = 512, 2048, 256, 8, 512
    P = T * K
    # at least the hidden and per-pair outputs of routed + shared rows, in bf16
    assert n >= 2 * (P * I + T * I + P * H + T * H)
    assert n < 2 * (P * I + T * I + P * H + T * H) + 16 * 2 ** 20
    assert n % 256 == 0
    bigger = L.LIB.moe_workspace_size(ctypes.byref(full_desc(L, T=1024)))
    assert bigger > n
    # T = 0 is valid
    assert L.LIB.moe_workspace_size(ctypes.byref(full_desc(L, T=0))) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(E=255), -1),                      # E not a multiple of n_group
    (dict(n_group=256, topk_group=4), -1),  # group size 1
    (dict(topk_group=9), -1),               # more kept groups than groups
    (dict(top_k=200), -1),                  # more experts than the kept groups hold
    (dict(T=-1), -1),
    (dict(I=0), -1),
    (dict(E=1024, n_group=8), -2),          # outside the kernels' envelope
    (dict(H=2000), -2),
    (dict(I=500), -2),
    (dict(I=2048), -2),
    (dict(top_k=17, topk_group=8), -2),
    (dict(n_group=128, topk_group=4), -2),
])
def test_invalid_descs_rejected(L, kw, code):
    d = full_desc(L, **kw)
    assert L.LIB.moe_workspace_size(ctypes.byref(d)) == 0
    rc = L.LIB.moe_route(ctypes.byref(d), None, None, None, None, None, None, None, 0, None)
    assert rc == code
    rc = L.LIB.moe_layer_forward(ctypes.byref(d), None, None, None, None, None, None, None, None,
                                 None, 0, None)
    assert rc == code


def test_bad_flags_and_dtype(L):
    d = full_desc(L)
    d.flags = 8
    assert L.LIB.moe_workspace_size(ctypes.byref(d)) == 0
    d = full_desc(L)
    d.dtype = 7
    assert L.LIB.moe_workspace_size(ctypes.byref(d)) == 0
    d = full_desc(L)
    d.routed_scaling_factor = float("nan")
    assert L.LIB.moe_workspace_size(ctypes.byref(d)) == 0


def test_null_and_workspace_errors(L):
    d = full_desc(L)
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: errors come first
    # required pointers missing
    assert L.LIB.moe_route(ctypes.byref(d), None, fake, None, None, fake, fake, fake, 1 << 40,
                           None) == -1
    # workspace too small / missing
    assert L.LIB.moe_route(ctypes.byref(d), fake, fake, None, None, fake, fake, fake, 16,
                           None) == -3
    assert L.LIB.moe_route(ctypes.byref(d), fake, fake, None, None, fake, fake, None, 1 << 40,
                           None) == -3
    # misaligned pointers
    odd = ctypes.c_void_p(0x100004)
    assert L.LIB.moe_route(ctypes.byref(d), odd, fake, None, None, fake, fake, fake, 1 << 40,
                           None) == -4
    # y aliasing x
    W = L.MoeWeights(fake, None, fake, fake, fake, fake, fake, fake)
    assert L.LIB.moe_layer_forward(ctypes.byref(d), fake, ctypes.byref(W), fake, None, None, None,
                                   None, None, fake, 1 << 40, None) == -1
    # shared-expert weights must match I_shared
    W2 = L.MoeWeights(fake, None, fake, fake, fake, None, None, None)
    assert L.LIB.moe_layer_forward(ctypes.byref(d), fake, ctypes.byref(W2), ctypes.c_void_p(0x200000),
                                   None, None, None, None, None, fake, 1 << 40, None) == -1
    d0 = full_desc(L, I_shared=0)
    assert L.LIB.moe_layer_forward(ctypes.byref(d0), fake, ctypes.byref(W), ctypes.c_void_p(0x200000),
                                   None, None, None, None, None, fake, 1 << 40, None) == -1


def test_zero_tokens_is_a_noop(L):
    d = ctypes.byref(full_desc(L, T=0))
    assert L.LIB.moe_route(d, None, None, None, None, None, None, None, 0, None) == 0
    assert L.LIB.moe_permute(d, None, None, None, None, None, None, None, 0, None) == 0
    assert L.LIB.moe_experts(d, None, None, None, None, None, None, None, None, 0, None) == 0
    assert L.LIB.moe_layer_forward(d, None, None, None, None, None, None, None, None, None, 0,
                                   None) == 0


def test_noalloc_host_errors(L):
    """moe_layer_forward_noalloc rejects, on the host and before any device
    call, a desc whose workspace exceeds its static buffer, the non-finite
    check flag (its status word is not readable), and invalid descs; T = 0
    is a no-op."""
    big = full_desc(L, T=4096)
    assert L.LIB.moe_workspace_size(ctypes.byref(big)) > L.MOE_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x100000)
    W = L.MoeWeights(fake, None, fake, fake, fake, fake, fake, fake)
    y = ctypes.c_void_p(0x200000)
    rc = L.LIB.moe_layer_forward_noalloc(ctypes.byref(big), fake, ctypes.byref(W), y, None, None,
                                         None, None, None, None)
    assert rc == L.MOE_ERR_SCRATCH == -6
    fits = full_desc(L, T=512)
    assert L.LIB.moe_workspace_size(ctypes.byref(fits)) <= L.MOE_NOALLOC_SCRATCH_BYTES
    fits.flags = L.MOE_F_CHECK_FINITE
    assert L.LIB.moe_layer_forward_noalloc(ctypes.byref(fits), fake, ctypes.byref(W), y, None,
                                           None, None, None, None, None) == -2
    bad = full_desc(L, E=255)
    assert L.LIB.moe_layer_forward_noalloc(ctypes.byref(bad), fake, ctypes.byref(W), y, None,
                                           None, None, None, None, None) == -1
    zero = full_desc(L, T=0)
    assert L.LIB.moe_layer_forward_noalloc(ctypes.byref(zero), None, None, None, None, None, None,
                                           None, None, None) == 0
    assert "MOE_NOALLOC_SCRATCH_BYTES" in L.strerror(-6)


def test_strerror(L):
    for c in [0, -1, -2, -3, -4, -5, -6, 99]:
        assert isinstance(L.strerror(c), str) and L.strerror(c)
    assert L.strerror(-3).startswith("workspace")


def test_binding_checks_shapes(L):
    import torch
    d = full_desc(L, T=4)
    x = torch.zeros(4, 2048, dtype=torch.bfloat16)  # on the CPU: rejected before any call
    with pytest.raises(ValueError):
        L.moe_route(d, x, torch.zeros(256, 2048), None, None, torch.zeros(4, 8, dtype=torch.int32),
                    torch.zeros(4, 8), torch.zeros(16, dtype=torch.uint8))


def test_balance_entry_points_reject_bad_arguments(L):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: errors come first
    odd = ctypes.c_void_p(0x100008)
    lib = L.LIB
    # statistics: shapes, nulls, alignment; L = 0 is a no-op
    assert lib.moe_expert_stats(-1, 256, 8, fake, fake, fake, None) == -1
    assert lib.moe_expert_stats(1, 255, 8, fake, fake, fake, None) == -1
    assert lib.moe_expert_stats(1, 2048, 8, fake, fake, fake, None) == -2
    assert lib.moe_expert_stats(1, 256, 128, fake, fake, fake, None) == -2
    assert lib.moe_expert_stats(1, 256, 8, None, fake, fake, None) == -1
    assert lib.moe_expert_stats(1, 256, 8, fake, odd, fake, None) == -4
    assert lib.moe_expert_stats(0, 256, 8, None, None, None, None) == 0
    # bias update
    assert lib.moe_bias_update(0, fake, None, fake, 0.1, None) == -1
    assert lib.moe_bias_update(256, None, None, fake, 0.1, None) == -1
    assert lib.moe_bias_update(256, fake, None, fake, float("inf"), None) == -1
    assert lib.moe_bias_update(4096, fake, None, fake, 0.1, None) == -2
    assert lib.moe_bias_update(256, fake, odd, fake, 0.1, None) == -4
    # aux loss: the mean over tokens needs one; workspace sized by T and E
    assert lib.moe_aux_loss_workspace_size(0, 256) == 0
    assert lib.moe_aux_loss_workspace_size(16, 2048) == 0
    n = lib.moe_aux_loss_workspace_size(16384, 256)
    assert n >= 256 * 8 and n % 256 == 0
    assert lib.moe_aux_loss(0, 256, fake, fake, fake, fake, fake, fake, n, None) == -1
    assert lib.moe_aux_loss(16384, 256, None, fake, fake, fake, fake, fake, n, None) == -1
    assert lib.moe_aux_loss(16384, 2048, fake, fake, fake, fake, fake, fake, n, None) == -2
    assert lib.moe_aux_loss(16384, 256, fake, fake, fake, fake, fake, fake, n - 1, None) == -3
    assert lib.moe_aux_loss(16384, 256, fake, fake, fake, fake, fake, None, n, None) == -3
    assert lib.moe_aux_loss(16384, 256, fake, fake, odd, fake, fake, fake, n, None) == -4


def test_backward_entry_points_reject_bad_arguments(L):
    """moe_backward_workspace_size / moe_layer_backward: the backward's
    envelope (bf16, shared expert as wide as the routed ones), T = 0 as a
    no-op, and argument errors found on the host before any launch."""
    lib = L.LIB
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: errors come first
    odd = ctypes.c_void_p(0x100008)
    d = full_desc(L)
    n = lib.moe_backward_workspace_size(ctypes.byref(d))
    assert n > 0 and n % 256 == 0
    # grows with the batch; unsupported descs give 0
    assert lib.moe_backward_workspace_size(ctypes.byref(full_desc(L, T=1024))) > n
    f32 = full_desc(L)
    f32.dtype = L.MOE_F32
    assert lib.moe_backward_workspace_size(ctypes.byref(f32)) == 0
    assert lib.moe_backward_workspace_size(ctypes.byref(full_desc(L, I_shared=128))) == 0
    assert lib.moe_backward_workspace_size(ctypes.byref(full_desc(L, I_shared=0))) > 0

    def call(desc, W, x=fake, idx=fake, lg=fake, dy=fake, dx=ctypes.c_void_p(0x200000),
             shared=True, ws=fake, nbytes=1 << 40):
        s = fake if shared else None
        return lib.moe_layer_backward(ctypes.byref(desc), x, ctypes.byref(W) if W else None, idx, lg,
                                      dy, dx, fake, fake, fake, fake, s, s, s, ws, nbytes, None)

    W = L.MoeWeights(fake, None, fake, fake, fake, fake, fake, fake)
    # T = 0: nothing to do, nothing checked past the descriptor
    d0 = full_desc(L, T=0)
    assert lib.moe_layer_backward(ctypes.byref(d0), None, None, None, None, None, None, None, None,
                                  None, None, None, None, None, None, 0, None) == 0
    assert call(f32, W) == -2                                # fp32 layer: unsupported
    assert call(full_desc(L, I_shared=128), W) == -2         # narrower shared expert
    assert call(d, None) == -1                               # no weights
    assert call(d, W, x=None) == -1
    assert call(d, W, lg=None) == -1
    assert call(d, W, dx=fake) == -1                         # dx aliasing x
    assert call(d, W, shared=False) == -1                    # shared gradients missing
    assert call(full_desc(L, I_shared=0), L.MoeWeights(fake, None, fake, fake, fake, None, None, None),
                shared=True) == -1                           # ... or given without a shared expert
    assert call(d, W, dy=odd) == -4
    assert call(d, W, nbytes=n - 1) == -3
    assert call(d, W, ws=None) == -3
    assert call(d, W, ws=odd) == -4


# --------------------------------------------------------------------------- measurement probes

PROBE_HEADER = os.path.join(ROOT, "include", "moe_probe.h")


def test_probe_library_exports_its_header():
    """libmoe_probe.so (the streaming-read and MFMA-loop kernels bench.py
    measures this GPU with) exports what include/moe_probe.h declares and
    rejects bad arguments on the host."""
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_probe_[a-z0-9_]+)\s*\(", src)))
    assert names == ["moe_probe_mfma_bf16", "moe_probe_stream_read"]
    lib = ctypes.CDLL(os.path.join(ROOT, "group_limited_top_amd", "libmoe_probe.so"))
    for n in names:
        assert hasattr(lib, n), n
    bad = 1  # hipErrorInvalidValue
    lib.moe_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    assert lib.moe_probe_stream_read(None, 4096, None, 16, None) == bad
    assert lib.moe_probe_stream_read(16, 4000, 16, 16, None) == bad      # not whole 4 KiB pieces
    assert lib.moe_probe_stream_read(8, 4096, 16, 16, None) == bad       # misaligned
    assert lib.moe_probe_stream_read(16, 4096, 16, 0, None) == bad       # no blocks
    lib.moe_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.moe_probe_mfma_bf16(None, 4, 4, None) == bad
    assert lib.moe_probe_mfma_bf16(16, 0, 4, None) == bad
