"""Error returns that need a device: handles whose buffers exceed device memory.

tp_mlp_shard_create must report TPM_ERR_OOM, clear *out and leave nothing allocated
(the header's contract for a failing create); the failure comes from the single
device allocation, before any kernel is launched."""
import ctypes

import pytest
import torch

import tensor_mlp_shard_amd as tpm

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

OOM = 5  # TPM_ERR_OOM


def say(*a):
    print(*a, flush=True)


def test_create_out_of_memory_leaves_nothing_allocated():
    lib = tpm.capi()
    torch.cuda.synchronize()
    free0, total = torch.cuda.mem_get_info()
    # hidden buffer alone: 2^24 padded rows x 16384 features x 2 bytes = 512 GiB
    d = tpm.make_desc(d_model=64, ffn_shard=16384, max_tokens=1 << 24, activation="silu_gate",
                      in_dtype=tpm.BF16, out_dtype=tpm.F32, path="auto")
    plan = tpm.tp_mlp_shard_plan(d)
    assert plan["workspace_bytes"] + plan["packed_weight_bytes"] > total
    a = torch.zeros(64, 2 * 16384, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(16384, 64, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    h = ctypes.c_void_p(1234)
    say("create with", plan["workspace_bytes"] + plan["packed_weight_bytes"], "bytes of", total)
    rc = lib.tp_mlp_shard_create(ctypes.byref(d), ctypes.c_void_p(a.data_ptr()),
                                 ctypes.c_void_p(b.data_ptr()), None, ctypes.byref(h))
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    assert rc == OOM
    assert h.value is None
    assert free2 == free1, (free1, free2)
    # the device is still usable afterwards
    c = (a.float().sum() + b.float().sum()).item()
    assert c == 0.0
    del a, b
    assert free0 >= free2


def test_projection_and_experts_create_out_of_memory():
    """The projection and grouped-expert handles keep the same contract: a create whose
    packed weights exceed device memory reports TPM_ERR_OOM, clears *out and leaves
    nothing allocated.  Their single allocation comes before the packing kernels, so the
    weight pointers (a small real tensor here) are never read."""
    lib = tpm.capi()
    torch.cuda.synchronize()
    _, total = torch.cuda.mem_get_info()
    need_proj = (1 << 20) * (1 << 19) * 2                       # packed [2^20 x 2^19] bf16
    need_moe = 2 * ((1 << 20) * (2 << 16) + (1 << 16) * (1 << 20)) * 2  # 2 experts' W1, W2
    if min(need_proj, need_moe) <= total:
        pytest.skip("the device holds the requested weights")
    w = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    pd = tpm.TpmProjDesc(1 << 20, 1 << 19, 8, tpm.BF16, tpm.F32, 0, 0)
    h = ctypes.c_void_p(1234)
    say("projection create with", need_proj, "bytes of weights on a device of", total)
    rc = lib.tp_proj_create(ctypes.byref(pd), ctypes.c_void_p(w.data_ptr()), None,
                            ctypes.byref(h))
    assert rc == OOM and h.value is None
    md = tpm.TpmMoeDesc(1 << 20, 1 << 16, 2, 64, 1, tpm.BF16, tpm.F32, 0)
    h = ctypes.c_void_p(1234)
    say("grouped-expert create with", need_moe, "bytes of weights")
    rc = lib.tp_moe_create(ctypes.byref(md), ctypes.c_void_p(w.data_ptr()),
                           ctypes.c_void_p(w.data_ptr()), None, ctypes.byref(h))
    assert rc == OOM and h.value is None
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    assert free2 == free1, (free1, free2)
    assert w.float().sum().item() == 0.0  # the device is still usable
