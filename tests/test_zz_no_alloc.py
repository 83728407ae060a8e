"""tp_mlp_shard_fwd_noalloc through the C ABI: the decode-path forward with the
library's per-device scratch array must return exactly what tp_mlp_shard_fwd
returns (same kernels, same order), call after call, including a second, smaller
call that reuses the array; and it must refuse what does not fit."""
import ctypes

import pytest
import torch

import oracle
import tensor_mlp_shard_amd as tpm
from tensor_mlp_shard_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
TOL_BF16 = 2e-2
OK, SHAPE = 0, 2


def say(*a):
    print(*a, flush=True)


def noalloc(handle, x, M, out):
    s = torch.cuda.current_stream().cuda_stream
    return tpm.capi().tp_mlp_shard_fwd_noalloc(ctypes.c_void_p(handle), ctypes.c_void_p(x.data_ptr()),
                                               int(M), ctypes.c_void_p(out.data_ptr()),
                                               ctypes.c_void_p(s))


def compare_calls(a, b, Ms, ref_handle_tokens=64):
    """Run each M in turn through both entry points on one handle; every noalloc
    result must equal the fwd result bit for bit and match the oracle."""
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=ref_handle_tokens)
    try:
        for M in Ms:
            x = synth.tokens(M)
            xd = x.to(DEV)
            say("noalloc vs fwd: d", a.shape[0], "F", b.shape[0], "M", M)
            want = sh.forward(xd)
            got = torch.full((M, a.shape[0]), float("nan"), device=DEV)
            assert noalloc(sh.handle, xd, M, got) == OK
            torch.cuda.synchronize()
            assert torch.equal(got.cpu(), want.cpu())
            err = oracle.rel_err(got.cpu(), oracle.shard_forward(x, a, b, "silu_gate"))
            say("err vs oracle", err)
            assert err <= TOL_BF16
    finally:
        sh.close()


def test_decode_shard_two_calls_smaller_second():
    a, b = synth.ModelSpec().shard(0, 8)  # 70B-class TP=8 rank: d 8192, F 3584
    compare_calls(a, b, (32, 5))


def test_narrow_shard_with_contraction_slices():
    # 1024 first-weight columns = 32 blocks: the first product slices the
    # contraction, so the arrival counters in the array are used and cleared
    a, b = synth.ModelSpec(ffn=512 * 8).shard(0, 8)
    compare_calls(a, b, (64, 8, 40))


def test_handle_without_workspace():
    a, b = synth.ModelSpec(d_model=1024, ffn=4096).shard(1, 8)
    x = synth.tokens(17, d=1024)
    bare = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=0)
    ref = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=17)
    try:
        assert bare.plan["workspace_bytes"] == 0
        out = torch.empty(17, 1024, device=DEV)
        assert noalloc(bare.handle, x.to(DEV), 17, out) == OK
        want = ref.forward(x.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), want.cpu())
    finally:
        bare.close()
        ref.close()


def test_refusals():
    a, b = synth.ModelSpec(d_model=1024, ffn=4096).shard(0, 8)
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=128)
    x = synth.tokens(65, d=1024).to(DEV)
    out = torch.empty(65, 1024, device=DEV)
    try:
        assert noalloc(sh.handle, x, 65, out) == SHAPE   # past the decode path
        assert noalloc(sh.handle, x, 0, out) == OK       # no-op
    finally:
        sh.close()
    # a shard whose hidden rows alone exceed the array: 64 MiB at M = 1
    d, F = 64, 1 << 20
    big_a = torch.zeros(d, F, dtype=torch.bfloat16, device=DEV)
    big_b = torch.zeros(F, d, dtype=torch.bfloat16, device=DEV)
    big = tpm.Shard(big_a, big_b, "tanh", max_tokens=0)
    try:
        x = torch.zeros(1, d, dtype=torch.bfloat16, device=DEV)
        o = torch.empty(1, d, device=DEV)
        assert noalloc(big.handle, x, 1, o) == SHAPE
    finally:
        big.close()
    torch.cuda.synchronize()
