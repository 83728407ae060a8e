"""GPU parity of single tensor-parallel projections (tp_proj_*) against the fp64
oracle, through the C ABI: the attention block's column-parallel QKV shard and
row-parallel output shard at the 70B-class TP=8 shapes, both kernel paths, ragged
and edge sizes, and the rank partials of the output projection summing to the
unsplit block.  Bounds as for the MLP (tests/tolerances.py)."""
import ctypes

import pytest
import torch

import oracle
import tensor_mlp_shard_amd as tpm
from tensor_mlp_shard_amd import synth
from tolerances import TOL_BF16, TOL_F32, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def run_proj(w, x, out_dtype=torch.float32, path="auto", max_tokens=None):
    p = tpm.Projection(w.to(DEV), max_tokens=max_tokens or max(x.shape[0], 1),
                       out_dtype=out_dtype, path=path)
    try:
        y = p.forward(x.to(DEV))
        torch.cuda.synchronize()
        return y.cpu()
    finally:
        p.close()


@pytest.mark.parametrize("path", ["stream", "tiled"])
@pytest.mark.parametrize("M", [1, 32, 64, 300])
def test_qkv_shard_tp8(path, M):
    wqkv, _ = synth.AttentionSpec().shard(0, 8)  # [8192 x 1280]
    x = synth.tokens(M)
    say("qkv shard", path, "M", M)
    y = run_proj(wqkv, x, torch.bfloat16, path)
    ref = oracle.projection(x, wqkv)
    assert oracle.rel_err(y, ref) <= tol_for(torch.bfloat16, ref)


@pytest.mark.parametrize("M", [1, 32, 2048])
def test_o_shard_tp8(M):
    _, wo = synth.AttentionSpec().shard(3, 8)  # [1024 x 8192]
    g = torch.Generator().manual_seed(M)
    a = torch.randn(M, 1024, generator=g).to(torch.bfloat16)
    say("o shard M", M)
    y = run_proj(wo, a, torch.float32)
    rows = synth.sample_rows(M, 64)
    assert oracle.rel_err(y[rows], oracle.projection(a[rows], wo)) <= TOL_BF16


def test_stream_forced_many_token_groups_narrow_projection():
    """A narrow projection (8 column blocks) with a long contraction on the forced
    streaming path: one token group slices the contraction, several do not."""
    g = torch.Generator().manual_seed(77)
    w = (torch.randn(8192, 256, generator=g) * 0.02).to(torch.bfloat16)
    p = tpm.Projection(w.to(DEV), max_tokens=200, out_dtype=torch.float32, path="stream")
    try:
        for M in (32, 8, 200, 1, 96, 32):
            x = synth.tokens(M)
            say("forced stream, narrow projection M", M)
            y = p.forward(x.to(DEV)).cpu()
            assert oracle.rel_err(y, oracle.projection(x, w)) <= TOL_BF16
    finally:
        p.close()


@pytest.mark.parametrize("K,N,M", [(64, 1, 3), (128, 100, 70), (192, 257, 1), (512, 700, 513)])
def test_ragged_shapes_both_paths(K, N, M):
    g = torch.Generator().manual_seed(K + N + M)
    w = (torch.randn(K, N, generator=g) * 0.1).to(torch.bfloat16)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    ref = oracle.projection(x, w)
    for path in ("stream", "tiled"):
        y = run_proj(w, x, torch.float32, path)
        assert oracle.rel_err(y, ref) <= TOL_BF16, path


def test_fp32_projection():
    g = torch.Generator().manual_seed(9)
    w = torch.randn(96, 40, generator=g) * 0.1
    x = torch.randn(7, 96, generator=g)
    y = run_proj(w, x, torch.float32)
    assert oracle.rel_err(y, oracle.projection(x, w)) <= TOL_F32


def test_attention_block_partials_sum_to_unsplit():
    """Eight ranks: QKV column shards (bf16 out), a stand-in per-head core (the
    query part passed through), output row shards to fp32 partials, summed on the
    GPU; against the unsplit product in fp64."""
    spec = synth.AttentionSpec(d_model=1024, q_heads=16, kv_heads=8, head_dim=64)
    x = synth.tokens(32, d=1024)
    qw = spec.q_width(8)
    parts, wq_all, wo_all = [], [], []
    for r in range(8):
        wqkv, wo = spec.shard(r, 8)
        y = run_proj(wqkv, x, torch.bfloat16)
        parts.append(run_proj(wo, y[:, :qw].contiguous(), torch.float32).to(DEV))
        wq_all.append(wqkv[:, :qw])
        wo_all.append(wo)
    z = tpm.partials_reduce(parts).cpu()
    Wq = torch.cat(wq_all, dim=1)
    Wo = torch.cat(wo_all, dim=0)
    want = oracle.projection(oracle.projection(x, Wq), Wo)
    err = oracle.rel_err(z, want)
    say("attention block, 8 ranks: err", err)
    assert err <= TOL_BF16


def test_tiled_weight_past_32bit_offsets():
    """A packed weight of 4 GiB (8192 x 262144 bf16) lies past the 32-bit buffer offsets
    of the prefill GEMM, which hands such products to the tiled kernel with 64-bit
    addresses.  The weight is drawn on the device (2^31 values) and is not periodic in
    any index, so an offset that wrapped would read a wrong value.  Sampled rows and
    columns against the oracle; the packed buffer is k-step-major, so every column's
    products read across the whole 4 GiB."""
    K, N, M = 8192, 262144, 300
    w = synth.randn_device((K, N), seed=4242, device=DEV, std=synth.WEIGHT_STD,
                           dtype=torch.bfloat16)
    x = synth.tokens(M, K)
    rows = synth.sample_rows(M, 16)
    cols = synth.sample_rows(N, 256, seed=11)
    w_cols = w[:, cols].cpu()
    say("tiled projection, packed weight 4 GiB:", K, "x", N, "M", M)
    p = tpm.Projection(w, max_tokens=M, out_dtype=torch.float32, path="tiled")
    del w
    try:
        y = p.forward(x.to(DEV))
        torch.cuda.synchronize()
        yc = y[rows][:, cols].cpu()
        del y
    finally:
        p.close()
        torch.cuda.empty_cache()
    err = oracle.rel_err(yc, oracle.projection(x[rows], w_cols))
    say("err", err)
    assert err <= TOL_BF16


def test_zero_tokens_and_bad_calls():
    w = torch.randn(64, 32).to(torch.bfloat16).to(DEV)
    p = tpm.Projection(w, max_tokens=8)
    try:
        buf = torch.full((1, 32), 5.0, device=DEV)
        rc = tpm.capi().tp_proj_fwd(ctypes.c_void_p(p.handle), ctypes.c_void_p(w.data_ptr()), 0,
                                    ctypes.c_void_p(buf.data_ptr()), None)
        assert rc == 0
        torch.cuda.synchronize()
        assert torch.all(buf == 5.0)
        x = torch.randn(9, 64).to(torch.bfloat16).to(DEV)
        with pytest.raises(tpm.TpmError):
            p.forward(x)  # M > max_tokens
    finally:
        p.close()
