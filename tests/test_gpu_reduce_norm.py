"""GPU parity of tp_partials_reduce_add_rmsnorm (partials sum + residual add +
RMSNorm, one kernel) against the fp64 oracle, through the C ABI.

Same error measure and bounds as the MLP parity tests: max|gpu - oracle| /
sqrt(mean(oracle^2)) <= 1e-5 when every tensor is fp32, <= 2e-2 when a bf16
tensor is involved (inputs rounded, or outputs rounded to bf16)."""
import ctypes

import pytest
import torch

import oracle
import tensor_mlp_shard_amd as tpm

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def case(k, rows, cols, seed, pdt=torch.float32, rdt=torch.float32):
    g = torch.Generator().manual_seed(seed)
    parts = [torch.randn(rows, cols, generator=g).to(pdt) for _ in range(k)]
    res = torch.randn(rows, cols, generator=g).to(rdt)
    gamma = (torch.rand(cols, generator=g) + 0.5).to(rdt)
    return parts, res, gamma


def run_gpu(parts, res, gamma, eps, ydt, inplace=False):
    pd = [p.to(DEV) for p in parts]
    rd = res.to(DEV)
    ro = rd if inplace else torch.empty_like(rd)
    y = torch.empty(res.shape, dtype=ydt, device=DEV)
    tpm.tp_partials_reduce_add_rmsnorm(pd, rd, gamma.to(DEV), eps, y, residual_out=ro)
    torch.cuda.synchronize()
    return ro.cpu(), y.cpu()


@pytest.mark.parametrize("k", [1, 3, 8])
@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 1000), (32, 8192), (2, 32768), (5, 520)])
def test_fp32_parity(k, rows, cols):
    parts, res, gamma = case(k, rows, cols, 100 * k + rows)
    eps = 1e-6
    say("reduce+norm fp32 k", k, "rows", rows, "cols", cols)
    h, y = run_gpu(parts, res, gamma, eps, torch.float32)
    rh, ry = oracle.reduce_add_rmsnorm(parts, res, gamma, eps)
    assert oracle.rel_err(h, rh) <= TOL_F32
    assert oracle.rel_err(y, ry) <= TOL_F32


@pytest.mark.parametrize("pdt,rdt,ydt", [
    (torch.float32, torch.bfloat16, torch.bfloat16),
    (torch.bfloat16, torch.bfloat16, torch.bfloat16),
    (torch.bfloat16, torch.float32, torch.float32),
    (torch.float32, torch.float32, torch.bfloat16),
])
def test_mixed_dtypes(pdt, rdt, ydt):
    parts, res, gamma = case(8, 32, 8192, 7, pdt, rdt)
    eps = 1e-5
    say("reduce+norm dtypes", pdt, rdt, ydt)
    h, y = run_gpu(parts, res, gamma, eps, ydt)
    rh, ry = oracle.reduce_add_rmsnorm(parts, res, gamma, eps)
    assert oracle.rel_err(h, rh) <= TOL_BF16
    assert oracle.rel_err(y, ry) <= TOL_BF16


def test_inplace_and_deterministic():
    parts, res, gamma = case(8, 32, 8192, 3)
    h1, y1 = run_gpu(parts, res, gamma, 1e-6, torch.float32)
    h2, y2 = run_gpu(parts, res, gamma, 1e-6, torch.float32, inplace=True)
    assert torch.equal(h1, h2) and torch.equal(y1, y2)


def test_large_rows_sampled_and_zero_rows():
    parts, res, gamma = case(8, 2048, 8192, 11)
    say("reduce+norm 2048 x 8192, k 8")
    h, y = run_gpu(parts, res, gamma, 1e-6, torch.float32)
    rows = [0, 1, 777, 1500, 2047]
    rh, ry = oracle.reduce_add_rmsnorm([p[rows] for p in parts], res[rows], gamma, 1e-6)
    assert oracle.rel_err(h[rows], rh) <= TOL_F32
    assert oracle.rel_err(y[rows], ry) <= TOL_F32
    # rows = 0 (pointers still valid, as the ABI requires): nothing is written
    base = torch.full((1, 64), 7.0, device=DEV)
    ybase = torch.full((1, 64), 9.0, device=DEV)
    gam = torch.ones(64, device=DEV)
    vp = ctypes.c_void_p
    arr = (vp * 1)(base.data_ptr())
    rc = tpm.capi().tp_partials_reduce_add_rmsnorm(arr, 1, 0, 64, 0, vp(base.data_ptr()),
                                                   vp(base.data_ptr()), 0, vp(gam.data_ptr()),
                                                   ctypes.c_float(1e-6), vp(ybase.data_ptr()), 0,
                                                   None)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.all(base == 7.0) and torch.all(ybase == 9.0)


def test_constant_rows_closed_form():
    # every row constant: y = c / sqrt(c^2 + eps) * gamma exactly up to fp32 rounding
    rows, cols, eps = 4, 4096, 0.25
    c = torch.tensor([0.5, -1.5, 3.0, 2.0 ** -10]).view(rows, 1).expand(rows, cols).contiguous()
    parts = [c / 2, c / 4]
    res = c / 4
    gamma = torch.linspace(0.5, 2.0, cols)
    h, y = run_gpu(parts, res, gamma, eps, torch.float32)
    want = c / torch.sqrt(c * c + eps) * gamma
    assert torch.allclose(h, c, rtol=0, atol=0)
    assert oracle.rel_err(y, want.double().numpy()) <= TOL_F32
