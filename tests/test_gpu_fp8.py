"""GPU parity of the FP8 partials (tp_partials_quantize_fp8, tp_partials_reduce_fp8)
against the oracle, through the C ABI.

The E4M3 codes and the row scales are integer / exactly specified work: they must
match the oracle bit for bit (both sides decide the codes in fp32, as the header
specifies).  The fp32 sum of dequantized partials is compared with the oracle's
fp64 sum of the same dequantized values within 1e-5 (max-abs / RMS)."""
import pytest
import torch

import oracle
import tensor_mlp_shard_amd as tpm

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_F32 = 1e-5
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def quant_gpu(x):
    rows, cols = x.shape
    q = torch.empty(rows, cols, dtype=torch.uint8, device=DEV)
    s = torch.empty(rows, dtype=torch.float32, device=DEV)
    tpm.tp_partials_quantize_fp8(x.to(DEV), q, s)
    torch.cuda.synchronize()
    return q.cpu(), s.cpu()


@pytest.mark.parametrize("rows,cols,dt", [(1, 16, torch.float32), (5, 48, torch.float32),
                                          (32, 8192, torch.float32), (7, 32768, torch.float32),
                                          (32, 8192, torch.bfloat16), (3, 17408, torch.bfloat16)])
def test_quantize_bit_exact(rows, cols, dt):
    g = torch.Generator().manual_seed(rows * 131 + cols)
    x = (torch.randn(rows, cols, generator=g) * torch.logspace(-6, 3, rows).view(rows, 1)).to(dt)
    if rows > 2:
        x[1] = 0.0           # zero row: scale 1, codes 0
        x[2, 3] = 1e-30      # a subnormal-range entry
    say("fp8 quantize", rows, cols, dt)
    q, s = quant_gpu(x)
    rq, rs = oracle.quantize_fp8(x)
    assert torch.equal(s, torch.from_numpy(rs))
    assert torch.equal(q, torch.from_numpy(rq))


def test_quantize_every_rounding_case():
    """Each E4M3 decision the quantizer can face, through the library: rows that start
    with 448 have amax 448, so the scale is 1 and every other entry is encoded as given.
    The entries are every E4M3 grid value, every midpoint between neighbours (the ties,
    subnormal ones included) and the fp32 values just below and above each midpoint,
    for both signs; codes must equal the oracle's table search bit for bit."""
    import numpy as np
    grid = np.array(sorted({abs(float(oracle.e4m3_value(c))) for c in range(256)
                            if np.isfinite(oracle.e4m3_value(c))}), dtype=np.float32)
    mids = ((grid[:-1].astype(np.float64) + grid[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (grid[:-1].astype(np.float64) + grid[1:]) / 2)
    vals = np.concatenate([grid, mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(np.inf))]).astype(np.float32)
    cols = 16 * ((len(vals) + 1 + 15) // 16)
    x = np.zeros((2, cols), dtype=np.float32)
    x[:, 0] = 448.0
    x[0, 1:1 + len(vals)] = vals
    x[1, 1:1 + len(vals)] = -vals
    say("fp8 rounding cases:", len(vals), "magnitudes, both signs")
    q, s = quant_gpu(torch.from_numpy(x))
    rq, rs = oracle.quantize_fp8(x)
    assert np.all(rs == 1.0) and torch.equal(s, torch.from_numpy(rs))
    bad = np.nonzero(q.numpy() != rq)
    assert bad[0].size == 0, [(float(x[r, c]), int(q[r, c]), int(rq[r, c])) for r, c in zip(*bad)][:10]


@pytest.mark.parametrize("k", [1, 2, 8, 16])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_reduce_fp8(k, out_dtype):
    g = torch.Generator().manual_seed(k)
    rows, cols = 32, 8192
    parts = [torch.randn(rows, cols, generator=g) for _ in range(k)]
    qs, ss = [], []
    for p in parts:
        q, s = quant_gpu(p)
        qs.append(q)
        ss.append(s)
    out = torch.empty(rows, cols, dtype=out_dtype, device=DEV)
    tpm.tp_partials_reduce_fp8([q.to(DEV) for q in qs], [s.to(DEV) for s in ss], out)
    torch.cuda.synchronize()
    ref = oracle.reduce_fp8([q.numpy() for q in qs], [s.numpy() for s in ss])
    tol = TOL_F32 if out_dtype == torch.float32 else 2e-2
    assert oracle.rel_err(out.cpu(), ref) <= tol
    # the FP8 path against the exact partials: within the E4M3 rounding bound (half
    # a grid spacing per element: 2^-4 of the magnitude, 2^-10 scale units near 0)
    exact = oracle.partials_sum(parts)
    bound = sum(p.double().abs().numpy() * 2.0 ** -4 + 2.0 ** -10 * s.double().numpy()[:, None]
                for p, s in zip(parts, ss))
    got = out.cpu().double().numpy()
    slack = 1e-5 * float((exact ** 2).mean() ** 0.5) if out_dtype == torch.float32 else \
        2.0 ** -8 * abs(exact).max()
    assert (abs(got - exact) <= bound + slack).all()
    say("k", k, "fp8 transport error (max-abs / RMS) vs exact sum", oracle.rel_err(got, exact))


def test_fp8_pipeline_after_mlp_shards_and_determinism():
    """Eight TP shards of a small SwiGLU MLP, partials through FP8, summed: bitwise
    repeatable, and element by element within the E4M3 rounding bound of the partials
    plus the bf16 path's own bound against the unsplit MLP."""
    from tensor_mlp_shard_amd import synth
    a_sh, b_sh = synth.ModelSpec(d_model=1024, ffn=4096).shards(8)
    x = synth.tokens(32, d=1024)
    Z = []
    for rep in range(2):
        qs, ss, ps = [], [], []
        for a, b in zip(a_sh, b_sh):
            sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=32)
            p = sh.forward(x.to(DEV))
            q = torch.empty(32, 1024, dtype=torch.uint8, device=DEV)
            s = torch.empty(32, dtype=torch.float32, device=DEV)
            tpm.tp_partials_quantize_fp8(p, q, s)
            torch.cuda.synchronize()
            sh.close()
            qs.append(q)
            ss.append(s)
            ps.append(p.cpu())
        z = torch.empty(32, 1024, device=DEV)
        tpm.tp_partials_reduce_fp8(qs, ss, z)
        torch.cuda.synchronize()
        Z.append(z.cpu())
    assert torch.equal(Z[0], Z[1])
    ref = oracle.unsplit_output(x, a_sh, b_sh, "silu_gate")
    rms = float((ref ** 2).mean() ** 0.5)
    # the exact (fp32-partial) path is within the bf16 bound of the unsplit MLP ...
    exact_gpu = oracle.partials_sum(ps)
    assert oracle.rel_err(exact_gpu, ref) <= 2e-2
    # ... and FP8 transport adds at most half a grid spacing per partial element (2^-4
    # of the magnitude, 2^-10 scale units near 0), so element by element
    bound = sum(p.double().numpy().__abs__() * 2.0 ** -4 + 2.0 ** -10 * s.cpu().double().numpy()[:, None]
                for p, s in zip(ps, ss))
    got = Z[0].double().numpy()
    assert (abs(got - ref) <= bound + 2e-2 * rms).all()
    say("fp8 partials, 8 shards: err vs unsplit", oracle.rel_err(Z[0], ref))
