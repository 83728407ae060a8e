"""GPU parity of tp_attn_partials_merge (page "LLM 推理并行化：先找瓶颈，再决定怎么切",
section 三.4, decode context parallelism) against the fp64 oracle, through the C
ABI: random partials at the decode shape (32 tokens x 64 heads, head width 128,
k = 8 ranks) and ragged shapes, partials computed from real attention against the
unsplit attention, empty ranks and rows, large maxima, merged statistics, a
second-level merge, in-place output, determinism and refused calls.
Bounds: 1e-5 (max-abs over RMS) for fp32 output; for bfloat16 output, element by
element, the format's rounding (2^-8 of the value) plus 1e-5 of the RMS."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import tensor_mlp_shard_amd as tpm
from tensor_mlp_shard_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_F32 = 1e-5
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def gpu_merge(vals, maxs, sums, out_dtype=torch.float32):
    out, m, s = tpm.attn_partials_merge([v.to(DEV) for v in vals], [x.to(DEV) for x in maxs],
                                        [x.to(DEV) for x in sums], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.cpu(), m.cpu(), s.cpu()


@pytest.mark.parametrize("rows,dim,k", [(2048, 128, 8), (1, 8, 1), (3, 136, 2), (257, 64, 16),
                                        (100, 512, 5),
                                        (4100, 1024, 3),    # more 8-value groups than the grid's cap: stride loop
                                        (2, 1 << 20, 2)])   # the largest dim the call accepts
def test_parity_fp32(rows, dim, k):
    vals, maxs, sums = synth.attn_partials(rows, dim, k, seed=rows + k)
    say("merge fp32 rows", rows, "dim", dim, "k", k)
    out, m, s = gpu_merge(vals, maxs, sums)
    ref, rm, rs = oracle.attn_partials_merge(vals, maxs, sums)
    err = oracle.rel_err(out, ref)
    say("err", err)
    assert err <= TOL_F32
    assert np.array_equal(m.numpy().astype(np.float64), rm)
    assert np.max(np.abs(s.numpy() - rs) / rs) <= 1e-5


@pytest.mark.parametrize("in_dtype,out_dtype", [(torch.bfloat16, torch.float32),
                                                (torch.float32, torch.bfloat16),
                                                (torch.bfloat16, torch.bfloat16)])
def test_bf16_values_and_output(in_dtype, out_dtype):
    vals, maxs, sums = synth.attn_partials(2048, 128, 8, dtype=in_dtype)
    out, _, _ = gpu_merge(vals, maxs, sums, out_dtype)
    assert out.dtype == out_dtype
    ref, _, _ = oracle.attn_partials_merge(vals, maxs, sums)  # the same bf16 values, widened
    if out_dtype == torch.float32:
        assert oracle.rel_err(out, ref) <= TOL_F32
    else:
        # Rounding the fp32 result to bfloat16 (8 significant bits, nearest) moves each
        # element by at most 2^-8 of its magnitude; the fp32 merge itself adds far less.
        # Rows with few effective keys have outputs well above the RMS, so a bound
        # normalised by the RMS would charge the format's rounding to the merge.
        got = out.double().numpy()
        bound = 2.0 ** -8 * np.abs(ref) + TOL_F32 * np.sqrt(np.mean(ref ** 2))
        assert np.all(np.abs(got - ref) <= bound)


def test_partials_of_real_attention_equal_the_unsplit_attention():
    """Scores and values of 64 query rows over 4096 keys, the keys split into 8 uneven
    contiguous shards (one empty); each rank's partial is computed in fp64 on the
    host, rounded to fp32 and merged on the GPU."""
    rng = np.random.default_rng(11)
    rows, L, dim = 64, 4096, 128
    scores = rng.normal(0.0, 2.0, size=(rows, L))
    values = rng.normal(0.0, 1.0, size=(L, dim))
    cuts = [0, 300, 300, 1000, 1800, 2600, 3500, 4000, L]
    vals, maxs, sums = [], [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        if hi == lo:
            maxs.append(torch.full((rows,), -math.inf))
            sums.append(torch.zeros(rows))
            vals.append(torch.zeros(rows, dim))
            continue
        z = scores[:, lo:hi]
        mx = z.max(axis=1)
        w = np.exp(z - mx[:, None])
        maxs.append(torch.tensor(mx, dtype=torch.float32))
        sums.append(torch.tensor(w.sum(axis=1), dtype=torch.float32))
        vals.append(torch.tensor(w @ values[lo:hi], dtype=torch.float32))
    w = np.exp(scores - scores.max(axis=1, keepdims=True))
    full = (w @ values) / w.sum(axis=1, keepdims=True)
    out, _, _ = gpu_merge(vals, maxs, sums)
    err = oracle.rel_err(out, full)
    say("merge vs unsplit attention", err)
    assert err <= TOL_F32


def test_empty_ranks_rows_and_large_maxima():
    vals, maxs, sums = synth.attn_partials(40, 16, 4, seed=3)
    maxs[1] = torch.full((40,), -math.inf)   # rank 1 holds no keys
    sums[1] = torch.zeros(40)
    vals[1] = torch.zeros(40, 16)
    for i in range(4):                      # rows 5..9: no keys anywhere
        maxs[i][5:10] = -math.inf
        sums[i][5:10] = 0.0
        vals[i][5:10] = 0.0
    maxs[2][20:] += 1000.0                  # scores far past exp's fp32 range
    out, m, s = gpu_merge(vals, maxs, sums)
    ref, rm, rs = oracle.attn_partials_merge(vals, maxs, sums)
    assert torch.all(torch.isfinite(out))
    assert torch.all(out[5:10] == 0) and torch.all(torch.isneginf(m[5:10])) and torch.all(s[5:10] == 0)
    assert oracle.rel_err(out, ref) <= TOL_F32


def test_second_level_merge_and_in_place_and_determinism():
    vals, maxs, sums = synth.attn_partials(512, 128, 8, seed=21)
    flat, _, _ = gpu_merge(vals, maxs, sums)
    a, am, asum = gpu_merge(vals[:4], maxs[:4], sums[:4])
    b, bm, bsum = gpu_merge(vals[4:], maxs[4:], sums[4:])
    two, _, _ = gpu_merge([a * asum[:, None], b * bsum[:, None]], [am, bm], [asum, bsum])
    assert oracle.rel_err(two, flat.double().numpy()) <= TOL_F32
    dv = [v.to(DEV) for v in vals]
    dm = [x.to(DEV) for x in maxs]
    ds = [x.to(DEV) for x in sums]
    o1 = torch.empty_like(dv[0])
    tpm.tp_attn_partials_merge(dv, dm, ds, o1)
    o2 = torch.empty_like(dv[0])
    tpm.tp_attn_partials_merge(dv, dm, ds, o2)
    tpm.tp_attn_partials_merge(dv, dm, ds, dv[0])  # in place over rank 0's values
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, dv[0])
    assert torch.equal(o1.cpu(), flat)


def test_refused_calls_and_zero_rows():
    lib = tpm.capi()
    vals, maxs, sums = synth.attn_partials(4, 16, 2)
    dv = [v.to(DEV) for v in vals]
    dm = [x.to(DEV) for x in maxs]
    ds = [x.to(DEV) for x in sums]
    out = torch.empty_like(dv[0])
    arr = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    def call(k=2, rows=4, dim=16, v=None, o=None, mo=None, eo=None, in_dt=0, out_dt=0):
        return lib.tp_attn_partials_merge(v or arr(dv), arr(dm), arr(ds), k, rows, dim, in_dt,
                                          o or out.data_ptr(), out_dt, mo, eo, None)
    assert call() == 0
    assert call(k=0) == 2 and call(k=17) == 2            # TPM_ERR_SHAPE
    assert call(dim=12) == 2 and call(dim=0) == 2
    assert call(o=out.data_ptr() + 4) == 3                 # TPM_ERR_ALIGN
    assert call(v=arr([dv[0][:, 2:], dv[1]])) == 3
    assert call(mo=dm[0].data_ptr(), eo=None) == 1        # one statistic without the other
    assert call(mo=dm[0].data_ptr(), eo=ds[1].data_ptr()) == 1  # output over an input
    assert call(o=dv[0].data_ptr(), out_dt=1) == 1        # in place with a dtype change
    assert call(in_dt=7) == 1
    before = out.clone()
    assert call(rows=0) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, before)
    with pytest.raises(ValueError):
        tpm.tp_attn_partials_merge(dv, dm[:1], ds, out)
