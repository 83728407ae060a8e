"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Error measure: max|gpu - oracle| / sqrt(mean(oracle^2)) over the compared outputs.
Bounds (tests/tolerances.py): 1e-5 for fp32 inputs, 2e-2 for bf16 inputs with fp32
accumulation, plus half an ulp of a bf16 output.
Large token counts compare a seeded subset of rows (rows are independent), always
including the first and the last row.
"""
import functools

import pytest
import torch

import oracle
import tensor_mlp_shard_amd as tpm
from tensor_mlp_shard_amd import synth
from tolerances import TOL_BF16, TOL_F32, tol_for, tol_hidden_rounding

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def gpu_shard(a, b, x, act, path="auto", out_dtype=torch.float32, max_tokens=None):
    sh = tpm.Shard(a.to(DEV), b.to(DEV), act, max_tokens=max_tokens or max(x.shape[0], 1),
                   out_dtype=out_dtype, path=path)
    try:
        p = sh.forward(x.to(DEV))
        torch.cuda.synchronize()
        return p.cpu()
    finally:
        sh.close()


@functools.lru_cache(maxsize=None)
def model_shards(tp, d=synth.D_MODEL, ffn=synth.FFN):
    spec = synth.ModelSpec(d_model=d, ffn=ffn)
    return spec.shards(tp)


# ------------------------------------------------------------------ toy, fp32
def test_toy_fp32_tp2_partials_and_sum():
    X, a_sh, b_sh = synth.toy_shards(2)
    say("toy fp32 tanh TP=2, X", tuple(X.shape))
    parts = []
    for a, b in zip(a_sh, b_sh):
        p = gpu_shard(a, b, X, "tanh")
        assert oracle.rel_err(p, oracle.shard_forward(X, a, b, "tanh")) <= TOL_F32
        parts.append(p.to(DEV))
    Z = tpm.partials_reduce(parts).cpu()
    ref = oracle.unsplit_output(X, a_sh, b_sh, "tanh")
    err = oracle.rel_err(Z, ref)
    say("toy err", err)
    assert err <= TOL_F32
    Z2 = tpm.tensor_parallel_output(X.to(DEV), [a.to(DEV) for a in a_sh],
                                    [b.to(DEV) for b in b_sh], "tanh").cpu()
    assert torch.equal(Z, Z2)


@pytest.mark.parametrize("act", ["tanh", "silu_gate", "identity"])
@pytest.mark.parametrize("M,d,F", [(1, 1, 1), (5, 37, 23), (70, 130, 90)])
def test_fp32_ragged_shapes(act, M, d, F):
    g = torch.Generator().manual_seed(M * 1000 + d + F)
    X = torch.randn(M, d, generator=g) * 0.5
    A = torch.randn(d, 2 * F if act == "silu_gate" else F, generator=g) * 0.2
    B = torch.randn(F, d, generator=g) * 0.2
    say("fp32", act, M, d, F)
    p = gpu_shard(A, B, X, act)
    assert oracle.rel_err(p, oracle.shard_forward(X, A, B, act)) <= TOL_F32


# ------------------------------------------------------------------ bf16, small
@pytest.mark.parametrize("path", ["stream", "tiled"])
@pytest.mark.parametrize("act", ["silu_gate", "tanh", "identity"])
@pytest.mark.parametrize("M", [1, 5, 33, 64, 65, 300])
def test_bf16_small_both_paths(path, act, M):
    d, ffn = 512, 1600  # per-rank F = 200 at tp=8: ragged against every tile width
    spec = synth.ModelSpec(d_model=d, ffn=ffn, pieces=8)
    a, b = spec.shard(3, 8, act)
    x = synth.tokens(M, d)
    say("bf16", path, act, "M", M, "d", d, "F", b.shape[0])
    p = gpu_shard(a, b, x, act, path=path)
    err = oracle.rel_err(p, oracle.shard_forward(x, a, b, act))
    say("err", err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("path", ["stream", "tiled"])
@pytest.mark.parametrize("act", ["silu_gate", "tanh", "identity"])
@pytest.mark.parametrize("M,F", [(1, 1), (3, 2), (65, 1)])
def test_bf16_smallest_shards(path, act, M, F):
    """The smallest bf16 shards: d = 64 (one contraction stage of the first product)
    and one or two hidden features, padded internally to a whole tile.  With so few
    hidden features the partial is (nearly) rank one and the one bf16 rounding of H does
    not average out, so the bound adds its worst case (tolerances.tol_hidden_rounding)."""
    g = torch.Generator().manual_seed(100 * M + F)
    cols = 2 * F if act == "silu_gate" else F
    a = (torch.randn(64, cols, generator=g) * 0.2).to(torch.bfloat16)
    b = (torch.randn(F, 64, generator=g) * 0.2).to(torch.bfloat16)
    x = torch.randn(M, 64, generator=g).to(torch.bfloat16)
    say("bf16 smallest", path, act, "M", M, "F", F)
    p = gpu_shard(a, b, x, act, path=path)
    ref = oracle.shard_forward(x, a, b, act)
    h = oracle.shard_forward(x, a, torch.eye(F, dtype=torch.float64), act)  # H itself
    tol = tol_hidden_rounding(h, b, ref)
    err = oracle.rel_err(p, ref)
    say("err", err, "bound", tol)
    assert err <= tol


@pytest.mark.parametrize("path", ["stream", "tiled"])
@pytest.mark.parametrize("M", [7, 300])
def test_bf16_model_width_not_a_tile_multiple(path, M):
    """d = 320 (a multiple of 64, not of the 256-column tile): the down product's last
    column tile is partly stored, and the contraction of the first product is padded
    to whole stages."""
    d, ffn = 320, 800  # per-rank F = 100 at tp=8
    spec = synth.ModelSpec(d_model=d, ffn=ffn, pieces=8)
    a, b = spec.shard(7, 8)
    x = synth.tokens(M, d)
    say("bf16 d=320", path, "M", M, "F", b.shape[0])
    ref = oracle.shard_forward(x, a, b, "silu_gate")
    for out_dtype in (torch.float32, torch.bfloat16):
        p = gpu_shard(a, b, x, "silu_gate", path=path, out_dtype=out_dtype)
        assert p.shape == (M, d) and p.dtype == out_dtype
        err = oracle.rel_err(p, ref)
        say("err", out_dtype, err)
        assert err <= tol_for(out_dtype, ref)


@pytest.mark.parametrize("path", ["stream", "tiled"])
def test_bf16_multi_tile_and_bf16_partial(path):
    d, ffn, M = 1024, 4096, 600  # several tiles in every dimension, ragged token tail
    spec = synth.ModelSpec(d_model=d, ffn=ffn, pieces=8)
    a, b = spec.shard(1, 2)
    x = synth.tokens(M, d)
    say("bf16 multi-tile", path, M, d, b.shape[0])
    ref = oracle.shard_forward(x, a, b, "silu_gate")
    p = gpu_shard(a, b, x, "silu_gate", path=path)
    assert oracle.rel_err(p, ref) <= TOL_BF16
    p16 = gpu_shard(a, b, x, "silu_gate", path=path, out_dtype=torch.bfloat16)
    assert p16.dtype == torch.bfloat16
    assert oracle.rel_err(p16, ref) <= tol_for(torch.bfloat16, ref)


def test_stream_and_tiled_agree_and_are_deterministic():
    d, ffn, M = 2048, 8192, 48
    spec = synth.ModelSpec(d_model=d, ffn=ffn, pieces=8)
    a, b = spec.shard(0, 2)
    x = synth.tokens(M, d).to(DEV)
    say("determinism", M, d)
    sh = {p: tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=M, path=p)
          for p in ("stream", "tiled")}
    try:
        r1 = {p: s.forward(x).cpu() for p, s in sh.items()}
        r2 = {p: s.forward(x).cpu() for p, s in sh.items()}
    finally:
        for s in sh.values():
            s.close()
    for p in sh:
        assert torch.equal(r1[p], r2[p]), p  # bitwise repeatable (fixed-order split-K)
    ref = oracle.shard_forward(x.cpu(), a, b, "silu_gate")
    for p in sh:
        assert oracle.rel_err(r1[p], ref) <= TOL_BF16


@pytest.mark.parametrize("M", [32, 64])
def test_stream_sliced_contraction_narrow_shard(M):
    """A narrow shard (few column blocks, long contraction) makes the streaming path
    slice the contraction over several workgroups and add the slices in a fixed
    order: check it against the oracle and for bitwise repeatability."""
    d, ffn = 8192, 2048  # per-rank F = 256 at tp=8: 16 gate/up column blocks
    spec = synth.ModelSpec(d_model=d, ffn=ffn, pieces=8)
    a, b = spec.shard(5, 8)
    x = synth.tokens(M, d)
    say("sliced stream", M, d, b.shape[0])
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=M, path="stream")
    try:
        xd = x.to(DEV)
        p1 = sh.forward(xd).cpu()
        p2 = sh.forward(xd).cpu()
    finally:
        sh.close()
    assert torch.equal(p1, p2)
    err = oracle.rel_err(p1, oracle.shard_forward(x, a, b, "silu_gate"))
    say("err", err)
    assert err <= TOL_BF16


def test_stream_forced_many_token_groups_narrow_shard():
    """The streaming path forced past one token group (M > 64) on a narrow shard
    with a long contraction: the plan slices the contraction only for a single
    token group, whose scratch and arrival counters the handle holds.  Sliced and
    unsliced calls alternate on one handle (the counters must return to zero)."""
    d, ffn = 8192, 1024  # per-rank F = 128 at tp=8: 8 gate/up column blocks
    spec = synth.ModelSpec(d_model=d, ffn=ffn, pieces=8)
    a, b = spec.shard(6, 8)
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=200, path="stream")
    try:
        for M in (32, 128, 200, 65, 32):
            x = synth.tokens(M, d)
            say("forced stream, narrow shard", "M", M, "d", d, "F", b.shape[0])
            p = sh.forward(x.to(DEV)).cpu()
            err = oracle.rel_err(p, oracle.shard_forward(x, a, b, "silu_gate"))
            say("err", err)
            assert err <= TOL_BF16
    finally:
        sh.close()


def test_m_zero_is_noop():
    spec = synth.ModelSpec(d_model=256, ffn=512, pieces=8)
    a, b = spec.shard(0, 2)
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=8)
    try:
        out = torch.full((0, 256), 7.0, device=DEV)
        x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
        sh.forward(x, out=out)
        torch.cuda.synchronize()
        with pytest.raises(tpm.TpmError):
            sh.forward(torch.zeros((9, 256), dtype=torch.bfloat16, device=DEV))  # > max_tokens
    finally:
        sh.close()


# ------------------------------------------------------------------ the 70B-class configs
def test_decode_shard_tp8_full():
    """Decode shard: one rank of TP=8, d 8192, F 3584, SiLU-gate, M 32, all outputs."""
    a, b = synth.ModelSpec().shard(0, 8)
    x = synth.tokens(32)
    say("decode shard M=32 d=8192 F=3584")
    p = gpu_shard(a, b, x, "silu_gate", max_tokens=64)
    err = oracle.rel_err(p, oracle.shard_forward(x, a, b, "silu_gate"))
    say("decode err", err)
    assert err <= TOL_BF16


def test_prefill_shard_tp8_sampled_rows():
    """Prefill shard: M 8192 on the tiled path, 256 sampled rows (rows 0 and 8191
    among them) against the oracle."""
    a, b = synth.ModelSpec().shard(0, 8)
    x = synth.tokens(8192)
    say("prefill shard M=8192 d=8192 F=3584")
    p = gpu_shard(a, b, x, "silu_gate", max_tokens=8192)
    rows = synth.sample_rows(8192, 256)
    err = oracle.rel_err(p[rows], oracle.shard_forward(x[rows], a, b, "silu_gate"))
    say("prefill err", err)
    assert err <= TOL_BF16
    assert torch.isfinite(p).all()


def test_prefill_shard_ragged_rows_in_split_round():
    """M = 8000 on the TP=8 shard: 896 tiles, whose last round (128 tiles, tile rows 24-31)
    runs as contraction halves, with the last tile row holding 64 of its 256 rows.
    Sampled rows, all rows of that partial tile row among them, against the oracle."""
    a, b = synth.ModelSpec().shard(2, 8)
    M = 8000
    x = synth.tokens(M)
    say("prefill shard M=%d (ragged last tile row in the split round)" % M)
    p = gpu_shard(a, b, x, "silu_gate", max_tokens=M)
    rows = sorted(set(synth.sample_rows(M, 96)) | set(range(7936, M, 9)) | {7936, 7998, 7999})
    err = oracle.rel_err(p[rows], oracle.shard_forward(x[rows], a, b, "silu_gate"))
    say("rows", len(rows), "err", err)
    assert err <= TOL_BF16
    assert torch.isfinite(p).all()


@pytest.mark.parametrize("M,nrows", [(32, None), (2048, 256)])
def test_all_eight_shards_plus_reduce(M, nrows):
    """All 8 rank shards computed one after another, summed by tp_partials_reduce,
    checked against the unsplit MLP."""
    a_sh, b_sh = model_shards(8)
    x = synth.tokens(M)
    say("8 shards + reduce M", M)
    xd = x.to(DEV)
    parts = []
    for a, b in zip(a_sh, b_sh):
        sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=M)
        parts.append(sh.forward(xd))
        torch.cuda.synchronize()
        sh.close()
    Z = tpm.partials_reduce(parts)
    torch.cuda.synchronize()
    Z = Z.cpu()
    rows = list(range(M)) if nrows is None else synth.sample_rows(M, nrows)
    ref = oracle.unsplit_output(x[rows], a_sh, b_sh, "silu_gate")
    err = oracle.rel_err(Z[rows], ref)
    say("8 shards err", err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("tp", [8, 4, 2, 1])
def test_tp_degree_sweep(tp):
    """Sweep: per-rank F = 28672 / tp, M in {1, 8, 32, 64, 4096}."""
    a, b = synth.ModelSpec().shard(0, tp)
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=4096)
    try:
        for M in (1, 8, 32, 64, 4096):
            x = synth.tokens(M)
            say("sweep tp", tp, "M", M)
            p = sh.forward(x.to(DEV))
            torch.cuda.synchronize()
            p = p.cpu()
            rows = synth.sample_rows(M, 64)  # every row for M <= 64
            err = oracle.rel_err(p[rows], oracle.shard_forward(x[rows], a, b, "silu_gate"))
            say("err", err)
            assert err <= TOL_BF16, (tp, M, err)
    finally:
        sh.close()


# ------------------------------------------------------------------ reduce
@pytest.mark.parametrize("k", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("numel", [1, 7, 8, 1000003])
def test_reduce_fp32(k, numel):
    g = torch.Generator().manual_seed(k * 31 + numel)
    parts = [torch.randn(numel, generator=g) for _ in range(k)]
    say("reduce fp32 k", k, "numel", numel)
    Z = tpm.partials_reduce([p.to(DEV) for p in parts]).cpu()
    ref = oracle.partials_sum(parts)
    assert oracle.rel_err(Z, ref) <= TOL_F32
    if k == 1:
        assert torch.equal(Z, parts[0])


def test_reduce_dtypes_inplace_and_determinism():
    g = torch.Generator().manual_seed(5)
    parts = [torch.randn(32, 8192, generator=g) for _ in range(8)]
    ref = oracle.partials_sum(parts)
    pd = [p.to(DEV) for p in parts]
    z16 = tpm.partials_reduce(pd, out_dtype=torch.bfloat16).cpu()
    assert oracle.rel_err(z16, ref) <= TOL_BF16
    pb = [p.to(torch.bfloat16).to(DEV) for p in parts]
    zb = tpm.partials_reduce(pb).cpu()
    assert oracle.rel_err(zb, oracle.partials_sum([p.cpu() for p in pb])) <= TOL_F32
    a1 = tpm.partials_reduce(pd).cpu()
    a2 = tpm.partials_reduce(pd).cpu()
    assert torch.equal(a1, a2)
    inplace = [p.clone() for p in pd]
    tpm.tp_partials_reduce(inplace, inplace[0])
    torch.cuda.synchronize()
    assert torch.equal(inplace[0].cpu(), a1)


# ------------------------------------------------------------------ hooks and capture
def test_timing_events_hook():
    hip = torch.cuda
    a, b = synth.ModelSpec(d_model=1024, ffn=4096).shard(0, 8)
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=32)
    evs = [hip.Event(enable_timing=True) for _ in range(4)]
    for e in evs:  # materialize the underlying events on the current stream
        e.record()
    torch.cuda.synchronize()
    try:
        sh.set_timing_events([e.cuda_event for e in evs])
        x = synth.tokens(32, 1024).to(DEV)
        sh.forward(x)
        torch.cuda.synchronize()
        t1 = evs[0].elapsed_time(evs[1])
        t2 = evs[2].elapsed_time(evs[3])
        say("kernel ms", t1, t2)
        assert t1 > 0 and t2 > 0
        sh.set_timing_events(None)
    finally:
        sh.close()


def test_graph_capture_replays_match_eager():
    a, b = synth.ModelSpec(d_model=1024, ffn=8192).shard(0, 8)
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=32)
    x = synth.tokens(32, 1024).to(DEV)
    out = torch.empty(32, 1024, device=DEV)
    try:
        eager = sh.forward(x).clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            sh.forward(x, out=out)  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sh.forward(x, out=out)
        for i in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), i
            sh.forward(x)  # eager work between replays
            torch.cuda.synchronize()
    finally:
        sh.close()
