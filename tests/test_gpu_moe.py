"""GPU parity of the grouped expert MLP (tp_moe_*) against the fp64 oracle, through
the C ABI: the page's example counts, random counts with empty and ragged groups,
counts that overrun the token rows (clamped), and determinism.  Bounds as in
tests/tolerances.py (bf16 inputs, fp32 accumulation, max-abs over RMS)."""
import ctypes

import pytest
import torch

import oracle
import tensor_mlp_shard_amd as tpm
from tensor_mlp_shard_amd import synth
from tolerances import TOL_BF16, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def run(spec, counts, T=None, act="silu_gate", out_dtype=torch.float32, seed=5, reps=1, path="auto"):
    w1, w2 = spec.weights(act)
    T = sum(counts) if T is None else T
    x = synth.tokens(T, d=spec.d_model, seed=seed)
    ge = tpm.GroupedExperts(w1.to(DEV), w2.to(DEV), act, max_tokens=max(T, 1), out_dtype=out_dtype,
                            path=path)
    try:
        c = torch.tensor(counts, dtype=torch.int32, device=DEV)
        outs = []
        for _ in range(reps):
            y = torch.full((T, spec.d_model), 7.0, device=DEV).to(out_dtype)
            ge.forward(x.to(DEV), c, out=y)
            torch.cuda.synchronize()
            outs.append(y.cpu())
        return x, w1, w2, outs
    finally:
        ge.close()


def check(x, counts, w1, w2, y, act="silu_gate", rows=None):
    n = min(sum(max(c, 0) for c in counts), x.shape[0])
    eff, left = [], n
    for c in counts:
        k = min(max(c, 0), left)
        eff.append(k)
        left -= k
    if rows is None:
        ref = oracle.grouped_experts(x[:n], eff, list(w1), list(w2), act)
        got = y[:n]
    else:
        # only the sampled rows: each through its own expert
        rows = sorted(r for r in rows if r < n)
        sub_counts, off, e_rows = [], 0, []
        for c in eff:
            mine = [r for r in rows if off <= r < off + c]
            sub_counts.append(len(mine))
            e_rows += mine
            off += c
        ref = oracle.grouped_experts(x[e_rows], sub_counts, list(w1), list(w2), act)
        got = y[e_rows]
    err = oracle.rel_err(got, ref)
    say("experts err", err)
    assert err <= tol_for(y.dtype, ref)


PATHS = ["stream", "tiled"]  # both projections: weight streaming or matrix-core tiles


@pytest.mark.parametrize("path", PATHS)
def test_page_example_counts(path):
    spec = synth.ExpertSpec(d_model=1024, ffn_expert=512, n_experts=3)
    counts = [128, 64, 96]
    x, w1, w2, (y,) = run(spec, counts, path=path)
    check(x, counts, w1, w2, y)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("act", ["silu_gate", "tanh", "identity"])
def test_ragged_and_empty_groups(act, path):
    """Experts of 0, 1 and 255-300 tokens: several 128-row tiles per expert on the
    streaming path (partly filled 32-row blocks, empty blocks skipped in both
    projections), partly filled 256-row tiles on the tiled one."""
    spec = synth.ExpertSpec(d_model=512, ffn_expert=300, n_experts=6)
    counts = [0, 300, 1, 255, 256, 257]
    x, w1, w2, (y,) = run(spec, counts, act=act, path=path)
    check(x, counts, w1, w2, y, act)


@pytest.mark.parametrize("path", PATHS)
def test_one_expert_takes_every_token(path):
    """All 500 tokens on the last expert: four row tiles of one expert (the last
    holding 116 rows, its fourth 32-row block partly filled), the others empty."""
    spec = synth.ExpertSpec(d_model=512, ffn_expert=256, n_experts=4)
    counts = [0, 0, 0, 500]
    x, w1, w2, (y,) = run(spec, counts, path=path)
    check(x, counts, w1, w2, y)


@pytest.mark.parametrize("path", PATHS)
def test_sixteen_experts_bf16_out_and_deterministic(path):
    spec = synth.ExpertSpec(d_model=2048, ffn_expert=1024, n_experts=16)
    counts = synth.expert_counts(16)
    x, w1, w2, ys = run(spec, counts, out_dtype=torch.bfloat16, reps=2, path=path)
    assert torch.equal(ys[0], ys[1])
    check(x, counts, w1, w2, ys[0], rows=synth.sample_rows(sum(counts), 200))


@pytest.mark.parametrize("path", PATHS)
def test_counts_past_the_rows_are_clamped_and_rows_past_the_counts_untouched(path):
    spec = synth.ExpertSpec(d_model=256, ffn_expert=128, n_experts=4)
    # the counts claim 40 + 50 + 60 + 70 rows, X holds 100: experts 0, 1 and the first
    # 10 rows of expert 2 are computed, nothing past row 100 is read or written
    x, w1, w2, (y,) = run(spec, [40, 50, 60, 70], T=100, path=path)
    check(x, [40, 50, 60, 70], w1, w2, y)
    # counts summing to less than T: rows past the sum keep their old value
    x, w1, w2, (y,) = run(spec, [10, -3, 5, 0], T=40, path=path)
    check(x, [10, 0, 5, 0], w1, w2, y)
    assert torch.all(y[15:] == 7.0)


@pytest.mark.parametrize("path", PATHS)
def test_default_out_is_zero_past_the_counts(path):
    # no out given and counts summing to less than T: the binding's own output buffer
    # starts at zero, so rows no expert owns come back as zeros (never stale memory)
    spec = synth.ExpertSpec(d_model=256, ffn_expert=128, n_experts=4)
    w1, w2 = spec.weights("silu_gate")
    x = synth.tokens(40, d=spec.d_model, seed=5)
    ge = tpm.GroupedExperts(w1.to(DEV), w2.to(DEV), "silu_gate", max_tokens=40, path=path)
    try:
        torch.empty(40 * 256 * 4, dtype=torch.float32, device=DEV).fill_(7.0)  # dirty the pool
        y = ge.forward(x.to(DEV), torch.tensor([10, 0, 5, 0], dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        y = y.cpu()
    finally:
        ge.close()
    check(x, [10, 0, 5, 0], w1, w2, y)
    assert torch.all(y[15:] == 0.0)


@pytest.mark.parametrize("path", PATHS)
def test_full_size_expert_layer_sampled(path):
    """The 16 experts of one GPU at the 70B-class width (d 8192, expert width 2048)."""
    spec = synth.ExpertSpec()
    counts = synth.expert_counts(spec.n_experts)
    say("16 experts d 8192, F 2048, tokens", sum(counts), "path", path)
    x, w1, w2, (y,) = run(spec, counts, path=path)
    check(x, counts, w1, w2, y, rows=synth.sample_rows(sum(counts), 48))


def test_streaming_launch_at_its_grid_limit():
    """The streaming path takes one grid row per 128-token tile plus one per expert:
    8388352 tokens on one expert fill 65535 rows exactly (sampled rows against the
    oracle); one token more is refused with TPM_ERR_SHAPE before any launch."""
    spec = synth.ExpertSpec(d_model=64, ffn_expert=64, n_experts=1)
    w1, w2 = spec.weights()
    t_ok = 128 * 65534
    ge = tpm.GroupedExperts(w1.to(DEV), w2.to(DEV), max_tokens=t_ok + 1, path="stream")
    try:
        g = torch.Generator(device=DEV).manual_seed(4242)
        x = torch.randn(t_ok + 1, 64, generator=g, device=DEV).to(torch.bfloat16)
        say("streaming grid limit: tokens", t_ok)
        y = ge.forward(x[:t_ok], torch.tensor([t_ok], dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        rows = synth.sample_rows(t_ok, 64)
        ref = oracle.grouped_experts(x[rows].cpu(), [len(rows)], list(w1), list(w2), "silu_gate")
        err = oracle.rel_err(y[rows].cpu(), ref)
        say("err", err)
        assert err <= TOL_BF16
        del y
        with pytest.raises(tpm.TpmError) as e:
            ge.forward(x, torch.tensor([t_ok + 1], dtype=torch.int32, device=DEV))
        assert e.value.status == 2  # TPM_ERR_SHAPE
        torch.cuda.synchronize()
    finally:
        ge.close()


def test_binding_refuses_mismatched_tokens_and_output():
    spec = synth.ExpertSpec(d_model=256, ffn_expert=128, n_experts=2)
    w1, w2 = spec.weights()
    g = tpm.GroupedExperts(w1.to(DEV), w2.to(DEV), max_tokens=64)
    try:
        counts = torch.tensor([8, 8], dtype=torch.int32, device=DEV)
        good = torch.zeros(16, 256, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(ValueError):
            g.forward(torch.zeros(16, 128, dtype=torch.bfloat16, device=DEV), counts)
        with pytest.raises(ValueError):
            g.forward(good.float(), counts)
        with pytest.raises(ValueError):
            g.forward(good, counts, out=torch.empty(8, 256, device=DEV))
        with pytest.raises(ValueError):
            g.forward(good, counts, out=torch.empty(16, 256, dtype=torch.bfloat16, device=DEV))
        y = g.forward(good, counts)
        torch.cuda.synchronize()
        assert y.shape == (16, 256) and torch.all(y == 0)
    finally:
        g.close()
