"""The seeded input generators: deterministic, and every TP degree slices one model."""
import torch

from tensor_mlp_shard_amd import synth


def test_same_seed_same_values():
    a = synth.randn((5, 7), seed=3, std=0.02, dtype=torch.bfloat16)
    b = synth.randn((5, 7), seed=3, std=0.02, dtype=torch.bfloat16)
    c = synth.randn((5, 7), seed=4, std=0.02, dtype=torch.bfloat16)
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_bf16_is_round_to_nearest_of_fp32_draw():
    v32 = synth.randn((64,), seed=9, std=0.02)
    v16 = synth.randn((64,), seed=9, std=0.02, dtype=torch.bfloat16)
    assert torch.equal(v32.to(torch.bfloat16), v16)


def test_degrees_slice_the_same_model():
    spec = synth.ModelSpec(d_model=64, ffn=256, pieces=8)
    a1, b1 = spec.shard(0, 1)
    F = 256
    for tp in (2, 4, 8):
        w = F // tp
        for r in range(tp):
            a, b = spec.shard(r, tp)
            assert a.shape == (64, 2 * w) and b.shape == (w, 64)
            assert torch.equal(a[:, :w], a1[:, r * w:(r + 1) * w])          # gate block
            assert torch.equal(a[:, w:], a1[:, F + r * w:F + (r + 1) * w])  # up block, same indices
            assert torch.equal(b, b1[r * w:(r + 1) * w])


def test_tanh_shard_is_gate_weight():
    spec = synth.ModelSpec(d_model=32, ffn=64, pieces=8)
    a, _ = spec.shard(1, 2, "tanh")
    g, _ = spec.shard(1, 2, "silu_gate")
    assert torch.equal(a, g[:, :32])


def test_seed_offset_gives_distinct_model():
    s0 = synth.ModelSpec(d_model=32, ffn=64, pieces=8)
    s1 = synth.ModelSpec(d_model=32, ffn=64, pieces=8, seed_offset=100)
    assert not torch.equal(s0.shard(0, 8)[0], s1.shard(0, 8)[0])


def test_toy_case_shapes_and_split():
    X, a, b = synth.toy_shards(2)
    assert X.shape == (4, 64) and X.dtype == torch.float32
    assert [t.shape for t in a] == [(64, 128)] * 2 and [t.shape for t in b] == [(128, 64)] * 2


def test_sample_rows_holds_ends():
    rows = synth.sample_rows(8192, 64)
    assert rows[0] == 0 and rows[-1] == 8191 and len(rows) == 64 and rows == sorted(set(rows))
    assert synth.sample_rows(5, 64) == [0, 1, 2, 3, 4]
