"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics, not by the oracle.

Each test names what it pins.  A plausible mistake in the oracle (a dropped term, a
wrong sign, a swapped gate/up, a transposed operand, a wrong shard index) fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tensor_mlp_shard_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ACTS = ["tanh", "silu_gate", "identity"]


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def _first_cols(F, act):
    return 2 * F if act == "silu_gate" else F


# ---------------------------------------------------------------- brute force
def _brute(X, A, B, act):
    """Per-element evaluation of the unsplit definition with exactly rounded sums."""
    M, d = X.shape
    F = B.shape[0]
    Z = np.zeros((M, B.shape[1]))
    for m in range(M):
        h = []
        for j in range(F):
            s = math.fsum(X[m, k] * A[k, j] for k in range(d))
            if act == "tanh":
                h.append(math.tanh(s))
            elif act == "identity":
                h.append(s)
            else:
                u = math.fsum(X[m, k] * A[k, F + j] for k in range(d))
                h.append(s / (1.0 + math.exp(-s)) * u)
        for n in range(B.shape[1]):
            Z[m, n] = math.fsum(h[j] * B[j, n] for j in range(F))
    return Z


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("M,d,F", [(1, 1, 1), (2, 3, 4), (3, 4, 6), (3, 2, 5)])
def test_brute_force_tiny(act, M, d, F):
    """Pin: brute force on tiny shapes (M<=3, d<=4, F<=6) for every activation."""
    X = _rand((M, d), 1)
    A = _rand((d, _first_cols(F, act)), 2)
    B = _rand((F, d), 3)
    got = oracle.shard_forward(X, A, B, act)
    ref = _brute(X, A, B, act)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- the pages' invariant
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_sum_of_partials_equals_unsplit(act, k):
    """Pin: sum_i act(X A_i) B_i equals the unsplit MLP (the column->row identity)."""
    M, d, F = 5, 48, 64
    X = _rand((M, d), 10)
    G = _rand((d, F), 11, 0.2)
    U = _rand((d, F), 12, 0.2)
    B = _rand((F, d), 13, 0.2)
    w = F // k
    if act == "silu_gate":
        a_shards = [np.concatenate([G[:, r * w:(r + 1) * w], U[:, r * w:(r + 1) * w]], axis=1)
                    for r in range(k)]
        A_full = np.concatenate([G, U], axis=1)
    else:
        a_shards = [G[:, r * w:(r + 1) * w] for r in range(k)]
        A_full = G
    b_shards = [B[r * w:(r + 1) * w] for r in range(k)]
    split = oracle.tensor_parallel_output(X, a_shards, b_shards, act)
    whole = oracle.shard_forward(X, A_full, B, act)
    assert oracle.rel_err(split, whole) < 1e-13
    # and the reassembled weights are the originals
    A2, B2 = oracle.unsplit_weights(a_shards, b_shards, act)
    assert np.array_equal(A2, A_full) and np.array_equal(B2, B)


# ---------------------------------------------------------------- library special case
@pytest.mark.parametrize("M,d,F", [(1, 8, 8), (7, 33, 20), (16, 64, 96)])
def test_identity_is_matrix_chain(M, d, F):
    """Pin: with no activation the MLP is the matrix chain X A B (NumPy float64 matmul)."""
    X = _rand((M, d), 20)
    A = _rand((d, F), 21)
    B = _rand((F, d), 22)
    got = oracle.shard_forward(X, A, B, "identity")
    ref = (X @ A) @ B
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_tanh_matches_numpy_composition():
    """Pin: the pages' NumPy form sum_i tanh(x @ a_i) @ b_i, evaluated with NumPy."""
    M, d, F, k = 3, 16, 24, 2
    x = _rand((M, d), 30)
    A = _rand((d, F), 31, 0.3)
    B = _rand((F, d), 32, 0.3)
    a_sh = [A[:, :12], A[:, 12:]]
    b_sh = [B[:12], B[12:]]
    ref = np.sum([np.tanh(x @ a) @ b for a, b in zip(a_sh, b_sh)], axis=0)
    got = oracle.tensor_parallel_output(x, a_sh, b_sh, "tanh")
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("act", ACTS)
def test_zero_input_gives_zero(act):
    """Pin: tanh(0) = SiLU(0) = 0, so X = 0 gives Z = 0."""
    d, F = 12, 10
    X = np.zeros((4, d))
    A = _rand((d, _first_cols(F, act)), 40)
    B = _rand((F, d), 41)
    assert np.all(oracle.shard_forward(X, A, B, act) == 0.0)


@pytest.mark.parametrize("act", ACTS)
def test_zero_second_weight_gives_zero(act):
    """Pin: B = 0 gives Z = 0 whatever the hidden values."""
    d, F = 12, 10
    X = _rand((4, d), 42)
    A = _rand((d, _first_cols(F, act)), 43)
    B = np.zeros((F, d))
    assert np.all(oracle.shard_forward(X, A, B, act) == 0.0)


def test_scalar_tanh_closed_form():
    """Pin: tanh(ln 2) = 3/5 exactly, so x=1, a=ln 2, b=5 gives Z = 3."""
    Z = oracle.shard_forward([[1.0]], [[math.log(2.0)]], [[5.0]], "tanh")
    assert Z.shape == (1, 1)
    assert abs(Z[0, 0] - 3.0) < 1e-14


def test_scalar_silu_gate_closed_form():
    """Pin: sigma(ln 3) = 3/4.  Gate pre-activation ln 3 and up value 2 give
    h = (3/4) ln 3 * 2; with b = 1/ln 3 the output is exactly 1.5.  SiLU with the sign
    flipped would give 0.5; SiLU on the up branch would give SiLU(2) = 1.7616."""
    ln3 = math.log(3.0)
    Z = oracle.shard_forward([[1.0]], [[ln3, 2.0]], [[1.0 / ln3]], "silu_gate")
    assert abs(Z[0, 0] - 1.5) < 1e-14


def test_silu_limits():
    """Pin: SiLU(x) -> x for large x and -> 0 for very negative x."""
    Zp = oracle.shard_forward([[1.0]], [[40.0, 1.0]], [[1.0]], "silu_gate")
    Zn = oracle.shard_forward([[1.0]], [[-40.0, 1.0]], [[1.0]], "silu_gate")
    assert abs(Zp[0, 0] - 40.0) < 1e-12
    assert abs(Zn[0, 0]) < 1e-15


def test_one_hot_row_selects_row_of_first_weight():
    """Pin: a one-hot token e_k sees the k-th row of A; identity act then gives A[k] B."""
    d, F = 6, 5
    A = _rand((d, F), 50)
    B = _rand((F, d), 51)
    for k in range(d):
        X = np.zeros((1, d))
        X[0, k] = 1.0
        Z = oracle.shard_forward(X, A, B, "identity")
        ref = np.array([sum(A[k, j] * B[j, n] for j in range(F)) for n in range(d)])
        np.testing.assert_allclose(Z[0], ref, rtol=1e-13, atol=1e-15)


def test_linear_in_second_weight_and_homogeneous_for_identity():
    """Pin: Z is linear in B for every activation; for identity it is linear in X too."""
    d, F = 10, 7
    X = _rand((3, d), 60)
    A = _rand((d, 2 * F), 61)
    B1 = _rand((F, d), 62)
    B2 = _rand((F, d), 63)
    z1 = oracle.shard_forward(X, A, B1, "silu_gate")
    z2 = oracle.shard_forward(X, A, B2, "silu_gate")
    z12 = oracle.shard_forward(X, A, 2.0 * B1 - B2, "silu_gate")
    np.testing.assert_allclose(z12, 2.0 * z1 - z2, rtol=1e-12, atol=1e-12)
    Ai = A[:, :F]
    zx = oracle.shard_forward(X, Ai, B1, "identity")
    z3x = oracle.shard_forward(3.0 * X, Ai, B1, "identity")
    np.testing.assert_allclose(z3x, 3.0 * zx, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- indexing
@pytest.mark.parametrize("act", ACTS)
def test_hidden_permutation_invariance(act):
    """Pin: permuting hidden indices consistently (columns of gate and up, rows of B)
    leaves Z unchanged; permuting only the up columns does not."""
    M, d, F = 4, 20, 16
    X = _rand((M, d), 70)
    G = _rand((d, F), 71, 0.3)
    U = _rand((d, F), 72, 0.3)
    B = _rand((F, d), 73, 0.3)
    perm = np.random.default_rng(74).permutation(F)
    if act == "silu_gate":
        A, Ap = np.concatenate([G, U], 1), np.concatenate([G[:, perm], U[:, perm]], 1)
    else:
        A, Ap = G, G[:, perm]
    z = oracle.shard_forward(X, A, B, act)
    zp = oracle.shard_forward(X, Ap, B[perm], act)
    assert oracle.rel_err(zp, z) < 1e-13
    if act == "silu_gate":
        zbad = oracle.shard_forward(X, np.concatenate([G, U[:, perm]], 1), B, act)
        assert oracle.rel_err(zbad, z) > 1e-2


def test_fused_gate_up_naive_split_is_not_the_method():
    """The rank's gate and up blocks must cover the same hidden indices: slicing a
    fused [G | U] weight into contiguous blocks pairs gate j with up j' != j and
    changes the result.  (The layout reading the shards follow.)"""
    M, d, F, k = 3, 16, 8, 2
    X = _rand((M, d), 80)
    G = _rand((d, F), 81, 0.5)
    U = _rand((d, F), 82, 0.5)
    B = _rand((F, d), 83, 0.5)
    whole = oracle.shard_forward(X, np.concatenate([G, U], 1), B, "silu_gate")
    w = F // k
    right = oracle.tensor_parallel_output(
        X, [np.concatenate([G[:, r * w:(r + 1) * w], U[:, r * w:(r + 1) * w]], 1) for r in range(k)],
        [B[r * w:(r + 1) * w] for r in range(k)], "silu_gate")
    fused = np.concatenate([G, U], 1)
    naive = oracle.tensor_parallel_output(
        X, [fused[:, r * 2 * w:(r + 1) * 2 * w] for r in range(k)],
        [B[r * w:(r + 1) * w] for r in range(k)], "silu_gate")
    assert oracle.rel_err(right, whole) < 1e-13
    assert oracle.rel_err(naive, whole) > 1e-2


def test_rows_are_independent_bitwise():
    """Row sampling (used at large M) returns exactly the rows of the full result."""
    M, d, F = 9, 24, 16
    X = _rand((M, d), 90)
    A = _rand((d, 2 * F), 91, 0.3)
    B = _rand((F, d), 92, 0.3)
    full = oracle.shard_forward(X, A, B, "silu_gate")
    rows = [0, 3, 8]
    sub = oracle.shard_forward(X[rows], A, B, "silu_gate")
    assert np.array_equal(sub, full[rows])


# ---------------------------------------------------------------- the worked example
def test_p3_worked_example_tp4_exact():
    """Pin: the page's TP=4 worked example shapes, with small integers so that the
    exact product X W1 W2 is known in integer arithmetic; split and unsplit both equal it."""
    spec = json.load(open(os.path.join(GOLDEN, "p3_worked_example_tp4.json")))
    tp = spec["tp"]
    rng = np.random.default_rng(2024)
    Bt = 3
    X = rng.integers(-3, 4, size=(Bt, spec["x_cols"]))
    W1 = rng.integers(-3, 4, size=tuple(spec["w1_shape"]))
    W2 = rng.integers(-3, 4, size=tuple(spec["w2_shape"]))
    exact = (X.astype(np.int64) @ W1.astype(np.int64)) @ W2.astype(np.int64)
    bw1 = spec["w1_block_shape"][1]
    bw2 = spec["w2_block_shape"][0]
    a_sh = [W1[:, r * bw1:(r + 1) * bw1] for r in range(tp)]
    b_sh = [W2[r * bw2:(r + 1) * bw2] for r in range(tp)]
    assert all(a.shape == tuple(spec["w1_block_shape"]) for a in a_sh)
    assert all(b.shape == tuple(spec["w2_block_shape"]) for b in b_sh)
    # The example's second weight is 8 x 4: the layer output has 4 columns, not 8.
    Z = oracle.tensor_parallel_output(X, a_sh, b_sh, "identity")
    assert Z.shape == (Bt, spec["w2_shape"][1])
    assert np.array_equal(Z, exact.astype(np.float64))
    assert np.array_equal(oracle.unsplit_output(X, a_sh, b_sh, "identity"), exact.astype(np.float64))


def test_p4_printed_value_is_recorded_not_fitted():
    spec = json.load(open(os.path.join(GOLDEN, "p4_printed_output.json")))
    assert spec["usable_as_pin"] is False and len(spec["printed"][0]) == 2


# ---------------------------------------------------------------- reduce
def test_partials_sum_rank_order_and_copy():
    """Pin: k=1 is a copy; the sum equals an exactly rounded sum within one rounding."""
    rng = np.random.default_rng(100)
    parts = [rng.normal(size=(7, 5)) for _ in range(8)]
    assert np.array_equal(oracle.partials_sum(parts[:1]), parts[0])
    got = oracle.partials_sum(parts)
    ref = np.array([[math.fsum(p[i, j] for p in parts) for j in range(5)] for i in range(7)])
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14)
    # rank order: ((p0 + p1) + p2) ... exactly
    seq = parts[0].copy()
    for p in parts[1:]:
        seq = seq + p
    assert np.array_equal(got, seq)


def test_shard_count_mismatch_raises():
    """The pages' function pairs shards with zip(strict=True): a count mismatch is an error."""
    x = np.ones((1, 2))
    with pytest.raises(ValueError):
        oracle.tensor_parallel_output(x, [np.ones((2, 1))] * 2, [np.ones((1, 2))] * 3)


# ---------------------------------------------------------------- the checker bites
def _small_model(k=4, d=256, ffn=512):
    spec = synth.ModelSpec(d_model=d, ffn=ffn, pieces=8)
    X = synth.tokens(8, d)
    a, b = spec.shards(k)
    return spec, X, a, b


def test_checker_catches_dropped_shard():
    _, X, a, b = _small_model()
    ref = oracle.tensor_parallel_output(X, a, b, "silu_gate")
    bad = oracle.tensor_parallel_output(X, a[:-1], b[:-1], "silu_gate")
    assert oracle.rel_err(bad, ref) > 2e-2


def test_checker_catches_swapped_gate_up():
    _, X, a, b = _small_model()
    ref = oracle.tensor_parallel_output(X, a, b, "silu_gate")
    sw = [torch.cat([t[:, t.shape[1] // 2:], t[:, : t.shape[1] // 2]], 1) for t in a]
    bad = oracle.tensor_parallel_output(X, sw, b, "silu_gate")
    assert oracle.rel_err(bad, ref) > 2e-2


def test_checker_catches_single_element_perturbation():
    _, X, a, b = _small_model()
    ref = oracle.tensor_parallel_output(X, a, b, "silu_gate")
    rms = float(np.sqrt(np.mean(ref * ref)))
    bad = ref.copy()
    bad[3, 17] += 3 * 2e-2 * rms
    assert oracle.rel_err(bad, ref) > 2e-2
    bad32 = ref.copy()
    bad32[0, 0] += 3 * 1e-5 * rms
    assert oracle.rel_err(bad32, ref) > 1e-5


def test_checker_catches_transposed_second_weight():
    d = 64
    spec = synth.ModelSpec(d_model=d, ffn=d * 8, pieces=8)
    X = synth.tokens(4, d)
    a, b = spec.shard(0, 8)  # F_i = d, so B_i is square and a transpose type-checks
    ref = oracle.shard_forward(X, a, b, "silu_gate")
    bad = oracle.shard_forward(X, a, b.T.contiguous(), "silu_gate")
    assert oracle.rel_err(bad, ref) > 2e-2


# ------------------------------------------------- partials sum + residual + RMSNorm
# Pins of oracle.reduce_add_rmsnorm (page "7.4 推理侧并行", section 7.4.2, kernel
# fusion of the residual add and RMSNorm after the all-reduce; RMSNorm in its
# textbook form y = h / sqrt(mean(h^2) + eps) * gamma).

def _norm_case(k, rows, cols, seed):
    parts = [_rand((rows, cols), seed + i) for i in range(k)]
    res = _rand((rows, cols), seed + 100)
    gamma = _rand((cols,), seed + 200) + 1.0
    return parts, res, gamma


def _norm_brute(parts, res, gamma, eps):
    """Element by element with exactly rounded sums (math.fsum), no NumPy reductions."""
    rows, cols = res.shape
    H = [[0.0] * cols for _ in range(rows)]
    Y = [[0.0] * cols for _ in range(rows)]
    for r in range(rows):
        for c in range(cols):
            H[r][c] = math.fsum([float(res[r, c])] + [float(p[r, c]) for p in parts])
        ms = math.fsum(v * v for v in H[r]) / cols
        inv = 1.0 / math.sqrt(ms + eps)
        for c in range(cols):
            Y[r][c] = H[r][c] * inv * float(gamma[c])
    return np.array(H), np.array(Y)


@pytest.mark.parametrize("k,rows,cols,eps", [(1, 1, 8, 0.0), (2, 3, 16, 1e-6), (3, 2, 24, 0.5),
                                             (8, 4, 40, 1e-5)])
def test_norm_brute_force_tiny(k, rows, cols, eps):
    parts, res, gamma = _norm_case(k, rows, cols, 31 + k)
    h, y = oracle.reduce_add_rmsnorm(parts, res, gamma, eps)
    hb, yb = _norm_brute(parts, res, gamma, eps)
    np.testing.assert_allclose(h, hb, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_norm_constant_row_closed_form():
    # h = c in every column: mean(h^2) = c^2, so y = c / sqrt(c^2 + eps) * gamma
    cols, c, eps = 64, 0.75, 0.0625
    parts = [np.full((1, cols), 0.5), np.full((1, cols), 0.125)]
    res = np.full((1, cols), 0.125)
    gamma = np.linspace(-2.0, 2.0, cols)
    h, y = oracle.reduce_add_rmsnorm(parts, res, gamma, eps)
    assert np.all(h == c)
    np.testing.assert_allclose(y[0], c / math.sqrt(c * c + eps) * gamma, rtol=1e-15)
    # c = 0.75, eps = 0.0625: sqrt(0.5625 + 0.0625) = sqrt(0.625)
    np.testing.assert_allclose(y[0, -1], 0.75 / math.sqrt(0.625) * 2.0, rtol=1e-15)


def test_norm_unit_rms_and_eps_shrink():
    parts, res, gamma = _norm_case(3, 5, 96, 7)
    ones = np.ones(96)
    h, y = oracle.reduce_add_rmsnorm(parts, res, ones, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    eps = 0.3
    _, y2 = oracle.reduce_add_rmsnorm(parts, res, ones, eps)
    ms = np.mean(h * h, axis=1)
    np.testing.assert_allclose(np.mean(y2 * y2, axis=1), ms / (ms + eps), rtol=1e-13)


def test_norm_scale_and_sign_invariance():
    parts, res, gamma = _norm_case(4, 3, 48, 9)
    _, y = oracle.reduce_add_rmsnorm(parts, res, gamma, 0.0)
    _, ys = oracle.reduce_add_rmsnorm([2.5 * p for p in parts], 2.5 * res, gamma, 0.0)
    _, yn = oracle.reduce_add_rmsnorm([-p for p in parts], -res, gamma, 0.0)
    np.testing.assert_allclose(ys, y, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(yn, -y, rtol=0, atol=0)


def test_norm_residual_out_is_residual_plus_sum():
    parts, res, gamma = _norm_case(3, 4, 32, 11)
    h, _ = oracle.reduce_add_rmsnorm(parts, res, gamma, 1e-6)
    np.testing.assert_array_equal(h, oracle._f64(res) + oracle.partials_sum(parts))


def test_norm_pins_catch_planted_mistakes():
    """Plausible wrong readings of the step, each rejected by one of the pins."""
    parts, res, gamma = _norm_case(3, 3, 40, 13)
    eps = 0.01
    _, ref = _norm_brute(parts, res, gamma, eps)
    H = oracle._f64(res) + oracle.partials_sum(parts)
    wrong = {
        "residual dropped": (H - oracle._f64(res)),
        "mean subtracted (LayerNorm)": H - H.mean(axis=1, keepdims=True),
    }
    for name, hh in wrong.items():
        y = hh / np.sqrt(np.mean(hh * hh, axis=1, keepdims=True) + eps) * gamma
        assert np.max(np.abs(y - ref)) > 1e-3, name
    variants = {
        "eps outside the root": H / (np.sqrt(np.mean(H * H, axis=1, keepdims=True)) + eps) * gamma,
        "sum instead of mean": H / np.sqrt(np.sum(H * H, axis=1, keepdims=True) + eps) * gamma,
        "gamma not applied": H / np.sqrt(np.mean(H * H, axis=1, keepdims=True) + eps),
        "root-mean over columns - 1": H / np.sqrt(np.sum(H * H, axis=1, keepdims=True)
                                                  / (H.shape[1] - 1) + eps) * gamma,
    }
    for name, y in variants.items():
        assert np.max(np.abs(y - ref)) > 1e-3, name


# ------------------------------------------------------------------ FP8 partials
# Pins of the E4M3 codec and of the per-row quantizer (page "7.4 推理侧并行",
# section 7.4.2, communication quantization; E4M3 values from the OCP FP8 format).

def test_e4m3_known_codes():
    known = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0xC0: -2.0, 0x7E: 448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x77: 240.0,
             0x30: 0.5, 0xB8: -1.0, 0x6F: 120.0}
    for c, v in known.items():
        assert oracle.e4m3_value(c) == v, hex(c)
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0


def test_e4m3_roundtrip_and_monotonic():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = [oracle.e4m3_value(c) for c in finite]
    enc = oracle.e4m3_encode(np.array(vals))
    for c, e, v in zip(finite, enc, vals):
        if v == 0.0:
            assert e in (0x00, 0x80)
        else:
            assert e == c, (hex(c), hex(int(e)))
    pos = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))


def test_e4m3_ties_to_even_and_saturation():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 1.5 * 2.0 ** -9: 0x02, 0.5 * 2.0 ** -9: 0x00,
             2.5 * 2.0 ** -9: 0x02, 432.0: 0x7E, 416.0: 0x7D, 400.0: 0x7C, 448.0: 0x7E, 463.9: 0x7E,
             1e9: 0x7E, -1e9: 0xFE, -1.0625: 0xB8, 1.07: 0x39}
    got = oracle.e4m3_encode(np.array(list(cases)))
    for (x, c), g in zip(cases.items(), got):
        assert g == c, (x, hex(int(g)), hex(c))


def test_quantize_fp8_rows():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(6, 64, generator=g)
    x[2] = 0.0
    x[4] *= 1e-3
    codes, scales = oracle.quantize_fp8(x)
    X = x.numpy()
    for r in range(6):
        if r == 2:
            assert scales[r] == 1.0 and np.all(codes[r] == 0)
            continue
        amax = np.float32(np.max(np.abs(X[r])))
        assert scales[r] == np.float32(amax / np.float32(448.0))
        # the largest magnitude lands on +-448
        j = int(np.argmax(np.abs(X[r])))
        assert codes[r, j] & 0x7F == 0x7E
        # every element within half a grid spacing (relative 2^-4) of its code
        deq = np.array([oracle.e4m3_value(int(c)) for c in codes[r]]) * float(scales[r])
        assert np.all(np.abs(deq - X[r]) <= np.abs(X[r]) * 2.0 ** -4 + 2.0 ** -10 * float(scales[r]))


def test_reduce_fp8_is_sum_of_dequantized():
    g = torch.Generator().manual_seed(4)
    parts = [torch.randn(3, 32, generator=g) for _ in range(4)]
    qs = [oracle.quantize_fp8(p) for p in parts]
    z = oracle.reduce_fp8([q for q, _ in qs], [s for _, s in qs])
    want = sum(np.array([[oracle.e4m3_value(int(c)) for c in row] for row in q]) * s[:, None].astype(np.float64)
               for q, s in qs)
    np.testing.assert_array_equal(z, want)
    # and it is within the E4M3 rounding of the exact sum: each partial element is
    # off by at most half a grid spacing, 2^-4 of its magnitude (2^-10 scale units
    # in the subnormal range)
    exact = oracle.partials_sum(parts)
    bound = sum(np.abs(oracle._f64(p)) * 2.0 ** -4 + 2.0 ** -10 * s[:, None].astype(np.float64)
                for p, (_, s) in zip(parts, qs))
    assert np.all(np.abs(z - exact) <= bound)


# ------------------------------------------------------------ single projections
# oracle.projection (page "大模型推理系统揭秘（07）Multi-GPU", sections 1.2.2 and
# 1.2.4: Y = XW; QKV column-parallel, output projection row-parallel).

def test_projection_brute_force_tiny():
    X = _rand((3, 5), 1)
    W = _rand((5, 4), 2)
    Y = oracle.projection(X, W)
    for i in range(3):
        for j in range(4):
            assert Y[i, j] == pytest.approx(math.fsum(float(X[i, k]) * float(W[k, j])
                                                      for k in range(5)), rel=1e-14, abs=1e-15)


def test_projection_chain_matches_mlp_identity():
    # two projections in a row = the MLP with the identity activation (C oracle)
    X, A, B = _rand((4, 16), 3), _rand((16, 24), 4), _rand((24, 16), 5)
    np.testing.assert_allclose(oracle.projection(oracle.projection(X, A), B),
                               oracle.shard_forward(X, A, B, "identity"), rtol=1e-12, atol=1e-12)


def test_attention_tp_identity_with_a_per_head_core():
    """Column shards of W_qkv, a core that acts within each head, row shards of W_o:
    the rank partials sum to the unsplit block (the column -> row identity of
    section 1.2.3 applied to attention, section 1.2.4).  The core here is a
    stand-in that keeps heads separate: tanh of each query head's values."""
    spec = synth.AttentionSpec(d_model=64, q_heads=8, kv_heads=4, head_dim=8,
                               dtype=torch.float32, std=0.2)
    X = _rand((5, 64), 6)
    full_q = []
    parts = []
    for r in range(4):
        wqkv, wo = spec.shard(r, 4)
        y = oracle.projection(X, wqkv)
        a = np.tanh(y[:, :spec.q_width(4)])
        parts.append(oracle.projection(a, wo))
        full_q.append((wqkv[:, :spec.q_width(4)], wo))
    Wq = np.concatenate([oracle._f64(q) for q, _ in full_q], axis=1)
    Wo = np.concatenate([oracle._f64(o) for _, o in full_q], axis=0)
    want = oracle.projection(np.tanh(oracle.projection(X, Wq)), Wo)
    np.testing.assert_allclose(oracle.partials_sum(parts), want, rtol=1e-12, atol=1e-12)
    # the shards slice one model: degree 2 gives the same block
    parts2 = []
    for r in range(2):
        wqkv, wo = spec.shard(r, 2)
        a = np.tanh(oracle.projection(X, wqkv)[:, :spec.q_width(2)])
        parts2.append(oracle.projection(a, wo))
    np.testing.assert_allclose(oracle.partials_sum(parts2), want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- grouped experts
# oracle.grouped_experts (page "大模型推理系统揭秘（07）Multi-GPU", MoE section).

def _experts(E, d, F, seed):
    spec = synth.ExpertSpec(d_model=d, ffn_expert=F, n_experts=E, dtype=torch.float32, std=0.2)
    return spec.weights("silu_gate")


def test_experts_single_group_is_the_mlp():
    w1, w2 = _experts(1, 16, 12, 0)
    X = _rand((7, 16), 21)
    np.testing.assert_array_equal(oracle.grouped_experts(X, [7], [w1[0]], [w2[0]]),
                                  oracle.shard_forward(X, w1[0], w2[0], "silu_gate"))


def test_experts_page_example_counts_rowwise():
    # the page's grouped-GEMM example: one GPU's experts receive 128, 64 and 96 tokens
    w1, w2 = _experts(3, 16, 8, 1)
    counts = [128, 64, 96]
    X = _rand((sum(counts), 16), 22)
    Y = oracle.grouped_experts(X, counts, list(w1), list(w2))
    off = 0
    for e, n in enumerate(counts):
        for r in (off, off + n - 1):  # first and last row of each group, brute force
            h = []
            for j in range(8):
                g = math.fsum(float(X[r, k]) * float(w1[e][k, j]) for k in range(16))
                u = math.fsum(float(X[r, k]) * float(w1[e][k, 8 + j]) for k in range(16))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for c in range(16):
                want = math.fsum(h[j] * float(w2[e][j, c]) for j in range(8))
                assert Y[r, c] == pytest.approx(want, rel=1e-12, abs=1e-13)
        off += n


def test_experts_permuting_groups_permutes_rows_and_empty_groups():
    w1, w2 = _experts(4, 16, 8, 2)
    counts = [3, 0, 5, 2]
    X = _rand((10, 16), 23)
    Y = oracle.grouped_experts(X, counts, list(w1), list(w2))
    # experts in the order 2, 0, 3 (expert 1 has no tokens): rows move with their groups
    order = [2, 0, 3]
    offs = {0: 0, 2: 3, 3: 8}
    rows = sum([list(range(offs[e], offs[e] + counts[e])) for e in order], [])
    Y2 = oracle.grouped_experts(X[rows], [counts[e] for e in order], [w1[e] for e in order],
                                [w2[e] for e in order])
    np.testing.assert_array_equal(Y2, Y[rows])
    with pytest.raises(ValueError):
        oracle.grouped_experts(X, [3, 0, 5, 1], list(w1), list(w2))
