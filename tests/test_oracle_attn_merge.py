"""Pins for the oracle's merge of attention partials (page "LLM 推理并行化：先找瓶颈，
再决定怎么切", section 三.4, decode context parallelism).

The page states that merging the ranks' partials (local maximum, sum of
exponentials, exponential-weighted value sum) gives the attention output of the
whole, unsplit KV history.  The main pin computes every partial by brute force
from raw scores and values (math.fsum) and compares the merge with softmax
attention over all keys, written as its textbook formula.  The rest are
invariants of the definition and the edge cases, plus plausible wrong merges that
the main pin must reject.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _attention_full(scores, values):
    """softmax(scores) @ values for one query, exactly rounded sums."""
    mx = max(scores)
    w = [math.exp(z - mx) for z in scores]
    den = math.fsum(w)
    return np.array([math.fsum(wj * values[j][c] for j, wj in enumerate(w)) / den
                     for c in range(len(values[0]))])


def _partial(scores, values, dim):
    """One rank's partial over its keys: (weighted value sum, maximum, sum of exps)."""
    if not scores:
        return np.zeros(dim), -math.inf, 0.0
    mx = max(scores)
    w = [math.exp(z - mx) for z in scores]
    v = np.array([math.fsum(wj * values[j][c] for j, wj in enumerate(w)) for c in range(dim)])
    return v, mx, math.fsum(w)


def _case(rows, L, dim, cuts, seed, scale=1.0):
    """Scores and values for `rows` queries over L keys, and the rank partials for the
    key ranges given by `cuts` (contiguous shards of the KV history; empty allowed)."""
    rng = np.random.default_rng(seed)
    scores = rng.normal(0.0, scale, size=(rows, L))
    values = rng.normal(0.0, 1.0, size=(L, dim))
    bounds = [0] + list(cuts) + [L]
    vals, maxs, sums = [], [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        vs, ms, ss = [], [], []
        for r in range(rows):
            v, m, s = _partial(list(scores[r, lo:hi]), values[lo:hi].tolist(), dim)
            vs.append(v), ms.append(m), ss.append(s)
        vals.append(np.array(vs)), maxs.append(np.array(ms)), sums.append(np.array(ss))
    full = np.array([_attention_full(list(scores[r]), values.tolist()) for r in range(rows)])
    return vals, maxs, sums, full


@pytest.mark.parametrize("cuts", [(), (5,), (3, 9, 10), (0, 7, 7, 15), (1, 2, 3, 4, 5, 6, 7)])
def test_merge_equals_attention_over_all_keys(cuts):
    vals, maxs, sums, full = _case(rows=4, L=16, dim=5, cuts=cuts, seed=len(cuts))
    out, gmax, gsum = oracle.attn_partials_merge(vals, maxs, sums)
    assert np.max(np.abs(out - full)) <= 1e-13 * np.max(np.abs(full))
    # merged statistics: the global maximum and the sum of exponentials relative to it
    rng = np.random.default_rng(len(cuts))
    scores = rng.normal(0.0, 1.0, size=(4, 16))
    assert np.array_equal(gmax, scores.max(axis=1))
    ref = [math.fsum(math.exp(z - scores[r].max()) for z in scores[r]) for r in range(4)]
    assert np.allclose(gsum, ref, rtol=1e-14, atol=0)


def test_large_scores_do_not_overflow():
    """The reason the page gives for the maximum: scores near 1000 overflow exp in
    fp64 without it; the merge stays finite and equals attention."""
    vals, maxs, sums, full = _case(rows=3, L=12, dim=4, cuts=(4, 8), seed=9, scale=1.0)
    shifted = [m + 1000.0 for m in maxs]
    out, gmax, _ = oracle.attn_partials_merge(vals, shifted, sums)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - full)) <= 1e-13 * np.max(np.abs(full))
    assert np.array_equal(gmax, np.max(np.stack(shifted), axis=0))


def test_single_rank_is_its_own_normalised_output():
    rng = np.random.default_rng(3)
    v, m, s = rng.normal(size=(6, 8)), rng.normal(size=6), rng.uniform(1.0, 9.0, size=6)
    out, gmax, gsum = oracle.attn_partials_merge([v], [m], [s])
    assert np.allclose(out, v / s[:, None], rtol=1e-15, atol=0)
    assert np.array_equal(gmax, m) and np.array_equal(gsum, s)


def test_rank_order_and_grouping_do_not_change_the_result():
    vals, maxs, sums, full = _case(rows=5, L=24, dim=6, cuts=(5, 11, 17), seed=4)
    flat, _, _ = oracle.attn_partials_merge(vals, maxs, sums)
    perm = [2, 0, 3, 1]
    permuted, _, _ = oracle.attn_partials_merge([vals[i] for i in perm], [maxs[i] for i in perm],
                                                [sums[i] for i in perm])
    assert np.max(np.abs(permuted - flat)) <= 1e-14
    # merge ranks 0-1 and 2-3 first, then merge the two merged partials: the merged
    # value sum is out * sum (relative to the merged maximum)
    a, am, asum = oracle.attn_partials_merge(vals[:2], maxs[:2], sums[:2])
    b, bm, bsum = oracle.attn_partials_merge(vals[2:], maxs[2:], sums[2:])
    two, _, _ = oracle.attn_partials_merge([a * asum[:, None], b * bsum[:, None]], [am, bm],
                                           [asum, bsum])
    assert np.max(np.abs(two - flat)) <= 1e-14


def test_shifting_a_partials_reference_maximum_changes_nothing():
    """A partial (v, m, s) and (v e^-c, m + c, s e^-c) describe the same keys."""
    vals, maxs, sums, full = _case(rows=4, L=10, dim=3, cuts=(6,), seed=5)
    c = 2.5
    out, _, _ = oracle.attn_partials_merge([vals[0] * math.exp(-c), vals[1]],
                                           [maxs[0] + c, maxs[1]], [sums[0] * math.exp(-c), sums[1]])
    assert np.max(np.abs(out - full)) <= 1e-13


def test_empty_ranks_contribute_nothing_and_no_keys_gives_zero():
    vals, maxs, sums, full = _case(rows=2, L=8, dim=4, cuts=(0, 8), seed=6)  # ranks 0 and 2 empty
    assert np.all(np.isneginf(maxs[0])) and np.all(sums[2] == 0)
    out, _, _ = oracle.attn_partials_merge(vals, maxs, sums)
    assert np.max(np.abs(out - full)) <= 1e-13
    z = np.zeros((3, 4))
    out, gmax, gsum = oracle.attn_partials_merge([z, z], [np.full(3, -np.inf)] * 2, [np.zeros(3)] * 2)
    assert np.array_equal(out, z) and np.all(np.isneginf(gmax)) and np.array_equal(gsum, np.zeros(3))


def _wrong_no_rescale(vals, maxs, sums):
    return sum(vals) / sum(sums)[:, None]


def _wrong_average_of_outputs(vals, maxs, sums):
    return sum(v / s[:, None] for v, s in zip(vals, sums)) / len(vals)


def _wrong_sign(vals, maxs, sums):
    g = np.max(np.stack(maxs), axis=0)
    sc = [np.exp(g - m) for m in maxs]
    return sum(c[:, None] * v for c, v in zip(sc, vals)) / sum(c * s for c, s in zip(sc, sums))[:, None]


@pytest.mark.parametrize("wrong", [_wrong_no_rescale, _wrong_average_of_outputs, _wrong_sign])
def test_the_attention_pin_rejects_plausible_wrong_merges(wrong):
    vals, maxs, sums, full = _case(rows=4, L=16, dim=5, cuts=(3, 9), seed=7, scale=2.0)
    assert np.max(np.abs(wrong(vals, maxs, sums) - full)) > 1e-3


def test_page_printed_merge_is_recorded_not_fitted():
    with open(os.path.join(GOLDEN, "p4_dcp_printed_output.json")) as f:
        g = json.load(f)
    assert g["usable_as_pin"] is False and len(g["printed"]) == 2
