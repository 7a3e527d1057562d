"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: a
hand-worked example, a closed form, an invariant, brute force on tiny inputs
or an independent library routine (torch's float64 scaled_dot_product_attention
and logsumexp).  A plausible slip in the oracle (a dropped term, a transposed
operand, pooling queries before the softmax, an exclusive top-p boundary, a
wrong tie order, a divisor of B instead of the ragged block size) fails at
least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, mask=None, scale=None):
    """torch float64 SDPA on CPU: an independent textbook attention."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)
    return out[0, 0].numpy()


# ---------------------------------------------------------------- hand example

def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    q = np.array(g["q"])[:, None]
    k = np.array(g["k"])[:, None]
    v = np.array(g["v"])[:, None]
    b, sc = g["block"], g["scale"]
    np.testing.assert_allclose(O.pool_keys(k, b)[:, 0], g["pooled_keys"], atol=0, rtol=0)
    s = O.score_head(q, k, b, sc)
    np.testing.assert_allclose(s, g["scores"], atol=1e-12)
    for key, p in (("select_p07", 0.7), ("select_p05", 0.5)):
        _, counts, lists = O.select_topp(s[None], [p])
        assert [list(map(int, r)) for r in lists[0]] == g[key]["lists"]
        assert list(counts[0]) == g[key]["counts"]
    out, lse = O.block_sparse_attention(q, k, v, b, g["select_p07"]["lists"], scale=sc)
    np.testing.assert_allclose(out[:, 0], g["attention_out"], atol=1e-12)
    np.testing.assert_allclose(lse, g["attention_lse"], atol=1e-12)
    f = g["drift_scale"]
    d = O.drift((f * q)[None], (f * k)[None], q[None], k[None])
    np.testing.assert_allclose(d, [g["drift_expected"]], rtol=1e-12)
    assert list(O.refresh_decision(d, 0.05)) == [1]
    assert list(O.refresh_decision(d, 0.2)) == [0]


# ---------------------------------------------------------------- pooling

def test_pool_blockwise_constant_keys_ragged():
    n, b, d = 70, 16, 5                     # 5 blocks, last one holds 6 tokens
    nb = O.num_blocks(n, b)
    const = np.random.default_rng(1).integers(-64, 64, (nb, d)) / 8.0   # short dyadics: exact sums
    k = np.repeat(const, b, axis=0)[:n]
    np.testing.assert_array_equal(O.pool_keys(k, b), const)


def test_pool_linear_ramp_closed_form():
    n, b = 45, 8
    k = np.arange(n, dtype=np.float64)[:, None] * np.array([[1.0, -2.0]])
    got = O.pool_keys(k, b)
    for j in range(O.num_blocks(n, b)):
        lo, hi = j * b, min(n, j * b + b)
        mid = (lo + hi - 1) / 2.0            # mean of lo..hi-1
        np.testing.assert_allclose(got[j], [mid, -2 * mid], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- scoring

@pytest.mark.parametrize("n,b,d", [(256, 64, 64), (100, 16, 8), (37, 8, 4)])
def test_score_rows_are_distributions(n, b, d):
    q, k = _rand((1, n, d), 2), _rand((1, n, d), 3)
    s = O.score_blocks(q, k, b)[0]
    assert (s >= 0).all()
    np.testing.assert_allclose(s.sum(axis=1), 1.0, atol=1e-12)


def test_score_zero_queries_is_uniform():
    n, b, d = 90, 16, 8
    s = O.score_blocks(np.zeros((1, n, d)), _rand((1, n, d), 4), b)[0]
    np.testing.assert_allclose(s, 1.0 / O.num_blocks(n, b), atol=1e-15)


def test_score_single_block_is_one():
    s = O.score_blocks(_rand((2, 50, 8), 5), _rand((2, 50, 8), 6), 64)
    np.testing.assert_allclose(s, 1.0, atol=1e-15)


@pytest.mark.parametrize("n,b,d", [(96, 16, 8), (100, 16, 8)])
def test_score_equals_sdpa_over_pooled_keys(n, b, d):
    """Steps 2-4 against torch SDPA: softmax over pooled keys, one-hot values."""
    q, k = _rand((n, d), 7, 2.0), _rand((n, d), 8, 2.0)
    nb = O.num_blocks(n, b)
    kbar = O.pool_keys(k, b)
    per_query = _sdpa(q, kbar, np.eye(nb))           # [n, nb] softmax rows
    want = np.stack([per_query[i * b:min(n, i * b + b)].mean(axis=0) for i in range(nb)])
    np.testing.assert_allclose(O.score_head(q, k, b, 1 / math.sqrt(d)), want, atol=1e-13)


def test_score_is_mean_dense_block_mass_for_blockwise_constant_keys():
    """Keys constant per block and B | N: S is the dense attention mass per block.

    The dense mass comes from torch SDPA over all tokens with block-indicator
    values, so a transposed S, a wrong softmax axis, a missing scale or
    pooling the queries before the softmax all fail here.
    """
    n, b, d = 128, 16, 8
    nb = n // b
    k = np.repeat(_rand((nb, d), 9, 1.5), b, axis=0)
    q = _rand((n, d), 10, 2.0)
    indicator = np.kron(np.eye(nb), np.ones((b, 1)))  # [n, nb]
    mass = _sdpa(q, k, indicator)
    want = mass.reshape(nb, b, nb).mean(axis=1)
    got = O.score_head(q, k, b, 1 / math.sqrt(d))
    np.testing.assert_allclose(got, want, atol=1e-13)
    # pooling queries first (the mismatch PARK's abstract names) differs here
    pooled = O.score_blocks_pooled_query(q[None], k[None], b)[0]
    assert np.abs(pooled - want).max() > 1e-3


def test_score_equal_queries_in_block_equals_pooled_query_scorer():
    n, b, d = 112, 16, 8
    nb = n // b
    q = np.repeat(_rand((nb, d), 11, 2.0), b, axis=0)
    k = _rand((n, d), 12, 2.0)
    np.testing.assert_allclose(O.score_blocks(q[None], k[None], b),
                               O.score_blocks_pooled_query(q[None], k[None], b), atol=1e-14)


def test_pooled_query_scorer_equals_sdpa():
    n, b, d = 100, 16, 8
    q, k = _rand((n, d), 13, 2.0), _rand((n, d), 14, 2.0)
    nb = O.num_blocks(n, b)
    want = _sdpa(O.pool_keys(q, b), O.pool_keys(k, b), np.eye(nb))
    np.testing.assert_allclose(O.score_blocks_pooled_query(q[None], k[None], b)[0], want, atol=1e-13)


def test_score_brute_force_loops_tiny():
    """Pure-Python loops with math.exp on a 1-head, 4-block case."""
    n, b, d = 64, 16, 4
    q, k = _rand((n, d), 15), _rand((n, d), 16)
    sc = 1 / math.sqrt(d)
    nb = n // b
    want = [[0.0] * nb for _ in range(nb)]
    for i_blk in range(nb):
        for i in range(i_blk * b, i_blk * b + b):
            logit = []
            for j_blk in range(nb):
                kb = [sum(k[t][c] for t in range(j_blk * b, j_blk * b + b)) / b for c in range(d)]
                logit.append(sc * sum(q[i][c] * kb[c] for c in range(d)))
            z = sum(math.exp(x) for x in logit)
            for j_blk in range(nb):
                want[i_blk][j_blk] += math.exp(logit[j_blk]) / z / b
    np.testing.assert_allclose(O.score_head(q, k, b, sc), want, atol=1e-13)


# ---------------------------------------------------------------- selection

def _brute_force_topp(s, p):
    """Minimum-size subsets with mass >= p; among them the max-mass one."""
    nb = len(s)
    if p >= 1.0:
        return tuple(range(nb))
    for size in range(1, nb + 1):
        best, best_mass = None, -1.0
        for sub in itertools.combinations(range(nb), size):
            mass = sum(s[j] for j in sub)
            if mass >= p and mass > best_mass:
                best, best_mass = sub, mass
        if best is not None:
            return tuple(sorted(best))
    return tuple(range(nb))


@pytest.mark.parametrize("seed", range(40))
def test_select_matches_subset_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(1, 12))
    s = rng.dirichlet(np.full(nb, 0.5))
    p = float(np.float32(rng.uniform(0.05, 0.99)))
    sel, kstar, _, _ = O.select_row(s, p)
    assert tuple(int(x) for x in sel) == _brute_force_topp(s, p)
    assert kstar == len(sel)


def test_select_boundary_is_inclusive():
    s = np.array([0.125, 0.5, 0.125, 0.25])      # dyadic: sums are exact
    sel, kstar, _, _ = O.select_row(s, 0.75)
    assert kstar == 2 and list(sel) == [1, 3]


def test_select_zero_queries_ceil_rule_and_tie_order():
    n, b, d = 160, 16, 8                           # NB = 10, uniform scores
    s = O.score_blocks(np.zeros((1, n, d)), _rand((1, n, d), 17), b)[0]
    for p in (0.05, 0.33, 0.71, 0.94):
        kk = math.ceil(p * 10)
        _, counts, lists = O.select_topp(s[None], [p])
        assert (counts == kk).all()
        for row in lists[0]:
            assert list(row) == list(range(kk))     # equal scores: lower index first


def test_select_monotone_in_p():
    rng = np.random.default_rng(18)
    s = rng.dirichlet(np.full(40, 0.3), size=20)
    ps = [0.1, 0.3, 0.5, 0.7, 0.9, 0.99]
    prev = None
    for p in ps:
        mask, _, _ = O.select_topp(s[None], [p])
        if prev is not None:
            assert (mask >= prev).all()
        prev = mask


def test_select_extremes_and_cap():
    s = np.random.default_rng(19).dirichlet(np.ones(9), size=5)
    m1, c1, _ = O.select_topp(s[None], [1.0])
    assert (m1 == 1).all() and (c1 == 9).all()
    m0, c0, l0 = O.select_topp(s[None], [0.0])
    assert (c0 == 1).all()
    for i in range(5):
        assert int(l0[0][i][0]) == int(np.argmax(s[i]))
    mc, cc, _ = O.select_topp(s[None], [0.99], max_blocks=3)
    assert (cc <= 3).all() and (mc.sum(axis=-1) == cc).all()


def test_density_counts_pairs():
    counts = np.array([[1, 2, 3], [3, 3, 3]])
    np.testing.assert_allclose(O.density(counts, 3), [6 / 9, 1.0])


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("n,b,d", [(128, 32, 16), (100, 16, 8)])
def test_attention_full_list_equals_dense_sdpa(n, b, d):
    q, k, v = _rand((n, d), 20, 1.5), _rand((n, d), 21, 1.5), _rand((n, d), 22)
    nb = O.num_blocks(n, b)
    lists = [list(range(nb))] * nb
    out, lse = O.block_sparse_attention(q, k, v, b, lists)
    np.testing.assert_allclose(out, _sdpa(q, k, v), atol=1e-13)
    logits = torch.from_numpy(q @ k.T / math.sqrt(d))
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).numpy(), atol=1e-13)


def test_attention_sparse_equals_masked_sdpa():
    n, b, d = 100, 16, 8
    nb = O.num_blocks(n, b)
    rng = np.random.default_rng(23)
    q, k, v = _rand((n, d), 24, 1.5), _rand((n, d), 25, 1.5), _rand((n, d), 26)
    block_mask = rng.random((nb, nb)) < 0.4
    block_mask[np.arange(nb), rng.integers(0, nb, nb)] = True
    lists = [np.flatnonzero(block_mask[i]) for i in range(nb)]
    tok = np.kron(block_mask, np.ones((b, b), bool))[:n, :n]   # independent expansion
    out, _ = O.block_sparse_attention(q, k, v, b, lists)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask=tok), atol=1e-13)


def test_attention_constant_values():
    n, b, d = 80, 16, 4
    q, k = _rand((n, d), 27), _rand((n, d), 28)
    v = np.tile([[0.5, -1.0, 2.0, 3.0]], (n, 1))
    lists = [[j for j in range(5) if (i + j) % 2 == 0] for i in range(5)]
    out, _ = O.block_sparse_attention(q, k, v, b, lists)
    np.testing.assert_allclose(out, v, atol=1e-14)


def test_attention_one_block_is_dense_over_that_block():
    n, b, d = 90, 16, 8
    q, k, v = _rand((n, d), 29), _rand((n, d), 30), _rand((n, d), 31)
    lists = [[3]] * O.num_blocks(n, b)
    out, _ = O.block_sparse_attention(q, k, v, b, lists)
    np.testing.assert_allclose(out, _sdpa(q, k[48:64], v[48:64]), atol=1e-13)
    lists = [[5]] * O.num_blocks(n, b)                      # the ragged block
    out, _ = O.block_sparse_attention(q, k, v, b, lists)
    np.testing.assert_allclose(out, _sdpa(q, k[80:90], v[80:90]), atol=1e-13)


def test_attention_empty_list():
    q = k = v = _rand((32, 4), 32)
    out, lse = O.block_sparse_attention(q, k, v, 16, [[], [0]])
    assert (out[:16] == 0).all() and np.isneginf(lse[:16]).all()
    assert np.isfinite(lse[16:]).all()


# ---------------------------------------------------------------- drift

def test_drift_identical_is_zero():
    q, k = _rand((3, 20, 4), 33), _rand((3, 20, 4), 34)
    assert (O.drift(q, k, q, k) == 0).all()


@pytest.mark.parametrize("eps", [0.01, -0.03, 0.5])
def test_drift_uniform_scaling_is_eps(eps):
    q, k = _rand((2, 30, 4), 35), _rand((2, 30, 4), 36)
    np.testing.assert_allclose(O.drift((1 + eps) * q, (1 + eps) * k, q, k), abs(eps), rtol=1e-12)


def test_drift_closed_form_single_entry():
    q_ref, k_ref = np.ones((1, 10, 2)), np.ones((1, 10, 2))
    q = q_ref.copy()
    q[0, 3, 1] += 0.6
    np.testing.assert_allclose(O.drift(q, k_ref, q_ref, k_ref), [0.6 / math.sqrt(40.0)], rtol=1e-14)


def test_drift_zero_reference():
    z = np.zeros((2, 4, 2))
    q = z.copy()
    q[1, 0, 0] = 1.0
    d = O.drift(q, z, z, z)
    assert d[0] == 0 and np.isinf(d[1])


def test_refresh_only_perturbed_head_and_strict_threshold():
    q, k = _rand((4, 50, 8), 37), _rand((4, 50, 8), 38)
    q2 = q.copy()
    q2[2] += 0.5 * _rand((50, 8), 39)
    d = O.drift(q2, k, q, k)
    assert list(O.refresh_decision(d, 0.05)) == [0, 0, 1, 0]
    tau = float(np.float32(0.25))
    assert list(O.refresh_decision([tau], tau)) == [0]          # "exceeds": strict


# ---------------------------------------------------------------- trajectory

def _walk(h, n, d, steps, sd, seed):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((h, n, d)), rng.standard_normal((h, n, d))
    out = []
    for _ in range(steps):
        out.append((q.copy(), k.copy()))
        q = q + sd * rng.standard_normal(q.shape)
        k = k + sd * rng.standard_normal(k.shape)
    return out


def test_trajectory_infinite_threshold_reuses_step0():
    steps = _walk(2, 64, 8, 5, 0.2, 40)
    res = list(O.cache_trajectory(steps, 16, [0.8, 0.6], np.inf))
    for s, (refresh, _, lists, _, _) in enumerate(res):
        assert refresh.all() if s == 0 else not refresh.any()
        assert lists == res[0][2]


def test_trajectory_zero_threshold_recomputes_every_step():
    steps = _walk(2, 64, 8, 4, 0.2, 41)
    res = list(O.cache_trajectory(steps, 16, [0.8, 0.6], 0.0))
    for (q, k), (refresh, _, lists, counts, scores) in zip(steps, res):
        assert refresh.all()
        fresh = O.score_blocks(q, k, 16)
        np.testing.assert_allclose(scores, fresh, atol=0)
        _, c2, l2 = O.select_topp(fresh, [0.8, 0.6])
        assert (counts == c2).all()
        assert [[list(r) for r in h] for h in lists] == [[list(r) for r in h] for h in l2]


def test_trajectory_drift_is_against_last_refresh_snapshot():
    steps = _walk(1, 64, 8, 6, 0.05, 42)
    res = list(O.cache_trajectory(steps, 16, [0.9], 0.08))
    snap = steps[0]
    for s in range(1, len(steps)):
        refresh, d, _, _, _ = res[s]
        want = O.drift(steps[s][0], steps[s][1], snap[0], snap[1])
        np.testing.assert_allclose(d, want, rtol=1e-14)
        if refresh[0]:
            snap = steps[s]


def test_turbo_decaying_p_is_nested_and_density_non_increasing():
    s = np.random.default_rng(43).dirichlet(np.full(30, 0.4), size=(2, 30))
    stages = O.turbo_schedule(s, [0.95, 0.9, 0.8, 0.6])
    for (m_prev, c_prev), (m, c) in zip(stages, stages[1:]):
        assert (m <= m_prev).all()
        assert (O.density(c, 30) <= O.density(c_prev, 30)).all()


# ---------------------------------------------------------------- retrieval accuracy

@pytest.mark.parametrize("n,b,d", [(96, 16, 8), (100, 16, 8), (37, 8, 5)])
def test_dense_block_mass_equals_sdpa_with_block_indicator_values(n, b, d):
    """Dense block mass against torch SDPA over all tokens with one-hot block
    values (ragged last block included): a wrong softmax axis, a missing
    scale, a divisor of B for the ragged query block or summing over the
    wrong axis all fail here."""
    q, k = _rand((n, d), 41, 2.0), _rand((n, d), 42, 2.0)
    nb = O.num_blocks(n, b)
    owner = np.arange(n) // b
    indicator = np.eye(nb)[owner]                              # [n, nb]
    per_query = _sdpa(q, k, indicator, scale=0.7)              # [n, nb] dense mass per block
    want = np.stack([per_query[i * b:min(n, i * b + b)].mean(axis=0) for i in range(nb)])
    got = O.dense_block_mass(q, k, b, scale=0.7)
    np.testing.assert_allclose(got, want, atol=1e-13)
    np.testing.assert_allclose(got.sum(axis=1), 1.0, atol=1e-13)
    np.testing.assert_allclose(O.dense_block_mass(q, k, b, scale=0.7, query_blocks=[nb - 1, 0]),
                               got[[nb - 1, 0]], atol=0)


def test_dense_block_mass_brute_force_tiny():
    n, b, d = 10, 4, 3                                         # blocks of 4, 4, 2 tokens
    q, k = _rand((n, d), 43), _rand((n, d), 44)
    s = 1 / math.sqrt(d)
    nb = 3
    want = np.zeros((nb, nb))
    for I in range(nb):
        rows = range(I * b, min(n, I * b + b))
        for i in rows:
            w = [math.exp(s * sum(q[i, x] * k[t, x] for x in range(d))) for t in range(n)]
            z = sum(w)
            for t in range(n):
                want[I, t // b] += w[t] / z / len(rows)
    np.testing.assert_allclose(O.dense_block_mass(q, k, b), want, atol=1e-14)


def test_dense_block_mass_closed_forms():
    n, b, d = 100, 16, 8
    k = _rand((n, d), 45)
    # zero queries: uniform attention, mass proportional to block sizes
    sizes = np.array([16] * 6 + [4], float)
    np.testing.assert_allclose(O.dense_block_mass(np.zeros((n, d)), k, b),
                               np.tile(sizes / n, (7, 1)), atol=1e-15)
    # one block: all mass on it
    np.testing.assert_allclose(O.dense_block_mass(_rand((12, d), 46), _rand((12, d), 47), 16), [[1.0]], atol=1e-15)


def test_dense_block_mass_equals_park_scores_for_blockwise_constant_keys():
    """Keys constant within each block and B | N: PARK's per-query block
    softmax is exactly the dense mass (two independent codes agree)."""
    n, b, d = 128, 16, 8
    nb = n // b
    k = np.repeat(_rand((nb, d), 48, 1.5), b, axis=0)
    q = _rand((n, d), 49, 2.0)
    np.testing.assert_allclose(O.dense_block_mass(q, k, b), O.score_head(q, k, b, 1 / math.sqrt(d)),
                               atol=1e-13)


def test_captured_mass():
    m = np.array([[0.5, 0.25, 0.25], [0.1, 0.2, 0.7], [1 / 3, 1 / 3, 1 / 3]])
    assert O.captured_mass(m, [[0], [2], []]) == pytest.approx((0.5 + 0.7 + 0.0) / 3, abs=1e-15)
    assert O.captured_mass(m, [[0, 1, 2]] * 3) == pytest.approx(1.0, abs=1e-15)
    assert O.captured_mass(m, [[1, 2], [0, 1], [2]]) == pytest.approx((0.5 + 0.3 + 1 / 3) / 3, abs=1e-15)


# ------------------------------------------------------- cached correction

def _random_lists(rng, nb, rows, extra=()):
    """Block lists read as sets: random order, repeats and out-of-range entries."""
    out = []
    for r in range(rows):
        c = int(rng.integers(0, nb + 1))
        lst = list(rng.choice(nb, c, replace=False)) + list(extra)
        if c and rng.random() < 0.5:
            lst.append(lst[0])                       # a repeat
        if rng.random() < 0.3:
            lst.append(nb + 3)                       # ignored
        rng.shuffle(lst)
        out.append(np.array(lst, np.int64))
    return out


def test_complement_lists_brute_force():
    rng = np.random.default_rng(71)
    for nb in (1, 2, 5, 9):
        for row, comp in zip(*(lambda l: (l, O.complement_lists(l, nb)))(_random_lists(rng, nb, 30))):
            listed = {int(j) for j in row if 0 <= j < nb}
            assert list(comp) == [j for j in range(nb) if j not in listed]
    assert [list(c) for c in O.complement_lists([[], [0, 1, 2]], 3)] == [[0, 1, 2], []]


@pytest.mark.parametrize("n,b,d", [(40, 8, 4), (37, 8, 5), (64, 16, 8)])
def test_sparse_merged_with_omitted_is_dense(n, b, d):
    """Attention over a list and over its complement join to dense attention,
    whatever the list (empty, full or partial, ragged last block)."""
    rng = np.random.default_rng(n * d)
    q, k, v = (_rand((n, d), 80 + i, 0.7) for i in range(3))
    nb = O.num_blocks(n, b)
    lists = _random_lists(rng, nb, nb)
    lists[0] = np.array([], np.int64)
    lists[-1] = np.arange(nb)
    o_s, l_s = O.block_sparse_attention(q, k, v, b, lists)
    o_o, l_o = O.omitted_attention(q, k, v, b, lists)
    out, lse = O.merge_partial(o_s, l_s, o_o, l_o)
    np.testing.assert_allclose(out, _sdpa(q, k, v), atol=1e-13)
    logits = torch.from_numpy(q @ k.T / np.sqrt(d))
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).numpy(), atol=1e-13)
    # the two parts really are disjoint: full list -> nothing omitted
    assert np.isneginf(l_o[(nb - 1) * b:]).all() and (o_o[(nb - 1) * b:] == 0).all()


def test_merge_with_an_empty_part():
    o = _rand((6, 3), 90)
    l = _rand(6, 91)
    z, ninf = np.zeros((6, 3)), np.full(6, -np.inf)
    out, lse = O.merge_partial(o, l, z, ninf)
    assert (out == o).all() and (lse == l).all()
    out, lse = O.merge_partial(z, ninf, o, l)
    assert (out == o).all() and (lse == l).all()
    out, lse = O.merge_partial(z, ninf, z, ninf)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_merge_weights_closed_form():
    """Equal log-sum-exps average the parts; a gap of log 3 weights them 3:1."""
    a, b_ = np.array([[1.0, -2.0]]), np.array([[5.0, 2.0]])
    out, lse = O.merge_partial(a, np.array([0.4]), b_, np.array([0.4]))
    np.testing.assert_allclose(out, [[3.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(lse, [0.4 + np.log(2.0)], atol=1e-15)
    out, lse = O.merge_partial(a, np.array([np.log(3.0)]), b_, np.array([0.0]))
    np.testing.assert_allclose(out, [[2.0, -1.0]], atol=1e-15)
    np.testing.assert_allclose(lse, [np.log(4.0)], atol=1e-15)


def test_stale_omitted_part_is_exact_when_only_listed_blocks_change():
    """Keys and values of blocks every row keeps change; the omitted blocks do
    not.  The cached omitted part then still holds exactly, and the merge with
    the fresh sparse pass is dense attention on the new inputs."""
    n, b, d = 45, 8, 6
    nb = O.num_blocks(n, b)
    rng = np.random.default_rng(5)
    q = _rand((n, d), 100, 0.6)
    k0, v0 = _rand((n, d), 101, 0.6), _rand((n, d), 102)
    lists = _random_lists(rng, nb, nb, extra=(0, nb - 1))    # every row keeps 0 and the ragged last block
    k1, v1 = k0.copy(), v0.copy()
    for j in (0, nb - 1):
        lo, hi = O.block_bounds(j, n, b)
        k1[lo:hi] += _rand((hi - lo, d), 103 + j, 0.5)
        v1[lo:hi] = _rand((hi - lo, d), 105 + j)
    cached = O.omitted_attention(q, k0, v0, b, lists)
    out, _ = O.merge_partial(*O.block_sparse_attention(q, k1, v1, b, lists), *cached)
    np.testing.assert_allclose(out, _sdpa(q, k1, v1), atol=1e-13)


def test_corrected_trajectory_refresh_is_dense_and_v_change_is_closed_form():
    """Step 0 (every head refreshed) is dense attention.  Step 1 changes only
    V, so no head refreshes: the output is dense attention with the new values
    on the kept blocks and the refresh step's values on the omitted ones."""
    h, n, b, d = 2, 40, 8, 4
    q, k = _rand((h, n, d), 110, 0.8), _rand((h, n, d), 111, 0.8)
    v0, v1 = _rand((h, n, d), 112), _rand((h, n, d), 113)
    steps = list(O.corrected_trajectory([(q, k, v0), (q, k, v1)], b, [0.6, 0.8], tau=0.05))
    refresh, lists, out, lse, s_out, _ = steps[0]
    assert refresh.all()
    for a in range(h):
        np.testing.assert_allclose(out[a], _sdpa(q[a], k[a], v0[a]), atol=1e-13)
        logits = torch.from_numpy(q[a] @ k[a].T / np.sqrt(d))
        np.testing.assert_allclose(lse[a], torch.logsumexp(logits, dim=1).numpy(), atol=1e-13)
    assert np.abs(s_out - out).max() > 1e-3          # the correction is not a no-op here
    refresh, lists1, out, _, _, _ = steps[1]
    assert not refresh.any() and all(
        (np.asarray(x) == np.asarray(y)).all() for la, lb in zip(lists, lists1) for x, y in zip(la, lb))
    nb = O.num_blocks(n, b)
    for a in range(h):
        for i in range(nb):
            lo, hi = O.block_bounds(i, n, b)
            kept = O.token_mask(n, b, lists[a][i])
            vmix = np.where(kept[:, None], v1[a], v0[a])
            want = _sdpa(q[a, lo:hi], k[a], vmix)
            np.testing.assert_allclose(out[a, lo:hi], want, atol=1e-13)


# ------------------------------------------------- query-aware key clustering

def _sk_lloyd(x, init, iters):
    """scikit-learn's Lloyd k-means from fixed initial centres (a library
    implementation independent of the oracle)."""
    from sklearn.cluster import KMeans
    km = KMeans(n_clusters=init.shape[0], init=init, n_init=1, max_iter=iters, algorithm="lloyd", tol=0.0)
    km.fit(x)
    return km.cluster_centers_, km.labels_


def _clustered_keys(n, d, nb, seed, spread=0.25):
    """Keys drawn around nb well separated centres, the centres visited in
    contiguous runs so the contiguous block means start near them."""
    rng = np.random.default_rng(seed)
    centres = rng.standard_normal((nb, d)) * 3.0
    owner = np.minimum(np.arange(n) * nb // n, nb - 1)
    return centres[owner] + spread * rng.standard_normal((n, d))


def test_metric_distance_is_mean_squared_score_gap():
    q = _rand((50, 6), 120)
    k = _rand((10, 6), 121)
    c = _rand(6, 122)
    g = O.query_gram(q)
    want = ((q @ k.T - (q @ c)[:, None]) ** 2).mean(axis=0)
    np.testing.assert_allclose(O.metric_distance(k, c, g), want, rtol=1e-12)


def test_kmeans_identity_metric_is_lloyd():
    """Queries whose Gram matrix is the identity: plain Euclidean k-means,
    checked against scikit-learn's Lloyd iterations from the same start."""
    n, d, b = 120, 4, 20
    q = np.sqrt(d) * np.eye(d)[np.arange(n) % d]
    np.testing.assert_allclose(O.query_gram(q), np.eye(d), atol=1e-15)
    k = _clustered_keys(n, d, n // b, 123, spread=1.5)
    for iters in (1, 3, 8):
        labels, cents, sizes = O.kmeans(k, O.query_gram(q), b, iters)
        sk_c, sk_l = _sk_lloyd(k, O.pool_keys(k, b), iters)
        np.testing.assert_allclose(cents, sk_c, atol=1e-12)
        assert (sizes == np.bincount(labels, minlength=n // b)).all()
    # the library's final labels are the assignment to its final centres
    assert (O.assign(k, cents, np.eye(d))[0] == sk_l).all()


def test_kmeans_query_metric_is_euclidean_on_transformed_keys():
    """G = L L^T: the query metric is Euclidean distance between keys mapped
    by x -> x L, so scikit-learn on the mapped keys reproduces it."""
    n, d, b = 150, 5, 25
    mix = _rand((d, d), 124)
    q = _rand((300, d), 125) @ mix
    g = O.query_gram(q)
    L = np.linalg.cholesky(g)
    k = _clustered_keys(n, d, n // b, 126, spread=1.0)
    for iters in (1, 4):
        labels, cents, _ = O.kmeans(k, g, b, iters)
        sk_c, sk_l = _sk_lloyd(k @ L, O.pool_keys(k, b) @ L, iters)
        np.testing.assert_allclose(cents @ L, sk_c, atol=1e-10)
    assert (O.assign(k, cents, g)[0] == sk_l).all()


def test_cluster_keys_is_kmeans_in_the_query_metric_then_stable_order():
    """The whole clustering of a head, pinned without the oracle's own metric
    helpers: a QR factor of the queries gives R with R^T R = Q^T Q, so the
    query metric is Euclidean distance between keys mapped by x -> x R^T /
    sqrt(N), and scikit-learn's Lloyd from the mapped contiguous block means
    (taken by reshaping, not by the oracle's pooling) gives the centroids.
    Sizes, the means of the returned clusters and the stable order are
    checked by brute force.  The queries see mostly two coordinates, so a
    metric built from the keys instead of the queries clusters differently."""
    rng = np.random.default_rng(131)
    n, d, b = 180, 6, 20
    q = rng.standard_normal((400, d)) * np.array([3.0, 0.2, 2.0, 0.1, 0.1, 0.1])
    k = _clustered_keys(n, d, n // b, 132, spread=1.5)
    R = np.linalg.qr(q, mode="r") / np.sqrt(q.shape[0])
    start = k.reshape(n // b, b, d).mean(axis=1)
    for iters in (1, 3):
        labels, cents, sizes, order = O.cluster_keys(q, k, b, iters)
        sk_c, _ = _sk_lloyd(k @ R.T, start @ R.T, iters)
        np.testing.assert_allclose(cents @ R.T, sk_c, atol=1e-10)
        assert (sizes == np.bincount(labels, minlength=n // b)).all()
        for j in np.flatnonzero(sizes):
            np.testing.assert_allclose(cents[j], k[labels == j].mean(axis=0), atol=1e-12)
        want = np.concatenate([np.flatnonzero(labels == j) for j in range(n // b)])
        assert (order == want).all()
        # the labels are the nearest centroids of the previous iteration's means
        prev = start if iters == 1 else _sk_lloyd(k @ R.T, start @ R.T, iters - 1)[0]
        dist = (((k @ R.T)[:, None, :] - prev[None, :, :] if iters > 1 else
                 (k @ R.T)[:, None, :] - (start @ R.T)[None, :, :]) ** 2).sum(-1)
        assert (labels == np.argmin(dist, axis=1)).all()
    # the same pipeline in the keys' own metric gives other clusters
    wrong, _, _ = O.kmeans(k, k.T @ k / n, b, 3)
    assert (wrong != O.cluster_keys(q, k, b, 3)[0]).any()


def test_query_aware_clusters_group_equal_scores():
    """Queries that only see coordinate 0: keys differ there by sign and
    elsewhere by large noise.  The query metric splits the keys by sign, so
    every cluster's keys get identical scores from every query; Euclidean
    clustering splits by the noise instead."""
    rng = np.random.default_rng(127)
    n, d = 200, 8
    q = np.zeros((60, d))
    q[:, 0] = rng.uniform(0.5, 2.0, 60)
    sign = np.where(np.arange(n) < n // 2, rng.random(n) < 0.7, rng.random(n) < 0.3)
    k = 3.0 * rng.standard_normal((n, d))
    k[:, 0] = np.where(sign, 1.0, -1.0)
    labels, _, _ = O.kmeans(k, O.query_gram(q), n // 2, 3)
    assert (labels == np.where(sign, 0, 1)).all()
    for j in (0, 1):
        scores = q @ k[labels == j].T
        assert np.ptp(scores, axis=1).max() == 0.0
    eu, _, _ = O.kmeans(k, np.eye(d), n // 2, 3)
    assert (eu != labels).mean() > 0.1


def test_kmeans_objective_never_increases():
    k = _rand((90, 4), 128)
    q = _rand((40, 4), 129)
    g = O.query_gram(q)
    prev = np.inf
    c = O.pool_keys(k, 10)
    for _ in range(6):
        labels, dist = O.assign(k, c, g)
        obj = dist[np.arange(90), labels].sum()
        assert obj <= prev + 1e-12
        prev = obj
        c, _ = O.update(k, labels, c)
        # assignment is optimal for the centroids it saw
        assert (dist[np.arange(90), labels] <= dist.min(axis=1) + 0.0).all()


def test_update_means_and_empty_cluster():
    k = _rand((7, 3), 130)
    labels = np.array([2, 0, 2, 2, 0, 3, 3], np.int32)
    c0 = _rand((4, 3), 131)
    c, sizes = O.update(k, labels, c0)
    assert sizes.tolist() == [2, 0, 3, 2]
    np.testing.assert_allclose(c[0], (k[1] + k[4]) / 2, rtol=1e-15)
    np.testing.assert_allclose(c[2], (k[0] + k[2] + k[3]) / 3, rtol=1e-15)
    assert (c[1] == c0[1]).all()


def test_cluster_order_is_stable_sort():
    labels = np.array([3, 1, 3, 0, 1, 1, 3, 0], np.int32)
    assert O.cluster_order(labels).tolist() == [3, 7, 1, 4, 5, 0, 2, 6]


def test_contiguous_clusters_reduce_to_park_blocks():
    """Clusters that are the contiguous blocks: cluster scores are PARK's
    block scores and cluster attention is block-sparse attention."""
    n, b, d = 45, 8, 5
    q, k, v = (_rand((n, d), 132 + i, 0.8) for i in range(3))
    nb = O.num_blocks(n, b)
    labels = (np.arange(n) // b).astype(np.int32)
    cents, sizes = O.update(k, labels, np.zeros((nb, d)))
    np.testing.assert_allclose(cents, O.pool_keys(k, b), rtol=1e-14)
    s = 1 / np.sqrt(d)
    np.testing.assert_allclose(O.cluster_scores(q, cents, sizes, b), O.score_head(q, k, b, s), atol=1e-15)
    rng = np.random.default_rng(135)
    lists = [rng.choice(nb, int(rng.integers(0, nb + 1)), replace=False) for _ in range(nb)]
    o1, l1 = O.cluster_attention(q, k, v, b, labels, lists)
    o2, l2 = O.block_sparse_attention(q, k, v, b, lists)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-13)       # -inf rows match as -inf


def test_cluster_scores_skip_empty_clusters():
    n, b, d = 40, 8, 4
    q, k = _rand((n, d), 136), _rand((n, d), 137)
    labels = np.array([0, 2, 3, 4] * 10, np.int32)            # cluster 1 is empty
    cents, sizes = O.update(k, labels, _rand((5, d), 138))
    sc = O.cluster_scores(q, cents, sizes, b)
    assert (sc[:, 1] == 0).all()
    np.testing.assert_allclose(sc.sum(axis=1), 1.0, rtol=1e-14)
    live = [0, 2, 3, 4]
    want = _sdpa(q, cents[live], np.eye(4), scale=1 / np.sqrt(d))
    np.testing.assert_allclose(sc[:, live], np.stack([want[i * b:(i + 1) * b].mean(0) for i in range(5)]),
                               atol=1e-14)


def test_cluster_attention_full_selection_is_dense():
    n, b, d = 37, 8, 4
    q, k, v = (_rand((n, d), 139 + i) for i in range(3))
    labels = np.random.default_rng(142).integers(0, 5, n).astype(np.int32)
    out, lse = O.cluster_attention(q, k, v, b, labels, [list(range(5))] * 5)
    np.testing.assert_allclose(out, _sdpa(q, k, v), atol=1e-13)
    sel = [[1, 3]] * 5
    out, _ = O.cluster_attention(q, k, v, b, labels, sel)
    mask = np.isin(labels, [1, 3])[None, :].repeat(n, 0)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask=mask), atol=1e-13)
