"""Pins of the oracle's group-pooled scoring (pooling="group") to things other
than itself.  QuoKA article, Table 4 caption (the method's cost counted in KV
heads rather than query heads) read as: pool the group's unit query rows per
token, sub-select on the pooled rows, score S = max over kept tokens of
(pooled row . key) / |key|.

Pins used:
* a hand-derived case where the two pooling orders give different scores;
* the pure-Python brute force (oracle/brute.py) on tiny inputs;
* reductions to the per-head reading: a group of one head with every query
  kept, and a group whose heads share the same unit-norm queries;
* the max-of-means <= mean-of-maxes inequality with every query kept;
* invariance to scaling any single query row or key row by a positive factor;
* a zero query row contributes nothing to the pooled row.
"""
import numpy as np
import pytest

from oracle import brute, quoka


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _chunks(rng, L, C, H_q, H_kv, d):
    out = []
    for t0 in range(0, L, C):
        n = min(C, L - t0)
        out.append((_rand(rng, H_q, n, d), _rand(rng, H_kv, n, d), _rand(rng, H_kv, n, d)))
    return out


def test_pooling_orders_differ_on_hand_case():
    """Two heads, two tokens, d = 2: head 0 asks (1,0) then (0,1), head 1 the
    reverse.  Key (1,0): per-head order gives mean(max(1,0), max(0,1)) = 1;
    pooling first gives pooled rows (1/2, 1/2) for both tokens, so 1/2.
    Key (1,1): per head mean(max(1/sqrt2, 1/sqrt2), ...) = 1/sqrt2; pooled
    (1/2,1/2).(1,1)/sqrt2 = 1/sqrt2."""
    Q = np.array([[[1.0, 0.0], [0.0, 1.0]], [[0.0, 1.0], [1.0, 0.0]]])
    K = np.array([[[1.0, 0.0], [1.0, 1.0], [0.0, 0.0]]])
    keep_all = [np.array([0, 1])]
    Sg = quoka.key_scores_group(quoka.pooled_queries(Q, 1), keep_all, K)
    Sh = quoka.key_scores(Q, [np.array([0, 1])] * 2, K)
    np.testing.assert_allclose(Sg[0], [0.5, 1 / np.sqrt(2), 0.0], atol=1e-15)
    np.testing.assert_allclose(Sh[0], [1.0, 1 / np.sqrt(2), 0.0], atol=1e-15)


def test_pooled_rows_closed_form():
    """qbar = mean of unit rows; a zero row contributes 0 (cos := 0 for zero norms)."""
    Q = np.zeros((2, 3, 2))
    Q[0] = [[3.0, 4.0], [0.0, 0.0], [0.0, -2.0]]
    Q[1] = [[0.0, 5.0], [1.0, 0.0], [0.0, -7.0]]
    qbar = quoka.pooled_queries(Q, 1)[0]
    np.testing.assert_allclose(qbar, [[0.3, 0.9], [0.5, 0.0], [0.0, -1.0]], atol=1e-15)


@pytest.mark.parametrize("L,C,H_q,H_kv,d,n_q,B,seed", [
    (6, 2, 2, 1, 4, 1, 2, 0),          # QuoKA article, Fig. 1(a): 6 tokens, chunks of 2
    (12, 4, 4, 2, 8, 2, 3, 1),
    (13, 5, 6, 2, 3, 2, 4, 2),         # ragged last chunk, G = 3
    (20, 4, 4, 4, 5, 3, 6, 3),         # G = 1
    (16, 8, 8, 1, 6, 8, 5, 4),         # MQA, N_q >= C keeps every token
])
def test_group_oracle_matches_brute_force(L, C, H_q, H_kv, d, n_q, B, seed):
    rng = np.random.default_rng(300 + seed)
    chunks = _chunks(rng, L, C, H_q, H_kv, d)
    ref = brute.prefill([tuple(x.tolist() for x in c) for c in chunks], n_q, B, pooling="group")
    got = quoka.prefill(chunks, n_q, B, keep_trace=True, pooling="group")
    for r, g in zip(ref, got["trace"]):
        assert [list(x) for x in g["idx"]] == r["idx"]
        if r["keep"] is None:
            assert g["keep"] is None
        else:
            assert [list(x) for x in g["keep"]] == r["keep"]
            np.testing.assert_allclose(g["S"], np.array(r["S"]), atol=1e-12)
        np.testing.assert_allclose(g["O"], np.array(r["O"]), atol=1e-12)


def test_group_of_one_with_all_queries_equals_per_head():
    """G = 1 and N_q >= C: the mean over one head is the identity and both
    orders score max_i cos(q_i, k)."""
    rng = np.random.default_rng(20)
    Q, K = _rand(rng, 3, 10, 8), _rand(rng, 3, 40, 8)
    a = quoka.select(Q, K, n_q=10, B=7, pooling="head")
    b = quoka.select(Q, K, n_q=10, B=7, pooling="group")
    np.testing.assert_allclose(a["S"], b["S"], atol=1e-14)
    assert [x.tolist() for x in a["idx"]] == [x.tolist() for x in b["idx"]]


def test_identical_unit_heads_equal_per_head():
    """Every head of a group asks the same unit-norm queries: the pooled row is
    that query, the mean query is the same, so both readings keep the same
    tokens and give the same scores."""
    rng = np.random.default_rng(21)
    H_kv, G, C, d = 2, 4, 12, 8
    base = _rand(rng, H_kv, C, d)
    base /= np.linalg.norm(base, axis=-1, keepdims=True)
    Q = np.repeat(base, G, axis=0)                   # heads g*G .. g*G+G-1 copy group g
    K = _rand(rng, H_kv, 50, d)
    a = quoka.select(Q, K, n_q=4, B=9, pooling="head")
    b = quoka.select(Q, K, n_q=4, B=9, pooling="group")
    for g in range(H_kv):
        assert a["keep"][g * G].tolist() == b["keep"][g].tolist()
    np.testing.assert_allclose(a["S"], b["S"], atol=1e-14)


def test_max_of_means_bounded_by_mean_of_maxes():
    """With every query kept, max_i mean_h c[h,i] <= mean_h max_i c[h,i]."""
    rng = np.random.default_rng(22)
    Q, K = _rand(rng, 8, 9, 6), _rand(rng, 2, 70, 6)
    a = quoka.select(Q, K, n_q=9, B=5, pooling="head")
    b = quoka.select(Q, K, n_q=9, B=5, pooling="group")
    assert np.all(b["S"] <= a["S"] + 1e-14)
    assert np.any(b["S"] < a["S"] - 1e-3)            # and the orders do differ


def test_group_scores_ignore_row_scaling():
    """Pooling unit rows: scaling any single query row (not only a whole head) or
    key row by a positive factor leaves keep, S and the index set unchanged."""
    rng = np.random.default_rng(23)
    Q, K = _rand(rng, 4, 16, 8), _rand(rng, 2, 60, 8)
    a = quoka.select(Q, K, n_q=5, B=11, pooling="group")
    Q2 = Q * rng.uniform(0.1, 10, size=(4, 16, 1))
    K2 = K * rng.uniform(0.1, 10, size=(2, 60, 1))
    b = quoka.select(Q2, K2, n_q=5, B=11, pooling="group")
    for x, y in zip(a["keep"], b["keep"]):
        assert x.tolist() == y.tolist()
    np.testing.assert_allclose(a["S"], b["S"], atol=1e-13)
    for x, y in zip(a["idx"], b["idx"]):
        assert x.tolist() == y.tolist()


def test_unknown_pooling_is_rejected():
    rng = np.random.default_rng(24)
    with pytest.raises(ValueError):
        quoka.select(_rand(rng, 2, 4, 3), _rand(rng, 1, 9, 3), 2, 3, pooling="tokens")
