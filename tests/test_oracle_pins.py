"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test names the passage it rests on.  Pins used:
* hand-derived closed forms (tests/golden/closed_form.json);
* B >= cache length reduces the method to textbook causal attention, checked
  against torch's scaled_dot_product_attention (fp64, explicit mask, its own GQA);
* special cases that reduce to a library routine (cosine row via scipy);
* a pure-Python brute force on tiny inputs (Fig. 1(a)'s 6-token, 3-chunk shape);
* invariants: key/query scaling, cache permutation, softmax rows, MQA/GQA repeats.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.spatial.distance import cdist

from oracle import brute, quoka

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_form.json")))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _chunks(rng, L, C, H_q, H_kv, d):
    out = []
    for t0 in range(0, L, C):
        n = min(C, L - t0)
        out.append((_rand(rng, H_q, n, d), _rand(rng, H_kv, n, d), _rand(rng, H_kv, n, d)))
    return out


# ----------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("case", GOLD["query_keep"])
def test_query_keep_closed_form(case):
    Q = np.array(case["Q"], dtype=np.float64)
    np.testing.assert_allclose(quoka.query_cosines(Q), case["cos"], atol=1e-14)
    for n_q, keep in case["keep"].items():
        assert quoka.query_keep(Q, int(n_q)).tolist() == keep


@pytest.mark.parametrize("case", GOLD["key_scores"])
def test_key_scores_closed_form(case):
    Q = np.array(case["Q"], dtype=np.float64)
    K = np.array(case["K"], dtype=np.float64)
    keep = [np.array(k) for k in case["keep"]]
    np.testing.assert_allclose(quoka.key_scores(Q, keep, K), case["S"], atol=1e-14)


@pytest.mark.parametrize("case", GOLD["top_b"])
def test_top_b_closed_form(case):
    S = np.array(case["S"], dtype=np.float64)
    for B, idx in case["idx"].items():
        assert quoka.top_b(S, int(B)).tolist() == idx


@pytest.mark.parametrize("case", GOLD["attend"])
def test_attend_closed_form(case):
    Q = np.array(case["Q"], dtype=np.float64)
    K_sel = [np.array(x, dtype=np.float64) for x in case["K_sel"]]
    V_sel = [np.array(x, dtype=np.float64) for x in case["V_sel"]]
    Kc = np.array(case["Kc"], dtype=np.float64)
    Vc = np.array(case["Vc"], dtype=np.float64)
    np.testing.assert_allclose(quoka.attend(Q, K_sel, V_sel, Kc, Vc), case["O"], atol=1e-12)


# ----------------------------------------------------------------------------- dense identity

def _sdpa_causal(Q, K, V):
    """Textbook causal attention over the whole prompt via torch (fp64, explicit mask, GQA)."""
    H_q, L, d = Q.shape
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=mask, enable_gqa=True)
    return o[0].numpy()


@pytest.mark.parametrize("L,C,H_q,H_kv,d", [(96, 32, 4, 2, 16), (100, 24, 8, 8, 8), (64, 64, 6, 1, 8), (70, 16, 4, 2, 32)])
def test_budget_covers_cache_equals_dense_causal(L, C, H_q, H_kv, d):
    """QuoKA article, Fig. 1(a): with B >= the cache length nothing is dropped, so chunked
    prefill over the compacted cache is plain dense causal attention over the prompt."""
    rng = np.random.default_rng(L * 7 + C)
    chunks = _chunks(rng, L, C, H_q, H_kv, d)
    res = quoka.prefill(chunks, n_q=3, B=L)
    O = np.concatenate(res["O"], axis=1)
    Q = np.concatenate([c[0] for c in chunks], axis=1)
    K = np.concatenate([c[1] for c in chunks], axis=1)
    V = np.concatenate([c[2] for c in chunks], axis=1)
    np.testing.assert_allclose(O, _sdpa_causal(Q, K, V), atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------- softmax rows

def test_values_all_one_give_one():
    """Softmax rows sum to one: V == 1 makes every output 1 (any selection)."""
    rng = np.random.default_rng(3)
    chunks = [(q, k, np.ones_like(v)) for q, k, v in _chunks(rng, 80, 20, 4, 2, 8)]
    res = quoka.prefill(chunks, n_q=5, B=13)
    for O in res["O"]:
        np.testing.assert_allclose(O, 1.0, atol=1e-13)


def test_one_hot_values_reproduce_probabilities():
    """V[j] = e_j makes O a probability row: non-negative, sums to 1, and the ratio
    of two entries is exp(scale * difference of their logits)."""
    rng = np.random.default_rng(4)
    d, n, C = 16, 5, 4
    Q = _rand(rng, 1, C, d)
    K_sel = [_rand(rng, n, d)]
    Kc = _rand(rng, 1, C, d)
    eye = np.eye(d)
    V_sel = [eye[:n]]
    Vc = eye[n:n + C][None]
    O = quoka.attend(Q, K_sel, V_sel, Kc, Vc)
    s = 1 / math.sqrt(d)
    for i in range(C):
        p = O[0, i]
        assert (p >= 0).all()
        assert abs(p.sum() - 1) < 1e-12
        assert np.all(p[n + i + 1:] == 0)                      # causal: later chunk keys get nothing
        z0 = s * Q[0, i] @ K_sel[0][0]
        for j in range(1, n):
            assert abs(p[j] / p[0] - math.exp(s * Q[0, i] @ K_sel[0][j] - z0)) < 1e-10


# ----------------------------------------------------------------------------- MQA / GQA

def test_mqa_equals_mha_with_repeated_kv():
    """Multi-query attention page, "Teknisk innsikt": with one K/V head every query head
    uses its own query against the same K/V, i.e. MHA with that K/V repeated per head."""
    rng = np.random.default_rng(5)
    H_q, C, d, T = 6, 12, 8, 40
    Q = _rand(rng, H_q, C, d)
    Kp, Vp = _rand(rng, 1, T, d), _rand(rng, 1, T, d)
    Kc, Vc = _rand(rng, 1, C, d), _rand(rng, 1, C, d)
    sel = quoka.select(Q, Kp, n_q=4, B=9)
    idx = sel["idx"][0]
    O1 = quoka.attend(Q, [Kp[0, idx]], [Vp[0, idx]], Kc, Vc)
    Orep = quoka.attend(Q, [Kp[0, idx]] * H_q, [Vp[0, idx]] * H_q,
                        np.repeat(Kc, H_q, axis=0), np.repeat(Vc, H_q, axis=0))
    np.testing.assert_allclose(O1, Orep, atol=1e-14)


def test_gqa_equals_mha_with_repeat_interleave():
    """Reading 10 (head map g = floor(h/G)) against torch's own GQA convention."""
    rng = np.random.default_rng(6)
    H_q, H_kv, C, d = 8, 2, 10, 8
    Q = _rand(rng, H_q, C, d)
    Kc, Vc = _rand(rng, H_kv, C, d), _rand(rng, H_kv, C, d)
    O = quoka.attend(Q, [np.zeros((0, d))] * H_kv, [np.zeros((0, d))] * H_kv, Kc, Vc)
    np.testing.assert_allclose(O, _sdpa_causal(Q, Kc, Vc), atol=1e-13)


def test_single_query_single_head_score_is_cosine_row():
    """N_q = C = 1 and G = 1: the score of key j is cos(q, k_j), a library routine."""
    rng = np.random.default_rng(7)
    H, d, T = 3, 16, 50
    Q = _rand(rng, H, 1, d)
    K = _rand(rng, H, T, d)
    K[1, 7] = 0.0
    S = quoka.key_scores(Q, [np.array([0])] * H, K)
    for h in range(H):
        ref = 1.0 - cdist(Q[h], K[h], metric="cosine")[0]
        ref[np.isnan(ref)] = 0.0                       # zero key: cosine 0 by convention
        if h == 1:
            ref[7] = 0.0
        np.testing.assert_allclose(S[h], ref, atol=1e-14)


def test_group_of_one_is_max_cosine():
    """G = 1: the mean over one head is the identity; S is the max cosine over kept queries."""
    rng = np.random.default_rng(8)
    Q = _rand(rng, 2, 9, 8)
    K = _rand(rng, 2, 30, 8)
    keep = [np.array([1, 4, 8]), np.array([0, 2])]
    S = quoka.key_scores(Q, keep, K)
    for h in range(2):
        ref = (1.0 - cdist(Q[h, keep[h]], K[h], metric="cosine")).max(axis=0)
        np.testing.assert_allclose(S[h], ref, atol=1e-14)


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("L,C,H_q,H_kv,d,n_q,B,seed", [
    (6, 2, 2, 1, 4, 1, 2, 0),          # Fig. 1(a): 6 tokens in 3 chunks of 2
    (6, 2, 4, 2, 4, 1, 1, 1),
    (12, 4, 4, 2, 8, 2, 3, 2),
    (13, 5, 2, 2, 3, 2, 4, 3),         # ragged last chunk
    (20, 4, 6, 3, 5, 3, 6, 4),
    (16, 8, 4, 1, 6, 8, 5, 5),         # N_q >= C keeps every query
])
def test_oracle_matches_brute_force(L, C, H_q, H_kv, d, n_q, B, seed):
    rng = np.random.default_rng(100 + seed)
    chunks = _chunks(rng, L, C, H_q, H_kv, d)
    ref = brute.prefill([tuple(x.tolist() for x in c) for c in chunks], n_q, B)
    got = quoka.prefill(chunks, n_q, B, keep_trace=True)
    for r, g in zip(ref, got["trace"]):
        assert [list(x) for x in g["idx"]] == r["idx"]
        if r["keep"] is None:
            assert g["keep"] is None
        else:
            assert [list(x) for x in g["keep"]] == r["keep"]
            np.testing.assert_allclose(g["S"], np.array(r["S"]), atol=1e-12)
        np.testing.assert_allclose(g["O"], np.array(r["O"]), atol=1e-12)


# ----------------------------------------------------------------------------- top-B

def test_top_b_properties_random():
    rng = np.random.default_rng(9)
    for T, B in [(100, 10), (1000, 123), (57, 57), (57, 80), (3000, 1)]:
        S = np.round(rng.standard_normal(T), 1)        # many exact ties
        idx = quoka.top_b(S, B)
        assert len(idx) == min(B, T)
        assert np.all(np.diff(idx) > 0)
        if B < T:
            rest = np.setdiff1d(np.arange(T), idx)
            assert S[idx].min() >= S[rest].max()
            # ties at the threshold: every unselected key at the threshold has a higher index
            thr = S[idx].min()
            assert rest[S[rest] == thr].min(initial=T) > idx[S[idx] == thr].max()
        ref = sorted(range(T), key=lambda j: (-S[j], j))[:B]   # Python's own stable sort
        assert idx.tolist() == sorted(ref)


# ----------------------------------------------------------------------------- invariances

def test_scaling_keys_and_queries_leaves_selection_unchanged():
    """Cosine ignores positive row scaling: scaled keys (e.g. the x4 sinks) keep their
    score; scaling all queries of a head keeps its sub-selection and the scores."""
    rng = np.random.default_rng(10)
    Q = _rand(rng, 4, 16, 8)
    K = _rand(rng, 2, 60, 8)
    a = quoka.select(Q, K, n_q=5, B=11)
    K2 = K * rng.uniform(0.1, 10, size=(2, 60, 1))
    Q2 = Q * rng.uniform(0.1, 10, size=(4, 1, 1))
    b = quoka.select(Q2, K2, n_q=5, B=11)
    for x, y in zip(a["keep"], b["keep"]):
        assert x.tolist() == y.tolist()
    np.testing.assert_allclose(a["S"], b["S"], atol=1e-13)
    for x, y in zip(a["idx"], b["idx"]):
        assert x.tolist() == y.tolist()


def test_permuting_cache_permutes_selection_and_keeps_output():
    rng = np.random.default_rng(11)
    H_q, H_kv, C, d, T = 4, 2, 8, 8, 50
    Q = _rand(rng, H_q, C, d)
    Kp, Vp = _rand(rng, H_kv, T, d), _rand(rng, H_kv, T, d)
    Kc, Vc = _rand(rng, H_kv, C, d), _rand(rng, H_kv, C, d)
    perm = rng.permutation(T)
    a = quoka.prefill_chunk(Q, Kc, Vc, Kp, Vp, n_q=3, B=12)
    b = quoka.prefill_chunk(Q, Kc, Vc, Kp[:, perm], Vp[:, perm], n_q=3, B=12)
    for g in range(H_kv):
        assert sorted(perm[b["idx"][g]].tolist()) == a["idx"][g].tolist()
    np.testing.assert_allclose(a["O"], b["O"], atol=1e-12)


def test_small_budget_is_not_dense():
    """Sanity: with B < T the method differs from dense attention (selection matters)."""
    rng = np.random.default_rng(12)
    chunks = _chunks(rng, 64, 16, 2, 1, 8)
    O = np.concatenate(quoka.prefill(chunks, n_q=2, B=4)["O"], axis=1)
    Q = np.concatenate([c[0] for c in chunks], axis=1)
    K = np.concatenate([c[1] for c in chunks], axis=1)
    V = np.concatenate([c[2] for c in chunks], axis=1)
    assert np.abs(O - _sdpa_causal(Q, K, V)).max() > 1e-3
