"""Pins of the selected-entry reuse oracle (oracle/reuse.py) to things other
than itself: hand-derived slot contents, the pure-Python brute force, the
invariants the rule must keep, and the method's own output (softmax attention
does not depend on key order, so every decode step with reuse must give the
output of the same step without it)."""
import json
import os

import numpy as np
import pytest

from oracle import brute, quoka, reuse

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_form.json")))


@pytest.mark.parametrize("case", GOLDEN["reuse_slots"], ids=lambda c: str(c["prev"]) + "->" + str(c["idx"]))
def test_reuse_slots_closed_form(case):
    r = reuse.reuse_slots(np.array(case["prev"]), np.array(case["idx"]))
    assert r["pos"].tolist() == case["pos"]
    assert r["hits"] == case["hits"] and r["misses"] == case["misses"]
    assert brute.reuse_slots(case["prev"], case["idx"]) == case["pos"]


def _random_state(rng, B, T):
    """A reachable previous state: some n0 <= B distinct positions < T in slots [0, n0)."""
    n0 = int(rng.integers(0, min(B, T) + 1))
    prev = np.full(B, -1, dtype=np.int64)
    prev[:n0] = rng.choice(T, size=n0, replace=False)
    return prev


def test_reuse_matches_brute_force_random():
    rng = np.random.default_rng([0x5EED, 71])
    for _ in range(600):
        B = int(rng.integers(1, 40))
        T = int(rng.integers(1, 90))
        prev = _random_state(rng, B, T)
        n = min(B, T)
        idx = np.sort(rng.choice(T, size=n, replace=False)) if rng.random() < 0.7 else \
            np.sort(rng.choice(T, size=int(rng.integers(0, n + 1)), replace=False))
        got = reuse.reuse_slots(prev, idx)["pos"].tolist()
        assert got == brute.reuse_slots(prev.tolist(), idx.tolist()), (prev, idx)


def test_reuse_invariants_random():
    """Slots [0, n) hold exactly the selected set, the rest are empty; a hit keeps
    its slot; hits + misses = n; misses fill the free slots in ascending order."""
    rng = np.random.default_rng([0x5EED, 72])
    for _ in range(400):
        B = int(rng.integers(1, 64))
        T = int(rng.integers(1, 200))
        prev = _random_state(rng, B, T)
        n = min(B, T)
        idx = np.sort(rng.choice(T, size=n, replace=False))
        r = reuse.reuse_slots(prev, idx)
        pos = r["pos"]
        assert sorted(pos[:n].tolist()) == idx.tolist() and np.all(pos[n:] == -1)
        assert np.all(pos[r["hit"]] == prev[r["hit"]])
        assert r["hits"] + r["misses"] == n
        assert r["hits"] == len(set(prev[:n].tolist()) & set(idx.tolist()))
        assert np.all(np.diff(r["miss_slots"]) > 0) and np.all(np.diff(r["miss_pos"]) > 0)


@pytest.mark.parametrize("H_q,H_kv,d,B", [(4, 2, 8, 6), (4, 1, 16, 10), (6, 3, 8, 1)])
def test_decode_with_reuse_equals_decode_without(H_q, H_kv, d, B):
    """Consecutive decode steps over a growing cache: with the selected-entry
    cache every step's kept set and output equal the plain step's (output within
    fp64 rounding), and the slots always hold exactly the kept positions."""
    rng = np.random.default_rng([0x5EED, 73, H_q, B])
    T0, steps = 5, 9
    K = rng.standard_normal((H_kv, T0 + steps, d))
    V = rng.standard_normal((H_kv, T0 + steps, d))
    prev = np.full((H_kv, B), -1, dtype=np.int64)
    hits_total = 0
    for t in range(steps):
        T = T0 + t
        q = rng.standard_normal((H_q, 1, d)) + 2.0 * np.repeat(np.ones((1, 1, d)), H_q, axis=0)
        kn, vn = K[:, T:T + 1], V[:, T:T + 1]
        plain = quoka.prefill_chunk(q, kn, vn, K[:, :T], V[:, :T], 1, B)
        r = reuse.decode_step(q, kn, vn, K[:, :T], V[:, :T], prev, 1, B)
        for g in range(H_kv):
            assert np.array_equal(r["idx"][g], plain["idx"][g])
            n = len(plain["idx"][g])
            assert sorted(r["pos"][g, :n].tolist()) == plain["idx"][g].tolist()
        assert np.abs(r["O"] - plain["O"]).max() < 1e-12
        hits_total += int(r["hits"].sum())
        prev = r["pos"]
    assert hits_total > 0            # consecutive steps do share kept entries
