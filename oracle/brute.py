"""Brute-force QuoKA chunk step in pure Python (lists, loops, the math module).

TEST INFRASTRUCTURE ONLY: an independent second reading of the same definition
as oracle/quoka.py, for tiny inputs, written without numpy so that a slip in the
vectorised oracle (a transposed operand, a wrong axis, a dropped term) shows up
as a disagreement.  Sources: QuoKA article (itsolotime.com) Fig. 1(a)-(b), the
method paragraph and Fig. 2; multi-query attention page, "Teknisk innsikt".
"""
from __future__ import annotations

import math
from typing import List, Sequence


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def _cos(a: Sequence[float], b: Sequence[float]) -> float:
    den = math.sqrt(_dot(a, a)) * math.sqrt(_dot(b, b))
    return 0.0 if den == 0.0 else _dot(a, b) / den


def keep_for_head(rows: List[List[float]], n_q: int) -> List[int]:
    C = len(rows)
    if n_q >= C:
        return list(range(C))
    d = len(rows[0])
    mean = [sum(rows[i][e] for i in range(C)) / C for e in range(d)]
    ranked = sorted((_cos(rows[i], mean), i) for i in range(C))   # least similar first
    return sorted(i for _, i in ranked[:n_q])


def _unit(a: Sequence[float]) -> List[float]:
    n = math.sqrt(_dot(a, a))
    return [0.0 if n == 0.0 else x / n for x in a]


def chunk_step(Q: List[List[List[float]]], Kc: List[List[List[float]]], Vc: List[List[List[float]]],
               Kp: List[List[List[float]]], Vp: List[List[List[float]]], n_q: int, B: int,
               scale: float | None = None, pooling: str = "head") -> dict:
    """Q[h][i][e]; Kc/Vc[g][t][e] (chunk); Kp/Vp[g][j][e] (prior cache, T rows).

    pooling="head": S = mean over the group's heads of the max over each head's
    kept queries of the cosine.  pooling="group" (QuoKA article, Table 4
    caption: cost in KV heads): the group's unit query rows are averaged per
    token first, the query rule picks tokens of that pooled stream, and S =
    max over kept tokens of (pooled row . key) / |key|."""
    H_q, C, d = len(Q), len(Q[0]), len(Q[0][0])
    H_kv, T = len(Kp), len(Kp[0])
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    keep = None
    S = None
    if T > B and pooling == "group":
        pooled = []
        for g in range(H_kv):
            rows = []
            for i in range(C):
                units = [_unit(Q[h][i]) for h in range(g * G, (g + 1) * G)]
                rows.append([sum(u[e] for u in units) / G for e in range(d)])
            pooled.append(rows)
        keep = [keep_for_head(pooled[g], n_q) for g in range(H_kv)]
        S = [[0.0] * T for _ in range(H_kv)]
        for g in range(H_kv):
            for j in range(T):
                kn = math.sqrt(_dot(Kp[g][j], Kp[g][j]))
                best = max(_dot(pooled[g][i], Kp[g][j]) for i in keep[g])
                S[g][j] = 0.0 if kn == 0.0 else best / kn
    elif T > B:
        keep = [keep_for_head(Q[h], n_q) for h in range(H_q)]
        S = [[0.0] * T for _ in range(H_kv)]
        for g in range(H_kv):
            for j in range(T):
                tot = 0.0
                for h in range(g * G, (g + 1) * G):
                    tot += max(_cos(Q[h][i], Kp[g][j]) for i in keep[h])
                S[g][j] = tot / G
    if T > B:
        idx = []
        for g in range(H_kv):
            ranked = sorted((-S[g][j], j) for j in range(T))
            idx.append(sorted(j for _, j in ranked[:B]))
    else:
        idx = [list(range(T)) for _ in range(H_kv)]
    O = [[[0.0] * d for _ in range(C)] for _ in range(H_q)]
    for h in range(H_q):
        g = h // G
        for i in range(C):
            keys = [Kp[g][j] for j in idx[g]] + [Kc[g][t] for t in range(i + 1)]
            vals = [Vp[g][j] for j in idx[g]] + [Vc[g][t] for t in range(i + 1)]
            z = [scale * _dot(Q[h][i], k) for k in keys]
            zmax = max(z)
            w = [math.exp(x - zmax) for x in z]
            tot = sum(w)
            for e in range(d):
                O[h][i][e] = sum(w[n] * vals[n][e] for n in range(len(vals))) / tot
    return {"keep": keep, "S": S, "idx": idx, "O": O}


def prefill(chunks, n_q: int, B: int, scale: float | None = None, pooling: str = "head") -> List[dict]:
    """chunks: list of (Q, Kc, Vc) nested lists; returns the per-chunk records."""
    Kp: List[List[List[float]]] = []
    Vp: List[List[List[float]]] = []
    out = []
    for Q, Kc, Vc in chunks:
        H_kv = len(Kc)
        if not Kp:
            Kp = [[] for _ in range(H_kv)]
            Vp = [[] for _ in range(H_kv)]
        out.append(chunk_step(Q, Kc, Vc, Kp, Vp, n_q, B, scale, pooling))
        for g in range(H_kv):
            Kp[g] = Kp[g] + [list(r) for r in Kc[g]]
            Vp[g] = Vp[g] + [list(r) for r in Vc[g]]
    return out


def reuse_slots(prev_pos: Sequence[int], idx: Sequence[int]) -> List[int]:
    """Slot contents after a decode step that selected idx (ascending), by the
    selected-entry cache rule (SQD page, sparse-attention paragraph; the
    reading in oracle/reuse.py): walk the slots in order, keep a slot below
    n = len(idx) whose position is selected again, then hand the remaining
    selected positions, smallest first, to the remaining slots below n,
    lowest first; slots from n on are empty (-1)."""
    n = len(idx)
    selected = set(idx)
    new = [-1] * len(prev_pos)
    taken = set()
    for s in range(n):
        p = prev_pos[s]
        if p >= 0 and p in selected and p not in taken:
            new[s] = p
            taken.add(p)
    waiting = [p for p in idx if p not in taken]
    w = 0
    for s in range(n):
        if new[s] == -1:
            new[s] = waiting[w]
            w += 1
    return new
