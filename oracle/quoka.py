"""CPU oracle for QuoKA chunked prefill: query sub-selection, cosine key scoring,
group-aware pooling, per-KV-head top-B, compaction and dense attention over the
compacted cache plus the chunk's own causal keys.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the bench's
CPU-baseline leg may import this module.  It shares no code with the HIP path
(neither imports the other) and is deliberately plain: fp64 numpy, no fusion,
no reordering beyond blocking the score matrix over keys so large prompts fit
in host memory (blocking over keys does not change any value: each key's score
is computed from its own column).

Sources (web pages on QuoKA, QUILT and multi-query attention):

* QuoKA article ("Qualcomm QuoKA", itsolotime.com), Figure 1(a): a prompt is cut
  into chunks; for each chunk the KV cache is first sub-selected, then the
  compacted cache goes through a dense attention kernel.
* Same page, Figure 1(b): queries are first filtered by cosine dissimilarity,
  then keys are filtered by query-key cosine similarity.
* Same page, method paragraph after Figure 1: three steps - query
  sub-selection, cosine-similarity scoring, group-aware aggregation; max pooling
  keeps strong interactions, mean pooling adapts the score to grouped-query
  attention (GQA).
* Same page, Figure 2: queries with a high S_q (low cosine to the mean query)
  interact more strongly with keys; S_q orders queries by dissimilarity.
* Multi-query attention page (aiunderstanding.org), "Teknisk innsikt": every
  query head uses its own query against one shared K/V head.

Readings taken where the pages are silent (each is listed in the design notes):

1. pooling order: mean over the query heads of a KV head, of the max over that
   head's retained queries;
2. query sub-selection is per query head;
3. the mean query is the arithmetic mean of the raw query rows of the chunk;
4. "least similar" = smallest cosine; ties keep the lower token index;
5. selection covers the prior cache [0, T); the chunk's own keys are always
   attended, causally;
6. T <= B keeps every prior key (no selection);
7. N_q >= C keeps every query;
8. softmax scale 1/sqrt(d) unless given; no bias, dropout or positional term;
9. queries and keys are consumed as given (any positional encoding is applied upstream);
10. KV head of query head h is floor(h / G), G = H_q / H_kv;
11. cos(x, y) = 0 when |x||y| = 0;
12. top-B ties keep the lower key index; index sets are reported ascending.

Group-pooled scoring (pooling="group", the other reading of the pooling order):
the QuoKA article's Table 4 caption states the method's cost with the number
of KV heads in place of the number of query heads.  Read as pooling first:
for each KV head g and chunk token i, qbar[g, i] = the mean over the G query
heads of g of q[h, i] / |q[h, i]| (a zero row contributes 0); the query
sub-selection is the per-head rule applied to the pooled rows qbar[g]; the
key score is S[g, j] = max over kept i of qbar[g, i] . k_j / |k_j|, which is
the max over kept tokens of the mean over heads of cos(q[h, i], k_j).

Every function takes fp64 arrays (exact widenings of the bf16 / fp32 inputs).
Nothing here is pinned only to itself: see tests/test_oracle_pins.py.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

KEY_BLOCK = 2048  # keys per block of the score matrix (memory only; values unchanged)


def _norms(X: np.ndarray) -> np.ndarray:
    return np.sqrt(np.einsum("...d,...d->...", X, X))


def _safe_div(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """num / den with 0 where den == 0 (cosine of a zero vector is defined as 0)."""
    out = np.zeros(np.broadcast(num, den).shape, dtype=np.float64)
    np.divide(num, den, out=out, where=(den != 0))
    return out


# ----------------------------------------------------------------------------- step 1

def query_cosines(Qh: np.ndarray) -> np.ndarray:
    """cos(q_i, m) for every query row q_i of one head, m = mean query of the chunk.

    QuoKA article, Fig. 1(b) (cosine dissimilarity filter) and Fig. 2 (S_q).
    Qh: [C, d] -> [C].
    """
    m = Qh.mean(axis=0)
    return _safe_div(Qh @ m, _norms(Qh) * np.linalg.norm(m))


def query_keep(Qh: np.ndarray, n_q: int) -> np.ndarray:
    """Indices of the min(n_q, C) least-similar queries (smallest cosine to the mean
    query, ties -> lower index), ascending.  QuoKA article, Fig. 1(b), Fig. 2."""
    C = Qh.shape[0]
    if n_q >= C:
        return np.arange(C, dtype=np.int64)
    c = query_cosines(Qh)
    order = np.lexsort((np.arange(C), c))          # ascending cosine, then index
    return np.sort(order[:n_q]).astype(np.int64)


def keep_all_heads(Qc: np.ndarray, n_q: int) -> List[np.ndarray]:
    return [query_keep(Qc[h], n_q) for h in range(Qc.shape[0])]


# ----------------------------------------------------------------------------- steps 2-3

def key_scores(Qc: np.ndarray, keep: Sequence[np.ndarray], K: np.ndarray) -> np.ndarray:
    """S[g, j] = mean over the G query heads h of KV head g of
    max over i in keep[h] of cos(Q_c[h, i], K[g, j]).

    QuoKA article, Fig. 1(b) (query-key cosine filter) and the method paragraph
    (max pooling over queries, then mean pooling over the group for GQA).
    Qc: [H_q, C, d]; K: [H_kv, T, d] (prior cache) -> S: [H_kv, T].
    """
    H_q = Qc.shape[0]
    H_kv, T, _ = K.shape
    G = H_q // H_kv
    S = np.zeros((H_kv, T), dtype=np.float64)
    for g in range(H_kv):
        kn = _norms(K[g])
        for h in range(g * G, (g + 1) * G):
            Qs = Qc[h, np.asarray(keep[h], dtype=np.int64)]
            qn = _norms(Qs)
            for j0 in range(0, T, KEY_BLOCK):
                j1 = min(T, j0 + KEY_BLOCK)
                cos = _safe_div(Qs @ K[g, j0:j1].T, qn[:, None] * kn[None, j0:j1])
                S[g, j0:j1] += cos.max(axis=0)
        S[g] /= G
    return S


# ----------------------------------------------------------------------------- group pooling

def pooled_queries(Qc: np.ndarray, H_kv: int) -> np.ndarray:
    """qbar[g, i] = (1/G) * sum over the G query heads h of KV head g of
    q[h, i] / |q[h, i]| (0 for a zero row).  QuoKA article, Table 4 caption
    (cost in KV heads) and the method paragraph (mean pooling over the group).
    Qc: [H_q, C, d] -> [H_kv, C, d]."""
    H_q, C, d = Qc.shape
    G = H_q // H_kv
    unit = _safe_div(Qc, _norms(Qc)[..., None])
    return unit.reshape(H_kv, G, C, d).mean(axis=1)


def key_scores_group(Qbar: np.ndarray, keep: Sequence[np.ndarray], K: np.ndarray) -> np.ndarray:
    """S[g, j] = max over i in keep[g] of qbar[g, i] . k_j / |k_j| (0 for a zero key):
    the max over the retained tokens of the mean over heads of the query-key
    cosine.  QuoKA article, Fig. 1(b) (query-key cosine filter, max pooling over
    queries) with the group's heads pooled first.
    Qbar: [H_kv, C, d]; K: [H_kv, T, d] -> [H_kv, T]."""
    H_kv, T, _ = K.shape
    S = np.zeros((H_kv, T), dtype=np.float64)
    for g in range(H_kv):
        Qs = Qbar[g, np.asarray(keep[g], dtype=np.int64)]
        kn = _norms(K[g])
        for j0 in range(0, T, KEY_BLOCK):
            j1 = min(T, j0 + KEY_BLOCK)
            S[g, j0:j1] = _safe_div((Qs @ K[g, j0:j1].T).max(axis=0), kn[j0:j1])
    return S


# ----------------------------------------------------------------------------- step 4

def top_b(S_g: np.ndarray, B: int) -> np.ndarray:
    """The min(B, T) highest-scoring key indices (ties -> lower index), ascending.
    QuoKA article, Fig. 1(a)-(b): keep the best-scoring keys of the cache."""
    T = S_g.shape[0]
    if B >= T:
        return np.arange(T, dtype=np.int64)
    order = np.lexsort((np.arange(T), -S_g))        # descending score, then index
    return np.sort(order[:B]).astype(np.int64)


# ----------------------------------------------------------------------------- step 6

def attend(Qc: np.ndarray, K_sel: Sequence[np.ndarray], V_sel: Sequence[np.ndarray],
           Kc: np.ndarray, Vc: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Dense softmax attention of every chunk query over the compacted prior keys
    (all visible) followed by the chunk's own keys under the causal mask.

    QuoKA article, Fig. 1(a) (the compacted cache is fed to a dense attention
    kernel); multi-query attention page, "Teknisk innsikt" (each query head uses
    its own query against the shared K/V of its group).
    Qc: [H_q, C, d]; K_sel[g], V_sel[g]: [n_g, d]; Kc, Vc: [H_kv, C, d] -> O [H_q, C, d].
    """
    H_q, C, d = Qc.shape
    H_kv = Kc.shape[0]
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.empty_like(Qc)
    causal = np.tril(np.ones((C, C), dtype=bool))
    for h in range(H_q):
        g = h // G
        n = K_sel[g].shape[0]
        keys = np.concatenate([K_sel[g], Kc[g]], axis=0)
        vals = np.concatenate([V_sel[g], Vc[g]], axis=0)
        z = scale * (Qc[h] @ keys.T)                         # [C, n + C]
        visible = np.concatenate([np.ones((C, n), dtype=bool), causal], axis=1)
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        O[h] = p @ vals
    return O


# ----------------------------------------------------------------------------- one chunk

def select(Qc: np.ndarray, K_prior: np.ndarray, n_q: int, B: int,
           keep: Optional[Sequence[np.ndarray]] = None, pooling: str = "head") -> Dict[str, object]:
    """Steps 1-4 for one chunk against the prior cache K_prior [H_kv, T, d].

    Returns keep (per query head, or per KV head with pooling="group"), S
    [H_kv, T] (None when T <= B) and idx (per KV head, ascending).  `keep` may
    be supplied to condition steps 2-4 on a given query sub-selection.
    """
    H_kv, T, _ = K_prior.shape
    if T <= B:
        return {"keep": None, "S": None, "idx": [np.arange(T, dtype=np.int64) for _ in range(H_kv)]}
    if pooling == "group":
        Qbar = pooled_queries(Qc, H_kv)
        if keep is None:
            keep = [query_keep(Qbar[g], n_q) for g in range(H_kv)]
        S = key_scores_group(Qbar, keep, K_prior)
    elif pooling == "head":
        if keep is None:
            keep = keep_all_heads(Qc, n_q)
        S = key_scores(Qc, keep, K_prior)
    else:
        raise ValueError(f"unknown pooling {pooling!r}")
    return {"keep": list(keep), "S": S, "idx": [top_b(S[g], B) for g in range(H_kv)]}


def prefill_chunk(Qc: np.ndarray, Kc: np.ndarray, Vc: np.ndarray,
                  K_prior: np.ndarray, V_prior: np.ndarray, n_q: int, B: int,
                  scale: Optional[float] = None, pooling: str = "head") -> Dict[str, object]:
    """Select over the prior cache, compact, attend (steps 1-6 of one chunk)."""
    sel = select(Qc, K_prior, n_q, B, pooling=pooling)
    idx = sel["idx"]
    K_sel = [K_prior[g, idx[g]] for g in range(K_prior.shape[0])]
    V_sel = [V_prior[g, idx[g]] for g in range(V_prior.shape[0])]
    sel["O"] = attend(Qc, K_sel, V_sel, Kc, Vc, scale)
    return sel


def prefill(chunks: Sequence[tuple], n_q: int, B: int, scale: Optional[float] = None,
            keep_trace: bool = False, pooling: str = "head") -> Dict[str, object]:
    """Whole-prompt chunked prefill: for chunk k (T = tokens so far) select over the
    cache, attend, then append the chunk's K/V (the cache grows by one chunk).

    QuoKA article, introduction (chunked prefill) and Fig. 1(a).
    chunks: sequence of (Q_c, K_c, V_c) fp64 arrays.  Returns O for every chunk
    and, when keep_trace, the per-chunk selection records.
    """
    Ks: List[np.ndarray] = []
    Vs: List[np.ndarray] = []
    outs, trace = [], []
    for Qc, Kc, Vc in chunks:
        H_kv, _, d = Kc.shape
        K_prior = np.concatenate(Ks, axis=1) if Ks else np.zeros((H_kv, 0, d))
        V_prior = np.concatenate(Vs, axis=1) if Vs else np.zeros((H_kv, 0, d))
        r = prefill_chunk(Qc, Kc, Vc, K_prior, V_prior, n_q, B, scale, pooling)
        outs.append(r["O"])
        if keep_trace:
            trace.append(r)
        Ks.append(Kc)
        Vs.append(Vc)
    return {"O": outs, "trace": trace}
