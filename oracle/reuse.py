"""CPU oracle for the cross-step reuse of selected keys and values in decode.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the bench's
CPU-baseline leg may import this module; it shares no code with the HIP path.

Source: SQD page ("rit.work", the paragraph on sparse attention): the top-k
selection scans the whole cache every step; the values of the selected
positions are kept in a cache of selected entries from one step to the next,
and only the misses are fetched (ahead of use).  The page gives no policy for
where a fetched entry goes or what happens to entries no longer selected.

Reading taken (the plainest one that makes every step's result the method's
result; listed in the design notes):

* The selected-entry cache of one (sequence, KV head) has B slots; slot s
  holds the cache position pos[s] (-1: empty) and that position's key and
  value rows.  Before a sequence's first step every slot is empty.
* A step selects n = min(B, T) positions idx (ascending), exactly as without
  reuse.  A slot s < n whose position is selected again keeps it: a hit (its
  rows are not fetched again).  Every other slot is free; slots s >= n end
  empty.
* The selected positions held by no hit slot are the misses.  In ascending
  position order they fill the free slots of [0, n) in ascending slot order,
  and their rows are fetched from the KV cache.
* Attention runs over slots [0, n) plus the step's own token.  Softmax
  attention does not depend on the order of its keys, so the output equals the
  output without reuse (the QuoKA article, Fig. 1(a): attention over the
  compacted cache).

Every function takes plain integer / fp64 arrays.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import quoka


def reuse_slots(prev_pos: np.ndarray, idx: np.ndarray) -> Dict[str, object]:
    """New slot contents after a step that selected `idx` (ascending, length n <= B).

    prev_pos: [B] int, the position each slot held after the previous step (-1 empty).
    Returns pos [B] (new contents), hit [B] bool (slot kept its position),
    miss_slots (the slots filled this step, ascending) and miss_pos (the
    positions fetched into them, ascending), hits and misses (counts).
    """
    prev_pos = np.asarray(prev_pos, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    B, n = prev_pos.shape[0], idx.shape[0]
    assert n <= B, "more selected positions than slots"
    slots = np.arange(B)
    hit = (slots < n) & (prev_pos >= 0) & np.isin(prev_pos, idx)
    held = np.isin(idx, prev_pos[hit])
    miss_pos = idx[~held]                                     # ascending, as idx is
    free = slots[(slots < n) & ~hit]                          # ascending
    assert free.shape[0] == miss_pos.shape[0]
    pos = np.full(B, -1, dtype=np.int64)
    pos[hit] = prev_pos[hit]
    pos[free] = miss_pos
    return {"pos": pos, "hit": hit, "miss_slots": free, "miss_pos": miss_pos,
            "hits": int(hit.sum()), "misses": int(miss_pos.shape[0])}


def decode_step(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, K_prior: np.ndarray, V_prior: np.ndarray,
                prev_pos: np.ndarray, n_q: int, B: int, idx: Optional[list] = None,
                scale: Optional[float] = None) -> Dict[str, object]:
    """One decode step of one sequence with the selected-entry cache.

    q [H_q, 1, d], k_new / v_new [H_kv, 1, d] (the step's own token), K_prior /
    V_prior [H_kv, T, d] (positions before it), prev_pos [H_kv, B].  The
    selection is quoka.select (or the given per-KV-head `idx`, to condition on
    another implementation's index sets); then reuse_slots per KV head and
    attention over the slot rows [0, n) plus the new token.
    Returns idx, pos [H_kv, B], hits / misses [H_kv] and O [H_q, 1, d].
    """
    H_kv = K_prior.shape[0]
    if idx is None:
        idx = quoka.select(q, K_prior, n_q, B)["idx"]
    pos, hits, misses, k_sel, v_sel = [], [], [], [], []
    for g in range(H_kv):
        r = reuse_slots(prev_pos[g], idx[g])
        n = len(idx[g])
        pos.append(r["pos"])
        hits.append(r["hits"])
        misses.append(r["misses"])
        k_sel.append(K_prior[g, r["pos"][:n]])
        v_sel.append(V_prior[g, r["pos"][:n]])
    O = quoka.attend(q, k_sel, v_sel, k_new, v_new, scale)
    return {"idx": idx, "pos": np.stack(pos), "hits": np.array(hits), "misses": np.array(misses), "O": O}
