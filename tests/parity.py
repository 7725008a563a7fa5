"""Parity checks shared by the GPU tests: compare what the HIP path returned for
one chunk with the CPU oracle on the same inputs.

Rules (tolerances written here, derived in the design notes):
  keep   kept query sets equal, except queries whose oracle cosine lies within
         KEEP_BAND of the N_q-th smallest cosine;
  S      |S_gpu - S_oracle| <= S_TOL, the oracle conditioned on the GPU's keep;
  idx    (a) the GPU's idx is exactly the top-B of the GPU's own fp32 scores
         (the integer decision taken in the kernel's precision), and
         (b) it equals the oracle's set except positions whose oracle score
         lies within IDX_BAND of the B-th score; sets have equal size;
  gather bit-exact, both the kvsel_select gather and the compacted lists
         kvsel_prefill_chunk hands to its attention;
  O      max |O_gpu - O_oracle| <= 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs),
         given the same index set.
"""
from __future__ import annotations

import numpy as np

from oracle import quoka

KEEP_BAND = 1e-5
IDX_BAND = 1e-4
S_TOL = 1e-5


def o_tol(dtype: str) -> float:
    return 1e-4 if dtype == "f32" else 2e-2


def check_keep(Qh: np.ndarray, n_q: int, keep_gpu: np.ndarray) -> None:
    C = Qh.shape[0]
    n = min(n_q, C)
    ref = quoka.query_keep(Qh, n_q)
    got = np.sort(keep_gpu[:n])
    assert len(set(got.tolist())) == n and got.min() >= 0 and got.max() < C
    if np.array_equal(got, ref):
        return
    c = quoka.query_cosines(Qh)
    thr = np.sort(c)[n - 1]
    band = np.abs(c - thr) <= KEEP_BAND
    a = set(got.tolist()) - set(np.nonzero(band)[0].tolist())
    b = set(ref.tolist()) - set(np.nonzero(band)[0].tolist())
    assert a == b, f"keep differs outside the {KEEP_BAND} band: {sorted(a ^ b)[:10]}"


def check_idx(S_oracle: np.ndarray, B: int, idx_gpu: np.ndarray, S_gpu: np.ndarray | None) -> None:
    T = S_oracle.shape[0]
    n = min(B, T)
    got = idx_gpu[:n]
    assert np.all(idx_gpu[n:] == -1), "idx must be -1 past min(B, T)"
    assert np.all(np.diff(got) > 0) and got.min(initial=0) >= 0 and got.max(initial=-1) < T, "idx ascending, in range"
    if S_gpu is not None:                       # same decision in the kernel's precision: exact
        own = quoka.top_b(S_gpu.astype(np.float64), B)
        assert np.array_equal(got, own), "idx is not the exact top-B of the GPU's own scores"
    ref = quoka.top_b(S_oracle, B)
    if np.array_equal(got, ref):
        return
    thr = np.sort(S_oracle)[::-1][n - 1]
    band = set(np.nonzero(np.abs(S_oracle - thr) <= IDX_BAND)[0].tolist())
    a, b = set(got.tolist()) - band, set(ref.tolist()) - band
    assert a == b, f"idx differs outside the {IDX_BAND} band at {sorted(a ^ b)[:10]}"


def check_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
    return err


def check_compaction(h, b, p, cache, ws, Ts, C, idx, prior_kv, chunk_kv, heads=None):
    """Rule 3 on the timed path: after kvsel_prefill_chunk, the compacted key
    list (and the value list, transposed for bf16) left in the workspace holds,
    bit for bit, the prior rows at idx, then the chunk's rows, then zeros.
    prior_kv[s] / chunk_kv[s]: (K, V) bit arrays [H_kv][rows][d] of sequence s.
    Returns False when the call builds no lists (gathering attention)."""
    from chunked_prefill_kv_amd import kvsel as K
    v = K.compacted_view(h, b, p, cache)
    if v is None:
        return False
    nb, H_kv, d, slots = len(Ts), h.h_kv, h.d, v["slots"]
    store = np.uint16 if h.dtype == K.KVSEL_BF16 else np.uint32
    esz = np.dtype(store).itemsize
    n_el = nb * H_kv * slots * d
    raw = ws.cpu().numpy()
    kl = raw[v["k_offset"]:v["k_offset"] + n_el * esz].view(store).reshape(nb, H_kv, slots, d)
    vl = raw[v["v_offset"]:v["v_offset"] + n_el * esz].view(store)
    vl = vl.reshape(nb, H_kv, d, slots).transpose(0, 1, 3, 2) if v["v_transposed"] else vl.reshape(nb, H_kv, slots, d)
    B = p.budget
    for s, T in enumerate(Ts):
        n = min(B, T)
        for g in (range(H_kv) if heads is None else heads):
            for lst, pk, ck, what in ((kl, prior_kv[s][0], chunk_kv[s][0], "K"), (vl, prior_kv[s][1], chunk_kv[s][1], "V")):
                want = np.zeros((slots, d), dtype=store)
                if n:
                    want[:n] = pk[g, idx[s, g, :n]].view(store)
                want[n:n + C] = ck[g].view(store)
                got = lst[s, g]
                bad = np.nonzero(np.any(got != want, axis=1))[0]
                assert bad.size == 0, f"compacted {what} seq {s} head {g}: {bad.size} slots differ, first {bad[:5]} (n={n}, C={C})"
    return True
