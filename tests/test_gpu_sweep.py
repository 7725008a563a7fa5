"""GPU parity over a seeded sweep of small random shapes: head counts, head
dim, element type, chunk length, ragged prior lengths, budget, kept queries,
contiguous or paged cache.  Each case runs kvsel_select and
kvsel_prefill_chunk through the C ABI and checks every sequence against the
CPU oracle with the rules of parity.py, the compacted lists bit for bit and
the cache append.  The sweep reaches launch shapes the named cases do not
(one-query scans beside multi-query ones, gathering and packed attention,
in-place lists, split scans, small and large problem counts)."""
import numpy as np
import pytest
import torch

import parity
from chunked_prefill_kv_amd import gen, runner
from chunked_prefill_kv_amd import kvsel as K
from oracle import quoka

pytestmark = pytest.mark.gpu

N_CASES = 24


def _cases():
    rng = np.random.default_rng([0x5EED, 9001])
    out = []
    for i in range(N_CASES):
        h_kv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8] + ([16] if h_kv == 1 else [])))
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        C = int(rng.choice([1, 3, 32, 64, 100, 128, 250, 300]))
        nb = int(rng.integers(1, 4))
        Ts = sorted(int(x) for x in rng.integers(0, 2001, size=nb))
        B = int(rng.integers(1, 1200))
        n_q = int(rng.integers(1, C + 20))
        bs = int(rng.choice([0, 0, 8, 16, 24]))
        out.append((i, h_kv, G, d, dtype, C, Ts, B, n_q, bs))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.load()


def _case_id(c):
    i, h_kv, G, d, dtype, C, Ts, B, n_q, bs = c
    return f"{i}-kv{h_kv}g{G}d{d}{dtype}-C{C}-T{'_'.join(map(str, Ts))}-B{B}-nq{n_q}-bs{bs}"


@pytest.mark.parametrize("case", CASES, ids=[_case_id(c) for c in CASES])
def test_random_shape_matches_oracle(case):
    i, h_kv, G, d, dtype, C, Ts, B, n_q, bs = case
    print(f"[case] sweep {_case_id(case)}", flush=True)
    base = gen.WORKLOADS["tiny_f32"] if dtype == "f32" else gen.WORKLOADS["llama8b_32k"]
    # room for every sequence's current chunk as a whole chunk of the generator
    wl = base.replace(L=(-(-max(Ts) // C) + 1) * C, C=C, H_q=h_kv * G, H_kv=h_kv, d=d, n_q=n_q, B=B)
    nb = len(Ts)
    store = np.float32 if dtype == "f32" else np.uint16
    kdt = K.KVSEL_F32 if dtype == "f32" else K.KVSEL_BF16
    # every sequence's prior tokens and current chunk from the workload's generator
    # (sequence s: chunk k covers positions [k*C, (k+1)*C); the prior rows are
    # the first T_s rows of the chunks before the current one)
    cur, logical = [], []
    for s, T in enumerate(Ts):
        k_cur = -(-T // C)
        chunks = [gen.chunk_inputs(wl, k, seq=100 * i + s) for k in range(k_cur)]
        kp = np.concatenate([c[1] for c in chunks], axis=1)[:, :T] if chunks else np.zeros((h_kv, 0, d), store)
        vp = np.concatenate([c[2] for c in chunks], axis=1)[:, :T] if chunks else np.zeros((h_kv, 0, d), store)
        logical.append((np.ascontiguousarray(kp), np.ascontiguousarray(vp)))
        cur.append(gen.chunk_inputs(wl, k_cur, seq=100 * i + s))
    dev = "cuda"
    cap = max(Ts) + C
    if bs == 0:
        kc = np.zeros((nb, h_kv, cap, d), dtype=store)
        vc = np.zeros_like(kc)
        for s, T in enumerate(Ts):
            kc[s, :, :T], vc[s, :, :T] = logical[s]
        k_d, v_d = runner.to_device(kc, dev), runner.to_device(vc, dev)
        cache = K.cache(k_d, v_d, cap)
        table = None
    else:
        nblk = [(T + C + bs - 1) // bs for T in Ts]
        perm = np.random.default_rng([0x5EED, 9002, i]).permutation(sum(nblk)).astype(np.int32)
        table = np.zeros((nb, max(nblk)), dtype=np.int32)
        pos = 0
        for s in range(nb):
            table[s, :nblk[s]] = perm[pos:pos + nblk[s]]
            pos += nblk[s]
        kpool = np.zeros((sum(nblk), h_kv, bs, d), dtype=store)
        vpool = np.zeros_like(kpool)
        for s, T in enumerate(Ts):
            for t in range(T):
                kpool[table[s, t // bs], :, t % bs] = logical[s][0][:, t]
                vpool[table[s, t // bs], :, t % bs] = logical[s][1][:, t]
        k_d, v_d = runner.to_device(kpool, dev), runner.to_device(vpool, dev)
        table_d = torch.tensor(table, dtype=torch.int32, device=dev)
        cache = K.cache(k_d, v_d, kpool.shape[0], bs, table_d)
    q = runner.to_device(np.stack([c[0] for c in cur]), dev)
    kn = runner.to_device(np.stack([c[1] for c in cur]), dev)
    vn = runner.to_device(np.stack([c[2] for c in cur]), dev)
    h = K.heads(h_kv * G, h_kv, d, kdt)
    p = K.Params(n_q, B)
    prior_d = torch.tensor(Ts, dtype=torch.int64, device=dev)     # kept alive: the batch holds its pointer
    b = K.batch(Ts, C, prior_d)
    ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
    nqp = min(n_q, C)
    idx = torch.full((nb, h_kv, B), -7, dtype=torch.int32, device=dev)
    keep = torch.full((nb, h_kv * G, nqp), -7, dtype=torch.int32, device=dev)
    S = torch.full((nb, h_kv, max(max(Ts), 1)), float("nan"), dtype=torch.float32, device=dev)
    K.kvsel_select(h, b, p, q, cache, idx, None, None, keep, S, ws)
    out = torch.empty(nb, h_kv * G, C, d, dtype=torch.float32, device=dev)
    idx2 = torch.full_like(idx, -7)
    K.kvsel_prefill_chunk(h, b, p, q, kn, vn, cache, out, idx2, ws)
    torch.cuda.synchronize()
    idx_all = idx.cpu().numpy()
    assert np.array_equal(idx_all, idx2.cpu().numpy()), "select and prefill chose different sets"
    parity.check_compaction(h, b, p, cache, ws, Ts, C, idx_all, logical, [(c[1], c[2]) for c in cur])
    # the chunk's rows appended, the prior rows untouched
    ka, va = runner.to_host_bits(k_d), runner.to_host_bits(v_d)
    for s, T in enumerate(Ts):
        for t in range(T + C):
            wk = cur[s][1][:, t - T] if t >= T else logical[s][0][:, t]
            wv = cur[s][2][:, t - T] if t >= T else logical[s][1][:, t]
            if bs == 0:
                gk, gv = ka[s, :, t], va[s, :, t]
            else:
                gk, gv = ka[table[s, t // bs], :, t % bs], va[table[s, t // bs], :, t % bs]
            assert np.array_equal(gk, wk) and np.array_equal(gv, wv), f"cache row {t} of sequence {s}"
    O = out.double().cpu().numpy()
    S_h, keep_h = S.cpu().numpy(), keep.cpu().numpy()
    for s, T in enumerate(Ts):
        Qc, Kn, Vn = (gen.to_f64(x) for x in cur[s])
        Kp, Vp = gen.to_f64(logical[s][0]), gen.to_f64(logical[s][1])
        idx_h = idx_all[s]
        if T > B:
            for hh in range(h_kv * G):
                parity.check_keep(Qc[hh], n_q, keep_h[s, hh])
            S_or = quoka.key_scores(Qc, [np.sort(keep_h[s, hh]) for hh in range(h_kv * G)], Kp)
            for g in range(h_kv):
                parity.check_close(S_h[s, g, :T], S_or[g], parity.S_TOL, f"S seq {s} head {g}")
                parity.check_idx(S_or[g], B, idx_h[g], S_h[s, g, :T])
        else:
            for g in range(h_kv):
                assert np.array_equal(idx_h[g, :T], np.arange(T)) and np.all(idx_h[g, T:] == -1)
        n = min(B, T)
        O_or = quoka.attend(Qc, [Kp[g, idx_h[g, :n]] for g in range(h_kv)],
                            [Vp[g, idx_h[g, :n]] for g in range(h_kv)], Kn, Vn)
        parity.check_close(O[s], O_or, parity.o_tol(dtype), f"O seq {s}")
