"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Small workloads span several tiles, ragged tails and the
degenerate cases; the full-size workloads are checked on sampled KV heads /
sequences in the launch configuration the bench times."""
import numpy as np
import pytest
import torch

import parity
from chunked_prefill_kv_amd import gen, runner
from chunked_prefill_kv_amd import kvsel as K
from oracle import quoka

pytestmark = pytest.mark.gpu

LLAMA = gen.WORKLOADS["llama8b_32k"]
TINY = gen.WORKLOADS["tiny_f32"]
SMALL = {
    "tiny_f32_full": TINY,                                                               # the fp32 workload, whole
    "f32_d128": TINY.replace(L=600, C=150, d=128, n_q=20, B=200),
    "bf16_gqa_ragged": LLAMA.replace(L=3000, C=700, H_q=8, H_kv=2, n_q=100, B=900),      # ragged chunk, N_q, B
    "bf16_mqa": gen.WORKLOADS["mqa_64k"].replace(L=2600, C=512, n_q=40, B=700),          # H_kv = 1, G = 16
    "bf16_g8_needles": gen.WORKLOADS["gqa_128k"].replace(L=6000, C=1000, H_q=16, H_kv=2, n_q=64, B=1100, needles=8),
    "bf16_d64": LLAMA.replace(L=2048, C=384, H_q=16, H_kv=2, d=64, n_q=64, B=500),
    "bf16_nq1": LLAMA.replace(L=1500, C=300, H_q=8, H_kv=2, n_q=1, B=400),               # one kept query per head
    "bf16_budget1": LLAMA.replace(L=1024, C=256, H_q=4, H_kv=2, n_q=8, B=1),
    "bf16_keep_all_queries": LLAMA.replace(L=1200, C=100, H_q=4, H_kv=1, n_q=128, B=150),
    "f32_keep_all_queries": TINY.replace(L=512, C=64, n_q=100, B=100),                  # N_q >= C, fp32 rows
    "bf16_dense": LLAMA.replace(L=1000, C=250, H_q=8, H_kv=2, n_q=16, B=1000),           # B >= T always
    "bf16_short_chunks": LLAMA.replace(L=600, C=25, H_q=8, H_kv=2, n_q=10, B=150),      # G*C <= 128: gathering attention
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.load()


def _f64(chunks):
    return [tuple(gen.to_f64(x) for x in c) for c in chunks]


def _prior(c64, k):
    H_kv, d = c64[0][1].shape[0], c64[0][1].shape[2]
    if k == 0:
        return np.zeros((H_kv, 0, d)), np.zeros((H_kv, 0, d))
    return (np.concatenate([c[1] for c in c64[:k]], axis=1), np.concatenate([c[2] for c in c64[:k]], axis=1))


def _bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32) if x.dtype == np.float32 else x


def check_chunk(r: runner.PromptRunner, k: int, chunks, c64, heads=None, pooling="head", otol=None):
    """select (with debug outputs) then prefill_chunk for chunk k; every rule on KV heads `heads`.
    pooling="group": the kept tokens are per KV head and are checked on the
    oracle's pooled rows; the scores against the oracle's group-pooled scan.
    otol: the output tolerance (default: that of the input type)."""
    wl = r.wl
    T, C = r.starts[k], r.lens[k]
    Qc, Kc, Vc = c64[k]
    Kp, Vp = _prior(c64, k)
    dev = r.device
    nqp = min(wl.n_q, C)
    idx = torch.full((1, wl.H_kv, wl.B), -7, dtype=torch.int32, device=dev)
    ks = torch.empty(1, wl.H_kv, wl.B, wl.d, dtype=r.dt, device=dev)
    vs = torch.empty_like(ks)
    keep_rows = wl.H_kv if pooling == "group" and C > 1 else wl.H_q
    keep = torch.full((1, keep_rows, nqp), -7, dtype=torch.int32, device=dev)
    S = torch.full((1, wl.H_kv, max(T, 1)), float("nan"), dtype=torch.float32, device=dev)
    K.kvsel_select(r.h, r.batches[k], r.p, r.chunks[k][0], r.cache, idx, ks, vs, keep, S, r.ws)
    r.run_chunk(k)
    torch.cuda.synchronize()
    idx_h = idx[0].cpu().numpy()
    assert np.array_equal(r.idx[k][0].cpu().numpy(), idx_h), "prefill_chunk and select disagree on idx"
    # the compacted lists the attention consumed, bit for bit (rule 3 on the prefill path)
    pk = (np.concatenate([c[1] for c in chunks[:k]], axis=1), np.concatenate([c[2] for c in chunks[:k]], axis=1)) \
        if k else (None, None)
    parity.check_compaction(r.h, r.batches[k], r.p, r.cache, r.ws, [T], C, idx_h[None], [pk], [(chunks[k][1], chunks[k][2])],
                     heads)
    G = wl.G
    heads = range(wl.H_kv) if heads is None else heads
    qh = [h for g in heads for h in range(g * G, (g + 1) * G)]
    if T > wl.B and keep_rows == wl.H_kv:
        keep_h = keep[0].cpu().numpy()
        Qbar = quoka.pooled_queries(Qc, wl.H_kv)
        S_h = S[0].cpu().numpy()
        for g in heads:
            parity.check_keep(Qbar[g], wl.n_q, keep_h[g])
            S_or = quoka.key_scores_group(Qbar[g:g + 1], [np.sort(keep_h[g])], Kp[g:g + 1])[0]
            parity.check_close(S_h[g, :T], S_or, parity.S_TOL, f"S chunk {k} head {g}")
            parity.check_idx(S_or, wl.B, idx_h[g], S_h[g, :T])
    elif T > wl.B:
        keep_h = keep[0].cpu().numpy()
        for h in qh:
            parity.check_keep(Qc[h], wl.n_q, keep_h[h])
        keep_list = [np.sort(keep_h[h]) for h in range(wl.H_q)]
        S_h = S[0].cpu().numpy()
        for g in heads:
            S_or = quoka.key_scores(Qc[g * G:(g + 1) * G], keep_list[g * G:(g + 1) * G], Kp[g:g + 1])[0]
            parity.check_close(S_h[g, :T], S_or, parity.S_TOL, f"S chunk {k} head {g}")
            parity.check_idx(S_or, wl.B, idx_h[g], S_h[g, :T])
    else:
        for g in heads:
            assert np.array_equal(idx_h[g, :T], np.arange(T)) and np.all(idx_h[g, T:] == -1)
    # gather: bit-exact copies of the cache rows
    kbits = [_bits(np.concatenate([c[1] for c in chunks[:k]], axis=1)) if k else None]
    vbits = [_bits(np.concatenate([c[2] for c in chunks[:k]], axis=1)) if k else None]
    ks_h, vs_h = _bits(runner.to_host_bits(ks[0])), _bits(runner.to_host_bits(vs[0]))
    n = min(wl.B, T)
    for g in heads:
        if n:
            assert np.array_equal(ks_h[g, :n], kbits[0][g, idx_h[g, :n]]), "gathered K not bit-exact"
            assert np.array_equal(vs_h[g, :n], vbits[0][g, idx_h[g, :n]]), "gathered V not bit-exact"
    # attention given the GPU's index set
    sel_k = [Kp[g, idx_h[g, :n]] for g in range(wl.H_kv)]
    sel_v = [Vp[g, idx_h[g, :n]] for g in range(wl.H_kv)]
    Og = r.outs[k][0].double().cpu().numpy()
    for g in heads:
        O_or = quoka.attend(Qc[g * G:(g + 1) * G], sel_k[g:g + 1], sel_v[g:g + 1], Kc[g:g + 1], Vc[g:g + 1])
        parity.check_close(Og[g * G:(g + 1) * G], O_or, otol or parity.o_tol(wl.dtype), f"O chunk {k} head {g}")
    return idx_h


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_matches_oracle(name):
    wl = SMALL[name]
    print(f"[case] prefill {name} {wl}", flush=True)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    if name == "bf16_gqa_ragged":                       # a zero key: cosine 0 by convention
        chunks[0][1][1, 5] = 0
    c64 = _f64(chunks)
    r = runner.PromptRunner(wl, out_dtype=torch.float32)
    r.load(chunks, keep_idx=True)
    for k in range(wl.n_chunks):
        check_chunk(r, k, chunks, c64)


GROUP = ["bf16_gqa_ragged", "bf16_mqa", "f32_d128", "tiny_f32_full", "bf16_d64", "bf16_nq1", "bf16_keep_all_queries",
         "bf16_g1"]


@pytest.mark.parametrize("name", GROUP)
def test_group_pooled_prefill_matches_oracle(name):
    """The group-first pooling order (KVSEL_POOL_GROUP) against the oracle's
    pooling="group" on every chunk: kept tokens of the pooled rows, scores
    (bf16 caches score the pooled rows as [hi | lo] bf16 pairs), index sets,
    gather and attention."""
    wl = SMALL[name] if name in SMALL else LLAMA.replace(L=1500, C=300, H_q=2, H_kv=2, n_q=40, B=400)
    print(f"[case] group-pooled prefill {name} {wl}", flush=True)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    if name == "bf16_gqa_ragged":                       # a zero key and a zero query row
        chunks[0][1][1, 5] = 0
        chunks[3][0][2, 17] = 0
    c64 = _f64(chunks)
    r = runner.PromptRunner(wl, out_dtype=torch.float32, pooling=K.KVSEL_POOL_GROUP)
    r.load(chunks, keep_idx=True)
    for k in range(wl.n_chunks):
        check_chunk(r, k, chunks, c64, pooling="group")


# bf16 output: d = 64 packed (key-split merge), in place (chunks with T <= B)
# and gathering (G*C <= 128) attention; the fp32 attention at d = 128 and 64
BF16_OUT = {
    "bf16_d64": SMALL["bf16_d64"],
    "bf16_d64_short": LLAMA.replace(L=600, C=16, H_q=16, H_kv=2, d=64, n_q=8, B=150),
    "f32_d128": SMALL["f32_d128"],
    "tiny_f32_full": TINY,
}


@pytest.mark.parametrize("name", list(BF16_OUT))
def test_prefill_bf16_output_matches_oracle(name):
    """Every chunk of the prompt with the output written as bf16: the same
    rules, the output within 2e-2 (its bf16 rounding included)."""
    wl = BF16_OUT[name]
    print(f"[case] prefill, bf16 output, {name} {wl}", flush=True)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    c64 = _f64(chunks)
    r = runner.PromptRunner(wl, out_dtype=torch.bfloat16)
    r.load(chunks, keep_idx=True)
    for k in range(wl.n_chunks):
        check_chunk(r, k, chunks, c64, otol=2e-2)


# selection only, in launch forms the prompts above do not reach:
#   statistics in 128-row blocks (at least 1024 workgroups of them);
#   the d = 64 scan with three and four 32-key blocks per wave (one round of
#   workgroups with 8 KV heads at T = 20000 and T = 30000);
#   the query top-k over a chunk longer than its on-chip key store (30720)
SELECT_FORMS = {
    "rows128_f32_d128": dict(dtype="f32", H_q=32, H_kv=8, d=128, C=4096, T=600, B=300, n_q=64),
    "rows128_f32_d64": dict(dtype="f32", H_q=32, H_kv=8, d=64, C=4096, T=600, B=300, n_q=64),
    "rows128_bf16_d64": dict(dtype="bf16", H_q=32, H_kv=8, d=64, C=4096, T=600, B=300, n_q=64),
    "scan_d64_nb3": dict(dtype="bf16", H_q=16, H_kv=8, d=64, C=64, T=20000, B=1024, n_q=16),
    "scan_d64_nb4": dict(dtype="bf16", H_q=16, H_kv=8, d=64, C=64, T=30000, B=1024, n_q=16),
    "keep_long_chunk": dict(dtype="bf16", H_q=1, H_kv=1, d=64, C=32768, T=200, B=100, n_q=64),
}


@pytest.mark.parametrize("name", list(SELECT_FORMS))
def test_select_forms_match_oracle(name):
    """kvsel_select on seeded inputs (queries with a shared direction, so the
    cosines to the mean spread): kept queries, scores and index sets against
    the oracle."""
    cfg = SELECT_FORMS[name]
    H_q, H_kv, d, C, T, B, n_q = (cfg[x] for x in ("H_q", "H_kv", "d", "C", "T", "B", "n_q"))
    G = H_q // H_kv
    print(f"[case] select {name} {cfg}", flush=True)
    rng = np.random.default_rng([0x5EED, 77, sum(map(ord, name))])
    shared = rng.standard_normal(d)
    qf = (0.6 * rng.standard_normal((H_q, C, d)) + shared).astype(np.float32)
    kf = (0.5 * rng.standard_normal((H_kv, T, d)) + 0.3 * shared).astype(np.float32)
    if cfg["dtype"] == "bf16":
        q, kc = gen.f32_to_bf16_bits(qf), gen.f32_to_bf16_bits(kf)
        kdt = K.KVSEL_BF16
    else:
        q, kc = qf, kf
        kdt = K.KVSEL_F32
    dev = "cuda"
    kd = runner.to_device(kc[None], dev)
    vd = torch.zeros_like(kd)
    h = K.heads(H_q, H_kv, d, kdt)
    p = K.Params(n_q, B)
    prior = torch.tensor([T], dtype=torch.int64, device=dev)
    b = K.batch([T], C, prior)
    cache = K.cache(kd, vd, T)
    ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
    nqp = min(n_q, C)
    idx = torch.full((1, H_kv, B), -7, dtype=torch.int32, device=dev)
    keep = torch.full((1, H_q, nqp), -7, dtype=torch.int32, device=dev)
    S = torch.full((1, H_kv, T), float("nan"), dtype=torch.float32, device=dev)
    K.kvsel_select(h, b, p, runner.to_device(q[None], dev), cache, idx, None, None, keep, S, ws)
    torch.cuda.synchronize()
    Q64, K64 = gen.to_f64(q), gen.to_f64(kc)
    keep_h, S_h, idx_h = keep[0].cpu().numpy(), S[0].cpu().numpy(), idx[0].cpu().numpy()
    for hh in range(H_q):
        parity.check_keep(Q64[hh], n_q, keep_h[hh])
    keep_list = [np.sort(keep_h[hh]) for hh in range(H_q)]
    for g in range(H_kv):
        S_or = quoka.key_scores(Q64[g * G:(g + 1) * G], keep_list[g * G:(g + 1) * G], K64[g:g + 1])[0]
        parity.check_close(S_h[g], S_or, parity.S_TOL, f"S head {g}")
        parity.check_idx(S_or, B, idx_h[g], S_h[g])


def test_needles_are_recalled():
    """Planted keys aligned with one chunk query (cos 0.9) are kept when that chunk is processed."""
    wl = SMALL["bf16_g8_needles"]
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    r = runner.PromptRunner(wl)
    r.load(chunks, keep_idx=True)
    r.run()
    torch.cuda.synchronize()
    hit = 0
    for nd in gen.needles(wl):
        hit += int(nd.pos in set(r.idx[nd.chunk][0, nd.head // wl.G].cpu().numpy().tolist()))
    print(f"needle recall {hit}/{len(gen.needles(wl))}")
    assert hit >= len(gen.needles(wl)) // 2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sparse_attn_given_oracle_set(dtype):
    """Rule 2: attention over the oracle's own compacted set, including ragged
    per-sequence counts and an empty set."""
    wl = (LLAMA.replace(L=2100, C=700, H_q=8, H_kv=2, n_q=100, B=900) if dtype == "bf16"
          else TINY.replace(L=512, C=128, n_q=16, B=200))
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    c64 = _f64(chunks)
    k = wl.n_chunks - 1
    Qc, Kc, Vc = c64[k]
    Kp, Vp = _prior(c64, k)
    sel = quoka.select(Qc, Kp, wl.n_q, wl.B)
    idx = sel["idx"]
    nmax = wl.B + 37
    counts = [len(idx[0]), 0, 13]
    bsz = len(counts)
    store = np.uint16 if dtype == "bf16" else np.float32
    ksel = np.zeros((bsz, wl.H_kv, nmax, wl.d), dtype=store)
    vsel = np.zeros_like(ksel)
    kbits = np.concatenate([c[1] for c in chunks[:k]], axis=1)
    vbits = np.concatenate([c[2] for c in chunks[:k]], axis=1)
    for b, n in enumerate(counts):
        for g in range(wl.H_kv):
            ksel[b, g, :n] = kbits[g, idx[g][:n]]
            vsel[b, g, :n] = vbits[g, idx[g][:n]]
    dev = "cuda"
    tq = runner.to_device(np.stack([chunks[k][0]] * bsz), dev)
    tkc = runner.to_device(np.stack([chunks[k][1]] * bsz), dev)
    tvc = runner.to_device(np.stack([chunks[k][2]] * bsz), dev)
    tks, tvs = runner.to_device(ksel, dev), runner.to_device(vsel, dev)
    nsel = torch.tensor(counts, dtype=torch.int32, device=dev)
    h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16 if dtype == "bf16" else K.KVSEL_F32)
    bt = K.batch([0] * bsz, gen.chunk_lengths(wl)[k], None)
    ws = torch.empty(K.sparse_attn_workspace_size(h, bt, nmax), dtype=torch.uint8, device=dev)
    out = torch.empty(bsz, wl.H_q, bt.chunk_len, wl.d, dtype=torch.float32, device=dev)
    K.kvsel_sparse_attn(h, bt, tq, tks, tvs, nsel, nmax, tkc, tvc, out, ws)
    torch.cuda.synchronize()
    O = out.double().cpu().numpy()
    for b, n in enumerate(counts):
        ref = quoka.attend(Qc, [Kp[g, idx[g][:n]] for g in range(wl.H_kv)],
                           [Vp[g, idx[g][:n]] for g in range(wl.H_kv)], Kc, Vc)
        parity.check_close(O[b], ref, parity.o_tol(dtype), f"sparse_attn seq {b} n_sel {n}")


def test_decode_group_pooling_single_token():
    """With one chunk token the group-first order scores the same as the
    per-head order (max over one token); the library then takes the per-head
    path.  Checked against the oracle's group-pooled scores."""
    wl = gen.WORKLOADS["decode_paged"].replace(batch=4, decode_len_lo=600, decode_len_hi=2000, B=500)
    print("[case] decode group pooling", flush=True)
    di = gen.decode_inputs(wl)
    dr = runner.DecodeRunner(wl, di, out_dtype=torch.float32, pooling=K.KVSEL_POOL_GROUP)
    T_max = int(di.prior_len.max())
    S = torch.full((wl.batch, wl.H_kv, T_max), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((wl.batch, wl.H_kv, wl.B), -7, dtype=torch.int32, device="cuda")
    K.kvsel_select(dr.h, dr.b, dr.p, dr.q, dr.cache, idx, None, None, None, S, dr.ws)
    torch.cuda.synchronize()
    S_h, idx_h = S.cpu().numpy(), idx.cpu().numpy()
    for b in range(wl.batch):
        T = int(di.prior_len[b])
        if T <= wl.B:
            continue
        kp, _ = di.logical_kv(b, wl.block_size)
        Kp = gen.to_f64(kp)
        Qbar = quoka.pooled_queries(gen.to_f64(di.q[b]), wl.H_kv)
        S_or = quoka.key_scores_group(Qbar, [np.array([0])] * wl.H_kv, Kp)
        for g in range(wl.H_kv):
            parity.check_close(S_h[b, g, :T], S_or[g], parity.S_TOL, f"S seq {b} head {g}")
            parity.check_idx(S_or[g], wl.B, idx_h[b, g], S_h[b, g, :T])


@pytest.mark.parametrize("variant", ["gqa", "mqa_g32", "gqa_block8", "gqa_block24", "g16_d64", "many_seqs"])
def test_decode_paged_matches_oracle(variant):
    """Ragged batch, chunk of 1, paged cache with a shuffled block table; some
    sequences are shorter than the budget (no selection).  Blocks of 8 and 24
    rows put a block boundary inside a 16-key group of the one-query scan; 16
    heads per KV head fill its MFMA rows, with d = 64.  300 sequences are more
    than the one-query scan lists in its launch arguments (its grid then spans
    every sequence's tiles up to the longest)."""
    base = gen.WORKLOADS["decode_paged"]
    wl = {"gqa": base.replace(batch=6, decode_len_lo=300, decode_len_hi=2500, B=512),
          "mqa_g32": base.replace(batch=3, decode_len_lo=700, decode_len_hi=1800, H_q=32, H_kv=1, B=400),
          "gqa_block8": base.replace(batch=4, decode_len_lo=300, decode_len_hi=2100, B=512, block_size=8),
          "gqa_block24": base.replace(batch=4, decode_len_lo=300, decode_len_hi=2100, B=512, block_size=24),
          "g16_d64": base.replace(batch=4, decode_len_lo=300, decode_len_hi=2100, B=512, H_q=32, H_kv=2, d=64),
          "many_seqs": base.replace(batch=300, decode_len_lo=60, decode_len_hi=700, B=128, H_q=8, H_kv=2)}[variant]
    print(f"[case] decode {variant}", flush=True)
    di = gen.decode_inputs(wl)
    dr = runner.DecodeRunner(wl, di, out_dtype=torch.float32)
    T_max = int(di.prior_len.max())
    S = torch.full((wl.batch, wl.H_kv, T_max), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((wl.batch, wl.H_kv, wl.B), -7, dtype=torch.int32, device="cuda")
    K.kvsel_select(dr.h, dr.b, dr.p, dr.q, dr.cache, idx, None, None, None, S, dr.ws)
    dr.run()
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), dr.idx.cpu().numpy())
    O = dr.out.double().cpu().numpy()
    S_h, idx_h = S.cpu().numpy(), dr.idx.cpu().numpy()
    pool_k = runner.to_host_bits(dr.k_pool)
    G = wl.G
    for b in range(wl.batch):
        T = int(di.prior_len[b])
        kp, vp = di.logical_kv(b, wl.block_size)
        Kp, Vp = gen.to_f64(kp), gen.to_f64(vp)
        Qc = gen.to_f64(di.q[b])
        if T > wl.B:
            S_or = quoka.key_scores(Qc, [np.array([0])] * wl.H_q, Kp)
            for g in range(wl.H_kv):
                parity.check_close(S_h[b, g, :T], S_or[g], parity.S_TOL, f"S seq {b} head {g}")
                parity.check_idx(S_or[g], wl.B, idx_h[b, g], S_h[b, g, :T])
        n = min(T, wl.B)
        ref = quoka.attend(Qc, [Kp[g, idx_h[b, g, :n]] for g in range(wl.H_kv)],
                           [Vp[g, idx_h[b, g, :n]] for g in range(wl.H_kv)],
                           gen.to_f64(di.k_new[b]), gen.to_f64(di.v_new[b]))
        parity.check_close(O[b], ref, parity.o_tol(wl.dtype), f"O seq {b}")
        # the new token's K landed in its paged slot
        blk = di.block_table[b, T // wl.block_size]
        assert np.array_equal(pool_k[blk, :, T % wl.block_size], di.k_new[b, :, 0])


def test_values_all_one_give_one():
    """Softmax rows sum to one on the GPU too: V == 1 gives O == 1 (bf16 P rounding only)."""
    wl = LLAMA.replace(L=1536, C=512, H_q=8, H_kv=2, n_q=64, B=600)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    one = gen.f32_to_bf16_bits(np.ones(1, dtype=np.float32))[0]
    chunks = [(q, k, np.full_like(v, one)) for q, k, v in chunks]
    r = runner.PromptRunner(wl, out_dtype=torch.float32)
    r.load(chunks)
    r.run()
    torch.cuda.synchronize()
    for o in r.outs:
        assert float((o - 1).abs().max()) < 4e-3


def test_bitwise_deterministic():
    wl = LLAMA.replace(L=2048, C=512, H_q=8, H_kv=2, n_q=64, B=700)
    r = runner.PromptRunner(wl)
    r.load(keep_idx=True)
    r.run()
    a = [o.clone() for o in r.outs] + [i.clone() for i in r.idx]
    r.reset()
    r.run()
    b = [o.clone() for o in r.outs] + [i.clone() for i in r.idx]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("C,Ts,B", [
    (200, [0, 400, 1600], 600),        # packed attention (G*C = 800): no prior, T <= B, selection
    (30, [0, 60, 300], 90),            # gathering attention (G*C = 120)
    (200, [600, 800], 600),            # T = B exactly (everything kept), T = B + one chunk
    (30, [90, 120, 150], 90),          # the same edge with the gathering attention
    # 8 sequences x 2 KV heads x 32 row blocks of 128 rows: one round of two
    # 4-wave workgroups per CU on 256 CUs, the heaviest row blocks paired with
    # the lightest on each CU, prior lists of 0, 1024 and 1500 keys
    (1024, [0, 1024, 2048, 3072, 2048, 3072, 1024, 3072], 1500),
])
def test_batched_prefill_ragged(C, Ts, B):
    """Several sequences in one kvsel_prefill_chunk call, each with its own
    prior length (an empty cache, T <= B, T > B): every sequence against the
    oracle on its own, and its chunk appended to the cache bit for bit."""
    wl = LLAMA.replace(L=max(Ts) + C, C=C, H_q=8, H_kv=2, n_q=24, B=B)
    print(f"[case] batched prefill C={C} T={Ts}", flush=True)
    nb, cap = len(Ts), max(Ts) + C
    cur = [gen.chunk_inputs(wl, T // C, seq=s) for s, T in enumerate(Ts)]
    prior = [[gen.chunk_inputs(wl, k, seq=s) for k in range(T // C)] for s, T in enumerate(Ts)]
    kc = np.zeros((nb, wl.H_kv, cap, wl.d), dtype=np.uint16)
    vc = np.zeros_like(kc)
    for s, T in enumerate(Ts):
        if T:
            kc[s, :, :T] = np.concatenate([c[1] for c in prior[s]], axis=1)
            vc[s, :, :T] = np.concatenate([c[2] for c in prior[s]], axis=1)
    dev = "cuda"
    kc_d, vc_d = runner.to_device(kc, dev), runner.to_device(vc, dev)
    q = runner.to_device(np.stack([c[0] for c in cur]), dev)
    kn = runner.to_device(np.stack([c[1] for c in cur]), dev)
    vn = runner.to_device(np.stack([c[2] for c in cur]), dev)
    h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16)
    p = K.Params(wl.n_q, wl.B)
    prior_d = torch.tensor(Ts, dtype=torch.int64, device=dev)
    b = K.batch(Ts, C, prior_d)
    cache = K.cache(kc_d, vc_d, cap)
    ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
    nqp = min(wl.n_q, C)
    idx = torch.full((nb, wl.H_kv, B), -7, dtype=torch.int32, device=dev)
    keep = torch.full((nb, wl.H_q, nqp), -7, dtype=torch.int32, device=dev)
    S = torch.full((nb, wl.H_kv, max(Ts)), float("nan"), dtype=torch.float32, device=dev)
    K.kvsel_select(h, b, p, q, cache, idx, None, None, keep, S, ws)
    out = torch.empty(nb, wl.H_q, C, wl.d, dtype=torch.float32, device=dev)
    idx2 = torch.full_like(idx, -7)
    K.kvsel_prefill_chunk(h, b, p, q, kn, vn, cache, out, idx2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx2.cpu().numpy())
    parity.check_compaction(h, b, p, cache, ws, Ts, C, idx2.cpu().numpy(), [(kc[s, :, :T], vc[s, :, :T]) for s, T in enumerate(Ts)],
                     [(c[1], c[2]) for c in cur])
    kc_after, vc_after = runner.to_host_bits(kc_d), runner.to_host_bits(vc_d)
    O = out.double().cpu().numpy()
    G = wl.G
    for s, T in enumerate(Ts):
        assert np.array_equal(kc_after[s, :, T:T + C], cur[s][1]) and np.array_equal(vc_after[s, :, T:T + C], cur[s][2])
        assert np.array_equal(kc_after[s, :, :T], kc[s, :, :T]), "prior rows must stay untouched"
        Qc, Kn, Vn = (gen.to_f64(x) for x in cur[s])
        Kp, Vp = gen.to_f64(kc[s, :, :T]), gen.to_f64(vc[s, :, :T])
        idx_h = idx[s].cpu().numpy()
        if T > B:
            keep_h = keep[s].cpu().numpy()
            for hh in range(wl.H_q):
                parity.check_keep(Qc[hh], wl.n_q, keep_h[hh])
            S_or = quoka.key_scores(Qc, [np.sort(keep_h[hh]) for hh in range(wl.H_q)], Kp)
            for g in range(wl.H_kv):
                parity.check_close(S[s, g, :T].cpu().numpy(), S_or[g], parity.S_TOL, f"S seq {s} head {g}")
                parity.check_idx(S_or[g], B, idx_h[g], S[s, g, :T].cpu().numpy())
        else:
            for g in range(wl.H_kv):
                assert np.array_equal(idx_h[g, :T], np.arange(T)) and np.all(idx_h[g, T:] == -1)
        n = min(B, T)
        O_or = quoka.attend(Qc, [Kp[g, idx_h[g, :n]] for g in range(wl.H_kv)],
                            [Vp[g, idx_h[g, :n]] for g in range(wl.H_kv)], Kn, Vn)
        parity.check_close(O[s], O_or, parity.o_tol(wl.dtype), f"O seq {s}")


@pytest.mark.parametrize("C,Ts,B,bs", [
    (200, [0, 400, 1600], 600, 16),    # packed attention over a paged cache
    (30, [60, 300, 990], 90, 16),      # gathering attention: rows through the block table
    (64, [704, 1536], 300, 24),        # blocks of 24 rows: block boundaries inside key groups
])
def test_batched_prefill_paged(C, Ts, B, bs):
    """Chunks of several tokens over a paged cache (shuffled block table): the
    same checks as the contiguous batch, and the chunk's rows written to their
    paged slots."""
    wl = LLAMA.replace(L=max(Ts) + C, C=C, H_q=8, H_kv=2, n_q=24, B=B)
    print(f"[case] paged prefill C={C} T={Ts} block={bs}", flush=True)
    nb = len(Ts)
    cur = [gen.chunk_inputs(wl, T // C, seq=s) for s, T in enumerate(Ts)]
    prior = [[gen.chunk_inputs(wl, k, seq=s) for k in range(T // C)] for s, T in enumerate(Ts)]
    nblk = [(T + C + bs - 1) // bs for T in Ts]
    perm = np.random.default_rng([0x5EED, 77, C, bs]).permutation(sum(nblk)).astype(np.int32)
    table = np.zeros((nb, max(nblk)), dtype=np.int32)
    pos = 0
    for s in range(nb):
        table[s, :nblk[s]] = perm[pos:pos + nblk[s]]
        pos += nblk[s]
    kpool = np.zeros((sum(nblk), wl.H_kv, bs, wl.d), dtype=np.uint16)
    vpool = np.zeros_like(kpool)
    logical = []
    for s, T in enumerate(Ts):
        kl = np.zeros((wl.H_kv, nblk[s] * bs, wl.d), dtype=np.uint16)
        vl = np.zeros_like(kl)
        if T:
            kl[:, :T] = np.concatenate([c[1] for c in prior[s]], axis=1)
            vl[:, :T] = np.concatenate([c[2] for c in prior[s]], axis=1)
        logical.append((kl[:, :T].copy(), vl[:, :T].copy()))
        for j in range(nblk[s]):
            kpool[table[s, j]] = kl[:, j * bs:(j + 1) * bs]
            vpool[table[s, j]] = vl[:, j * bs:(j + 1) * bs]
    dev = "cuda"
    kp_d, vp_d = runner.to_device(kpool, dev), runner.to_device(vpool, dev)
    table_d = torch.tensor(table, dtype=torch.int32, device=dev)
    q = runner.to_device(np.stack([c[0] for c in cur]), dev)
    kn = runner.to_device(np.stack([c[1] for c in cur]), dev)
    vn = runner.to_device(np.stack([c[2] for c in cur]), dev)
    h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16)
    p = K.Params(wl.n_q, wl.B)
    prior_d = torch.tensor(Ts, dtype=torch.int64, device=dev)      # kept alive: the batch holds its pointer
    b = K.batch(Ts, C, prior_d)
    cache = K.cache(kp_d, vp_d, kpool.shape[0], bs, table_d)
    ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
    nqp = min(wl.n_q, C)
    idx = torch.full((nb, wl.H_kv, B), -7, dtype=torch.int32, device=dev)
    keep = torch.full((nb, wl.H_q, nqp), -7, dtype=torch.int32, device=dev)
    S = torch.full((nb, wl.H_kv, max(max(Ts), 1)), float("nan"), dtype=torch.float32, device=dev)
    K.kvsel_select(h, b, p, q, cache, idx, None, None, keep, S, ws)
    out = torch.empty(nb, wl.H_q, C, wl.d, dtype=torch.float32, device=dev)
    idx2 = torch.full_like(idx, -7)
    K.kvsel_prefill_chunk(h, b, p, q, kn, vn, cache, out, idx2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx2.cpu().numpy())
    parity.check_compaction(h, b, p, cache, ws, Ts, C, idx2.cpu().numpy(), logical, [(c[1], c[2]) for c in cur])
    kpa, vpa = runner.to_host_bits(kp_d), runner.to_host_bits(vp_d)
    O = out.double().cpu().numpy()
    for s, T in enumerate(Ts):
        # the chunk's rows in their paged slots, the prior rows untouched
        for t in range(T + C):
            blk, off = table[s, t // bs], t % bs
            want_k = cur[s][1][:, t - T] if t >= T else logical[s][0][:, t]
            want_v = cur[s][2][:, t - T] if t >= T else logical[s][1][:, t]
            assert np.array_equal(kpa[blk, :, off], want_k) and np.array_equal(vpa[blk, :, off], want_v), (s, t)
        Qc, Kn, Vn = (gen.to_f64(x) for x in cur[s])
        Kp, Vp = gen.to_f64(logical[s][0]), gen.to_f64(logical[s][1])
        idx_h = idx[s].cpu().numpy()
        if T > B:
            keep_h = keep[s].cpu().numpy()
            for hh in range(wl.H_q):
                parity.check_keep(Qc[hh], wl.n_q, keep_h[hh])
            S_or = quoka.key_scores(Qc, [np.sort(keep_h[hh]) for hh in range(wl.H_q)], Kp)
            for g in range(wl.H_kv):
                parity.check_close(S[s, g, :T].cpu().numpy(), S_or[g], parity.S_TOL, f"S seq {s} head {g}")
                parity.check_idx(S_or[g], B, idx_h[g], S[s, g, :T].cpu().numpy())
        else:
            for g in range(wl.H_kv):
                assert np.array_equal(idx_h[g, :T], np.arange(T)) and np.all(idx_h[g, T:] == -1)
        n = min(B, T)
        O_or = quoka.attend(Qc, [Kp[g, idx_h[g, :n]] for g in range(wl.H_kv)],
                            [Vp[g, idx_h[g, :n]] for g in range(wl.H_kv)], Kn, Vn)
        parity.check_close(O[s], O_or, parity.o_tol(wl.dtype), f"O seq {s}")


def test_sparse_attn_empty_set_without_arrays():
    """n_sel_max = 0 with no compacted arrays at all (k_sel = v_sel = NULL, as
    the header allows): every query attends to the chunk's own keys only,
    causally; checked against the oracle with empty selected sets."""
    wl = LLAMA.replace(L=1400, C=700, H_q=8, H_kv=2, n_q=100, B=900)
    print("[case] sparse_attn n_sel_max=0, NULL k_sel/v_sel", flush=True)
    chunks = [gen.chunk_inputs(wl, k, seq=s) for s, k in enumerate([0, 1])]
    dev = "cuda"
    q = runner.to_device(np.stack([c[0] for c in chunks]), dev)
    kc = runner.to_device(np.stack([c[1] for c in chunks]), dev)
    vc = runner.to_device(np.stack([c[2] for c in chunks]), dev)
    h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16)
    bt = K.batch([0, 0], wl.C, None)
    nsel = torch.zeros(2, dtype=torch.int32, device=dev)
    ws = torch.empty(K.sparse_attn_workspace_size(h, bt, 0), dtype=torch.uint8, device=dev)
    out = torch.empty(2, wl.H_q, wl.C, wl.d, dtype=torch.float32, device=dev)
    K.kvsel_sparse_attn(h, bt, q, None, None, nsel, 0, kc, vc, out, ws)
    torch.cuda.synchronize()
    O = out.double().cpu().numpy()
    empty = np.zeros((0, wl.d))
    for s, c in enumerate(chunks):
        Qc, Kc, Vc = (gen.to_f64(x) for x in c)
        ref = quoka.attend(Qc, [empty] * wl.H_kv, [empty] * wl.H_kv, Kc, Vc)
        parity.check_close(O[s], ref, parity.o_tol("bf16"), f"O seq {s}")


@pytest.mark.parametrize("dup,H_q,T", [(12000, 4, 20480), (9000, 4, 20480), (12000, 2, 20480), (12000, 4, 40960)])
def test_topb_boundary_bin_over_capacity(dup, H_q, T):
    """More prior keys than the threshold search keeps on chip (6144) share
    the value bin of the B-th score (an exact-duplicate key row repeated `dup`
    times, plus near-duplicates one
    bf16 step apart in a few coordinates): the top-B's threshold search then
    works over the whole score row instead of the on-chip boundary list.  The
    kept set must be the exact top-B of the GPU's own scores (ties to the lower
    index) and match the oracle outside the 1e-4 band.  With 2 query heads the
    scan splits the KV head at most twice and the threshold launch also sums
    the partials and counts the histogram itself (the fused form).  With 40960
    keys the threshold search holds the scores in a ring of four 8192-key
    steps of registers and reloads it."""
    rng = np.random.default_rng([0x5EED, 4242, dup] + ([] if T == 20480 else [T]))
    H_kv, d, C = 1, 128, 64
    base = gen.WORKLOADS["llama8b_32k"]
    wl = base.replace(L=T + C, C=C, H_q=H_q, H_kv=H_kv, n_q=8, B=1)
    q = gen.f32_to_bf16_bits((0.5 * rng.standard_normal((H_q, C, d)) + 1.0).astype(np.float32))
    other = (0.5 * rng.standard_normal((T, d)) + 0.3 * rng.standard_normal(d)).astype(np.float32)
    row = (0.5 * rng.standard_normal(d) + 1.0).astype(np.float32)
    keys = gen.f32_to_bf16_bits(other)
    pos = rng.permutation(T)
    dup_pos, near_pos = pos[:dup], pos[dup:dup + 2000]
    rb = gen.f32_to_bf16_bits(row[None])[0]
    keys[dup_pos] = rb
    near = np.repeat(rb[None], len(near_pos), axis=0).astype(np.int32)
    big = np.nonzero(np.abs(row) > 0.25)[0]                # coordinates far from zero: +-1 on the bits is +-1 ulp
    cols = big[rng.integers(0, len(big), size=(len(near_pos), 3))]
    steps = rng.choice([-1, 1], size=(len(near_pos), 3))
    for j in range(3):
        near[np.arange(len(near_pos)), cols[:, j]] += steps[:, j]           # one bf16 ulp per coordinate
    keys[near_pos] = near.astype(np.uint16)
    Q64, K64 = gen.to_f64(q), gen.to_f64(keys)[None]
    keep = [quoka.query_keep(Q64[hh], wl.n_q) for hh in range(H_q)]
    S_or = quoka.key_scores(Q64, keep, K64)[0]
    s_dup = S_or[dup_pos[0]]
    above = int(np.sum(S_or > s_dup + 1e-9))
    B = above + dup // 2                      # the B-th score falls among the duplicates
    print(f"[case] top-B boundary bin: {dup} duplicates, H_q={H_q}, {above} keys above them, B={B}", flush=True)
    dev = "cuda"
    kcache = np.zeros((1, H_kv, T, d), dtype=np.uint16)
    kcache[0, 0] = keys
    vcache = gen.f32_to_bf16_bits(rng.standard_normal((1, H_kv, T, d)).astype(np.float32))
    h = K.heads(H_q, H_kv, d, K.KVSEL_BF16)
    p = K.Params(wl.n_q, B)
    prior = torch.tensor([T], dtype=torch.int64, device=dev)
    b = K.batch([T], C, prior)
    kd, vd = runner.to_device(kcache, dev), runner.to_device(vcache, dev)
    cache = K.cache(kd, vd, T)
    ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
    idx = torch.full((1, H_kv, B), -7, dtype=torch.int32, device=dev)
    keep_d = torch.full((1, H_q, wl.n_q), -7, dtype=torch.int32, device=dev)
    S = torch.full((1, H_kv, T), float("nan"), dtype=torch.float32, device=dev)
    ks = torch.empty(1, H_kv, B, d, dtype=torch.bfloat16, device=dev)
    vs = torch.empty_like(ks)
    K.kvsel_select(h, b, p, runner.to_device(q[None], dev), cache, idx, ks, vs, keep_d, S, ws)
    torch.cuda.synchronize()
    keep_h = keep_d[0].cpu().numpy()
    for hh in range(H_q):
        parity.check_keep(Q64[hh], wl.n_q, keep_h[hh])
    S_c = quoka.key_scores(Q64, [np.sort(keep_h[hh]) for hh in range(H_q)], K64)[0]
    S_h, idx_h = S[0, 0].cpu().numpy(), idx[0, 0].cpu().numpy()
    parity.check_close(S_h, S_c, parity.S_TOL, "S")
    # the GPU's boundary bin really holds more than 8192 keys
    thr = np.sort(S_h)[::-1][B - 1]
    in_bin = np.sum(np.floor((S_h.astype(np.float32) + np.float32(1)) * np.float32(2048)) ==
                    np.floor((np.float32(thr) + np.float32(1)) * np.float32(2048)))
    assert in_bin > 8192, in_bin
    parity.check_idx(S_c, B, idx_h, S_h)
    n = B
    assert np.array_equal(runner.to_host_bits(ks[0, 0])[:n], keys[idx_h[:n]])
    assert np.array_equal(runner.to_host_bits(vs[0, 0])[:n], vcache[0, 0, idx_h[:n]])


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_in_place_when_nothing_selected(d):
    """When no sequence selects (every T_b <= B) on a contiguous cache, the call
    appends the chunk and attends to the cache prefix in place (no compacted
    copy).  Ragged prior lengths including 0; the cache rows past each
    sequence's T_b + C hold NaN, so any read beyond the key list would show in
    O.  Every sequence against the oracle with every prior key kept."""
    C, Ts, B = 200, [0, 200, 600, 450], 600
    wl = LLAMA.replace(L=max(Ts) + C, C=C, H_q=8, H_kv=2, d=d, n_q=24, B=B)
    print(f"[case] in-place prefill d={d} T={Ts}", flush=True)
    nb, cap = len(Ts), max(Ts) + C + 64
    cur = [gen.chunk_inputs(wl, T // C if T % C == 0 else 0, seq=s) for s, T in enumerate(Ts)]
    rng = np.random.default_rng([0x5EED, 991, d])
    nan = np.uint16(0x7FC0)
    kc = np.full((nb, wl.H_kv, cap, wl.d), nan, dtype=np.uint16)
    vc = np.full_like(kc, nan)
    for s, T in enumerate(Ts):
        kc[s, :, :T] = gen.f32_to_bf16_bits(rng.standard_normal((wl.H_kv, T, wl.d)).astype(np.float32))
        vc[s, :, :T] = gen.f32_to_bf16_bits(rng.standard_normal((wl.H_kv, T, wl.d)).astype(np.float32))
    dev = "cuda"
    kc_d, vc_d = runner.to_device(kc, dev), runner.to_device(vc, dev)
    q = runner.to_device(np.stack([c[0] for c in cur]), dev)
    kn = runner.to_device(np.stack([c[1] for c in cur]), dev)
    vn = runner.to_device(np.stack([c[2] for c in cur]), dev)
    h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16)
    p = K.Params(wl.n_q, wl.B)
    prior_d = torch.tensor(Ts, dtype=torch.int64, device=dev)
    b = K.batch(Ts, C, prior_d)
    cache = K.cache(kc_d, vc_d, cap)
    assert K.compacted_view(h, b, p, cache) is None, "expected the in-place attention (no compacted lists)"
    ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
    out = torch.empty(nb, wl.H_q, C, wl.d, dtype=torch.float32, device=dev)
    idx = torch.full((nb, wl.H_kv, B), -7, dtype=torch.int32, device=dev)
    K.kvsel_prefill_chunk(h, b, p, q, kn, vn, cache, out, idx, ws)
    torch.cuda.synchronize()
    kc_after, vc_after = runner.to_host_bits(kc_d), runner.to_host_bits(vc_d)
    O = out.double().cpu().numpy()
    idx_h = idx.cpu().numpy()
    assert not np.isnan(O).any(), "a NaN row past the key list was read"
    for s, T in enumerate(Ts):
        assert np.array_equal(kc_after[s, :, T:T + C], cur[s][1]) and np.array_equal(vc_after[s, :, T:T + C], cur[s][2])
        assert np.array_equal(kc_after[s, :, :T], kc[s, :, :T]) and np.array_equal(kc_after[s, :, T + C:], kc[s, :, T + C:])
        for g in range(wl.H_kv):
            assert np.array_equal(idx_h[s, g, :T], np.arange(T)) and np.all(idx_h[s, g, T:] == -1)
        Qc, Kn, Vn = (gen.to_f64(x) for x in cur[s])
        Kp, Vp = gen.to_f64(kc[s, :, :T]), gen.to_f64(vc[s, :, :T])
        O_or = quoka.attend(Qc, [Kp[g] for g in range(wl.H_kv)], [Vp[g] for g in range(wl.H_kv)], Kn, Vn)
        parity.check_close(O[s], O_or, parity.o_tol(wl.dtype), f"O seq {s}")
