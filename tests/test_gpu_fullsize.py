"""Full-size workloads on the GPU, in the launch configuration the bench times
(bf16 output, every chunk through kvsel_prefill_chunk), checked against the
oracle on sampled chunks and KV heads (prefill) or sampled sequences (decode).
"""
import numpy as np
import pytest
import torch

import parity
from chunked_prefill_kv_amd import gen, runner
from chunked_prefill_kv_amd import kvsel as K
from oracle import quoka

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.load()


def _sampled_chunk(r, chunks, k, heads, pooling="head"):
    """Rules 1-3 and O for chunk k on KV heads `heads`, after chunks < k ran through prefill."""
    wl = r.wl
    T, C = r.starts[k], r.lens[k]
    G = wl.G
    dev = r.device
    nqp = min(wl.n_q, C)
    idx = torch.full((1, wl.H_kv, wl.B), -7, dtype=torch.int32, device=dev)
    ks = torch.empty(1, wl.H_kv, wl.B, wl.d, dtype=r.dt, device=dev)
    vs = torch.empty_like(ks)
    group = pooling == "group" and C > 1
    keep = torch.full((1, wl.H_kv if group else wl.H_q, nqp), -7, dtype=torch.int32, device=dev)
    S = torch.full((1, wl.H_kv, max(T, 1)), float("nan"), dtype=torch.float32, device=dev)
    K.kvsel_select(r.h, r.batches[k], r.p, r.chunks[k][0], r.cache, idx, ks, vs, keep, S, r.ws)
    r.run_chunk(k)
    torch.cuda.synchronize()
    idx_h, keep_h, S_h = idx[0].cpu().numpy(), keep[0].cpu().numpy(), S[0].cpu().numpy()
    assert np.array_equal(r.idx[k][0].cpu().numpy(), idx_h)
    Og = r.outs[k][0].float().cpu().numpy().astype(np.float64)
    ks_h, vs_h = runner.to_host_bits(ks[0]), runner.to_host_bits(vs[0])
    # the compacted lists the timed attention consumed, bit for bit, on every KV head
    pk = (np.concatenate([c[1] for c in chunks[:k]], axis=1), np.concatenate([c[2] for c in chunks[:k]], axis=1)) \
        if k else (None, None)
    parity.check_compaction(r.h, r.batches[k], r.p, r.cache, r.ws, [T], C, idx_h[None], [pk], [(chunks[k][1], chunks[k][2])])
    recall = []
    for g in heads:
        hs = slice(g * G, (g + 1) * G)
        Qc = gen.to_f64(chunks[k][0][hs])
        kp_bits = np.concatenate([c[1][g:g + 1] for c in chunks[:k]], axis=1)
        vp_bits = np.concatenate([c[2][g:g + 1] for c in chunks[:k]], axis=1)
        Kp, Vp = gen.to_f64(kp_bits), gen.to_f64(vp_bits)
        if T <= wl.B:                          # nothing to select: every prior key kept
            assert np.array_equal(idx_h[g, :T], np.arange(T)) and np.all(idx_h[g, T:] == -1)
        elif group:
            Qbar = quoka.pooled_queries(Qc, 1)
            parity.check_keep(Qbar[0], wl.n_q, keep_h[g])
            S_or = quoka.key_scores_group(Qbar, [np.sort(keep_h[g])], Kp)[0]
        else:
            for i, h in enumerate(range(g * G, (g + 1) * G)):
                parity.check_keep(Qc[i], wl.n_q, keep_h[h])
            S_or = quoka.key_scores(Qc, [np.sort(keep_h[h]) for h in range(g * G, (g + 1) * G)], Kp)[0]
        if T > wl.B:
            parity.check_close(S_h[g, :T], S_or, parity.S_TOL, f"S chunk {k} head {g}")
            parity.check_idx(S_or, wl.B, idx_h[g], S_h[g, :T])
        n = min(wl.B, T)
        sel = idx_h[g, :n]
        assert np.array_equal(ks_h[g, :n], kp_bits[0, sel]) and np.array_equal(vs_h[g, :n], vp_bits[0, sel])
        O_or = quoka.attend(Qc, [Kp[0, sel]], [Vp[0, sel]], gen.to_f64(chunks[k][1][g:g + 1]),
                            gen.to_f64(chunks[k][2][g:g + 1]))
        parity.check_close(Og[hs], O_or, parity.o_tol(wl.dtype), f"O chunk {k} head {g}")
        recall.append(set(sel.tolist()))
    return recall


ALL8 = list(range(8))


@pytest.mark.parametrize("name,sample", [
    ("llama8b_32k", {2: ALL8, 8: ALL8, 15: ALL8}),  # the bench workload: T = B, a mid and the last chunk, every KV head
    ("mqa_64k", {5: [0], 31: [0]}),                 # the single shared KV head: first selecting and last chunk
    ("tiny_f32", {3: [0, 1], 7: [0, 1]}),
])
def test_fullsize_prefill_sampled(name, sample):
    wl = gen.WORKLOADS[name]
    print(f"[case] full-size prefill {name}", flush=True)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    r = runner.PromptRunner(wl, out_dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32)
    r.load(chunks, keep_idx=True)
    for k in range(wl.n_chunks):
        if k in sample:
            _sampled_chunk(r, chunks, k, sample[k])
        else:
            r.run_chunk(k)


def test_fullsize_prefill_group_pooling_sampled():
    """The bench's 32K layer with the group-first pooling order: a mid and the last chunk."""
    wl = gen.WORKLOADS["llama8b_32k"]
    print("[case] full-size group-pooled prefill llama8b_32k", flush=True)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    r = runner.PromptRunner(wl, out_dtype=torch.bfloat16, pooling=K.KVSEL_POOL_GROUP)
    r.load(chunks, keep_idx=True)
    sample = {9: ALL8, 15: ALL8}
    for k in range(wl.n_chunks):
        if k in sample:
            _sampled_chunk(r, chunks, k, sample[k], pooling="group")
        else:
            r.run_chunk(k)


def test_fullsize_gqa_128k_last_chunk_and_needles():
    """The 128K GQA layer: the last chunk on every KV head, and the recall of
    the 64 planted needles at their chunks (a diagnostic of the selection)."""
    wl = gen.WORKLOADS["gqa_128k"]
    print("[case] full-size prefill gqa_128k", flush=True)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    r = runner.PromptRunner(wl, out_dtype=torch.bfloat16)
    r.load(chunks, keep_idx=True)
    for k in range(wl.n_chunks - 1):
        r.run_chunk(k)
    _sampled_chunk(r, chunks, wl.n_chunks - 1, ALL8)
    hits = sum(int(nd.pos in set(r.idx[nd.chunk][0, nd.head // wl.G].cpu().numpy().tolist()))
               for nd in gen.needles(wl))
    print(f"needle recall {hits}/{wl.needles}")
    assert hits >= wl.needles // 2


def test_fullsize_decode_all_sequences():
    """64 ragged sequences (4K-64K) over a paged cache, every sequence checked."""
    wl = gen.WORKLOADS["decode_paged"]
    print("[case] full-size decode", flush=True)
    di = gen.decode_inputs(wl)
    dr = runner.DecodeRunner(wl, di, out_dtype=torch.bfloat16)
    T_max = int(di.prior_len.max())
    S = torch.full((wl.batch, wl.H_kv, T_max), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((wl.batch, wl.H_kv, wl.B), -7, dtype=torch.int32, device="cuda")
    K.kvsel_select(dr.h, dr.b, dr.p, dr.q, dr.cache, idx, None, None, None, S, dr.ws)
    dr.run()
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), dr.idx.cpu().numpy())
    O = dr.out.float().cpu().numpy().astype(np.float64)
    for b in range(wl.batch):
        T = int(di.prior_len[b])
        kp, vp = di.logical_kv(b, wl.block_size)
        Kp, Vp = gen.to_f64(kp), gen.to_f64(vp)
        Qc = gen.to_f64(di.q[b])
        S_or = quoka.key_scores(Qc, [np.array([0])] * wl.H_q, Kp)
        S_h, idx_h = S[b].cpu().numpy(), dr.idx[b].cpu().numpy()
        for g in range(wl.H_kv):
            parity.check_close(S_h[g, :T], S_or[g], parity.S_TOL, f"S seq {b} head {g}")
            parity.check_idx(S_or[g], wl.B, idx_h[g], S_h[g, :T])
        ref = quoka.attend(Qc, [Kp[g, idx_h[g]] for g in range(wl.H_kv)], [Vp[g, idx_h[g]] for g in range(wl.H_kv)],
                           gen.to_f64(di.k_new[b]), gen.to_f64(di.v_new[b]))
        parity.check_close(O[b], ref, parity.o_tol(wl.dtype), f"O seq {b}")
