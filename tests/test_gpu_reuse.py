"""kvsel_decode_reuse on the GPU against the oracle over consecutive decode
steps: the kept index sets (as kvsel_select's, which are checked against the
oracle's scores), the slot contents and hit / miss counts bit for bit against
oracle/reuse.py given the GPU's index sets, the slot rows bit for bit against
the cache, the output within the bf16 tolerance, and the append of each step's
token.  SQD page (rit.work), sparse-attention paragraph."""
import numpy as np
import pytest
import torch

import parity
from chunked_prefill_kv_amd import gen, runner
from chunked_prefill_kv_amd import kvsel as K
from oracle import quoka, reuse

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.load()


def _paged(wl, di, steps, seed):
    """A shuffled paged pool with room for `steps` more tokens per sequence, holding di's prior rows."""
    bs, nb = wl.block_size, wl.batch
    T = di.prior_len.astype(np.int64)
    nblk = [int((t + steps + bs - 1) // bs) for t in T]
    perm = np.random.default_rng([0x5EED, 501, seed]).permutation(sum(nblk)).astype(np.int32)
    table = np.full((nb, max(nblk)), -1, dtype=np.int32)
    kpool = np.zeros((sum(nblk), wl.H_kv, bs, wl.d), dtype=np.uint16)
    vpool = np.zeros_like(kpool)
    logical, at = [], 0
    for b in range(nb):
        table[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += nblk[b]
        kp, vp = di.logical_kv(b, bs)
        kl = np.zeros((wl.H_kv, (T[b] + steps), wl.d), dtype=np.uint16)
        vl = np.zeros_like(kl)
        kl[:, :T[b]], vl[:, :T[b]] = kp, vp
        logical.append([kl, vl])
        for p in range(T[b]):
            kpool[table[b, p // bs], :, p % bs] = kp[:, p]
            vpool[table[b, p // bs], :, p % bs] = vp[:, p]
    return table, kpool, vpool, logical


@pytest.mark.parametrize("variant", ["gqa", "g16_d64", "mqa_g32"])
def test_decode_reuse_consecutive_steps(variant):
    base = gen.WORKLOADS["decode_paged"]
    wl = {"gqa": base.replace(batch=4, decode_len_lo=300, decode_len_hi=2100, B=512),
          "g16_d64": base.replace(batch=3, decode_len_lo=500, decode_len_hi=1500, B=400, H_q=32, H_kv=2, d=64),
          "mqa_g32": base.replace(batch=2, decode_len_lo=700, decode_len_hi=1800, H_q=32, H_kv=1, B=600)}[variant]
    steps = 4
    print(f"[case] decode reuse {variant}, {steps} steps", flush=True)
    di = gen.decode_inputs(wl)
    table, kpool, vpool, logical = _paged(wl, di, steps, 1)
    rng = np.random.default_rng([0x5EED, 502, wl.H_q, wl.d])
    dev = "cuda"
    kp_d, vp_d = runner.to_device(kpool, dev), runner.to_device(vpool, dev)
    table_d = torch.tensor(table, dtype=torch.int32, device=dev)
    cache = K.cache(kp_d, vp_d, kpool.shape[0], wl.block_size, table_d)
    h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16)
    p = K.Params(1, wl.B)
    sel_k = torch.empty(wl.batch, wl.H_kv, wl.B, wl.d, dtype=torch.bfloat16, device=dev)
    sel_v = torch.empty_like(sel_k)
    pos = torch.full((wl.batch, wl.H_kv, wl.B), -1, dtype=torch.int32, device=dev)
    counts = torch.full((wl.batch, wl.H_kv, 2), -7, dtype=torch.int32, device=dev)
    sel = K.sel_cache(sel_k, sel_v, pos, counts)
    prev = np.full((wl.batch, wl.H_kv, wl.B), -1, dtype=np.int64)
    q0 = gen.to_f64(di.q)
    hits_total = 0
    for t in range(steps):
        T = (di.prior_len + t).astype(np.int64)
        # this step's query: the sequence's query plus a small change per step; its new key / value row
        q = gen.f32_to_bf16_bits((q0 + 0.3 * rng.standard_normal(q0.shape)).astype(np.float32))
        kn = gen.f32_to_bf16_bits(rng.standard_normal((wl.batch, wl.H_kv, 1, wl.d)).astype(np.float32))
        vn = gen.f32_to_bf16_bits(rng.standard_normal((wl.batch, wl.H_kv, 1, wl.d)).astype(np.float32))
        prior_d = torch.tensor(T, dtype=torch.int64, device=dev)
        b = K.batch(T.tolist(), 1, prior_d)
        ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
        qd, knd, vnd = (runner.to_device(x, dev) for x in (q, kn, vn))
        S = torch.full((wl.batch, wl.H_kv, int(T.max())), float("nan"), dtype=torch.float32, device=dev)
        idx_sel = torch.full((wl.batch, wl.H_kv, wl.B), -7, dtype=torch.int32, device=dev)
        K.kvsel_select(h, b, p, qd, cache, idx_sel, None, None, None, S, ws)
        out = torch.empty(wl.batch, wl.H_q, 1, wl.d, dtype=torch.float32, device=dev)
        idx = torch.full_like(idx_sel, -7)
        K.kvsel_decode_reuse(h, b, p, qd, knd, vnd, cache, sel, out, idx, ws)
        torch.cuda.synchronize()
        idx_h, S_h = idx.cpu().numpy(), S.cpu().numpy()
        assert np.array_equal(idx_h, idx_sel.cpu().numpy()), f"step {t}: decode_reuse and select disagree on idx"
        pos_h, cnt_h = pos.cpu().numpy().astype(np.int64), counts.cpu().numpy()
        sk_h, sv_h = runner.to_host_bits(sel_k), runner.to_host_bits(sel_v)
        O = out.double().cpu().numpy()
        kpa, vpa = runner.to_host_bits(kp_d), runner.to_host_bits(vp_d)
        for bi in range(wl.batch):
            Tb = int(T[bi])
            n = min(wl.B, Tb)
            kl, vl = logical[bi]
            Kp, Vp = gen.to_f64(kl[:, :Tb]), gen.to_f64(vl[:, :Tb])
            Qc = gen.to_f64(q[bi])
            if Tb > wl.B:
                S_or = quoka.key_scores(Qc, [np.array([0])] * wl.H_q, Kp)
                for g in range(wl.H_kv):
                    parity.check_close(S_h[bi, g, :Tb], S_or[g], parity.S_TOL, f"S step {t} seq {bi} head {g}")
                    parity.check_idx(S_or[g], wl.B, idx_h[bi, g], S_h[bi, g, :Tb])
            gidx = [idx_h[bi, g, :n].astype(np.int64) for g in range(wl.H_kv)]
            ref = reuse.decode_step(Qc, gen.to_f64(kn[bi]), gen.to_f64(vn[bi]), Kp, Vp, prev[bi], 1, wl.B, idx=gidx)
            assert np.array_equal(pos_h[bi], ref["pos"]), f"step {t} seq {bi}: slot contents differ"
            assert np.array_equal(cnt_h[bi, :, 0], ref["hits"]) and np.array_equal(cnt_h[bi, :, 1], ref["misses"])
            for g in range(wl.H_kv):
                slots = ref["pos"][g, :n]
                assert np.array_equal(sk_h[bi, g, :n], kl[g, slots]) and np.array_equal(sv_h[bi, g, :n], vl[g, slots]), \
                    f"step {t} seq {bi} head {g}: slot rows differ from the cache rows"
            parity.check_close(O[bi], ref["O"], parity.o_tol("bf16"), f"O step {t} seq {bi}")
            # the step's token landed in its paged slot
            blk = table[bi, Tb // wl.block_size]
            assert np.array_equal(kpa[blk, :, Tb % wl.block_size], kn[bi, :, 0])
            assert np.array_equal(vpa[blk, :, Tb % wl.block_size], vn[bi, :, 0])
            kl[:, Tb], vl[:, Tb] = kn[bi, :, 0], vn[bi, :, 0]
            hits_total += int(ref["hits"].sum())
        prev = pos_h
    assert hits_total > 0
