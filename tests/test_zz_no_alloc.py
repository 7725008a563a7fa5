"""kvsel_prefill_chunk_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's fixed per-GPU scratch array) against
kvsel_prefill_chunk with a caller workspace, through the C ABI: the same
outputs, cache append and kept index sets, bit for bit, over consecutive calls
of decreasing size (the scratch keeps the previous call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

from chunked_prefill_kv_amd import gen, runner
from chunked_prefill_kv_amd import kvsel as K

pytestmark = pytest.mark.gpu

LLAMA = gen.WORKLOADS["llama8b_32k"]


def _case(wl, Ts, seed):
    """Inputs of one batched call: chunk tensors and a contiguous cache holding the prior rows."""
    C = wl.C
    cap = max(Ts) + C
    cur = [gen.chunk_inputs(wl, T // C, seq=seed + s) for s, T in enumerate(Ts)]
    kc = np.zeros((len(Ts), wl.H_kv, cap, wl.d), dtype=np.uint16)
    vc = np.zeros_like(kc)
    for s, T in enumerate(Ts):
        for k in range(T // C):
            c = gen.chunk_inputs(wl, k, seq=seed + s)
            kc[s, :, k * C:(k + 1) * C] = c[1]
            vc[s, :, k * C:(k + 1) * C] = c[2]
    return cur, kc, vc, cap


def _run(wl, Ts, cur, kc, vc, cap, noalloc):
    dev = "cuda"
    h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16)
    p = K.Params(wl.n_q, wl.B)
    prior = torch.tensor(Ts, dtype=torch.int64, device=dev)
    b = K.batch(Ts, wl.C, prior)
    kd, vd = runner.to_device(kc, dev), runner.to_device(vc, dev)
    cache = K.cache(kd, vd, cap)
    q = runner.to_device(np.stack([c[0] for c in cur]), dev)
    kn = runner.to_device(np.stack([c[1] for c in cur]), dev)
    vn = runner.to_device(np.stack([c[2] for c in cur]), dev)
    out = torch.full((len(Ts), wl.H_q, wl.C, wl.d), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((len(Ts), wl.H_kv, wl.B), -7, dtype=torch.int32, device=dev)
    if noalloc:
        K.kvsel_prefill_chunk_noalloc(h, b, p, q, kn, vn, cache, out, idx)
    else:
        ws = torch.empty(K.workspace_size(h, b, p), dtype=torch.uint8, device=dev)
        K.kvsel_prefill_chunk(h, b, p, q, kn, vn, cache, out, idx, ws)
    torch.cuda.synchronize()
    return out.cpu(), idx.cpu(), runner.to_host_bits(kd), runner.to_host_bits(vd)


CALLS = [
    # packed attention with selection on both sequences, then a smaller packed
    # call (one selecting sequence, one with T <= B), then a short-chunk call
    # (gathering attention, no packed lists)
    (LLAMA.replace(L=3584, C=512, H_q=8, H_kv=2, n_q=64, B=900), [2560, 3072], 11),
    (LLAMA.replace(L=2048, C=256, H_q=8, H_kv=2, n_q=40, B=700), [1536, 512], 21),
    (LLAMA.replace(L=1200, C=30, H_q=8, H_kv=2, n_q=10, B=150), [600], 31),
]


def test_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.load()
    for i, (wl, Ts, seed) in enumerate(CALLS):
        print(f"[case] no-alloc call {i}: T={Ts} C={wl.C} B={wl.B}", flush=True)
        cur, kc, vc, cap = _case(wl, Ts, seed)
        ref = _run(wl, Ts, cur, kc, vc, cap, noalloc=False)
        got = _run(wl, Ts, cur, kc, vc, cap, noalloc=True)
        assert torch.equal(got[1], ref[1]), f"call {i}: kept index sets differ"
        assert torch.equal(got[0], ref[0]), f"call {i}: outputs differ"
        assert not torch.isnan(got[0]).any()
        assert np.array_equal(got[2], ref[2]) and np.array_equal(got[3], ref[3]), f"call {i}: cache differs"


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A workspace need above KVSEL_NOALLOC_SCRATCH_BYTES (64 MiB) is refused before any launch."""
    lib = K.load()
    h, p = K.heads(64, 8, 128, K.KVSEL_BF16), K.Params(512, 8192)
    b = K.batch([126976], 4096, None)
    b.prior_len_dev = 256
    n = ctypes.c_size_t()
    assert lib.kvsel_workspace_size(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value > 64 << 20
    fake = 1 << 20
    c = K.Cache(fake, fake, 131072, 0, 0, None)
    st = lib.kvsel_prefill_chunk_noalloc(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake, fake, fake,
                                         ctypes.byref(c), fake, K.KVSEL_BF16, None, None)
    assert st == K.KVSEL_ERR_UNSUPPORTED and "scratch" in K.last_error()
