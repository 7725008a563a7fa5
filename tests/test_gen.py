"""Seeded input generators: determinism, shapes, rounding and the structure of each workload."""
import numpy as np
import pytest
import torch

from chunked_prefill_kv_amd import gen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * rng.choice([1e-3, 1, 1e3], size=100000)).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]      # exact ties: to even
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_chunks_are_deterministic_and_regenerable():
    wl = gen.WORKLOADS["llama8b_32k"].replace(L=4096)
    a = gen.chunk_inputs(wl, 1)
    b = gen.chunk_inputs(wl, 1)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and np.array_equal(x, y)
    assert a[0].shape == (32, 2048, 128) and a[1].shape == (8, 2048, 128)
    # a sub-range of rows regenerates identically from the row generator
    rows = gen._q_rows_f32(wl, 3, 0, 2048 + 100, 50)
    assert np.array_equal(gen.f32_to_bf16_bits(rows), a[0][3, 100:150])


def test_ragged_last_chunk():
    wl = gen.WORKLOADS["tiny_f32"].replace(L=1000)
    assert gen.chunk_lengths(wl) == [128] * 7 + [104]
    q, k, v = gen.chunk_inputs(wl, 7)
    assert q.shape == (8, 104, 64) and q.dtype == np.float32


def test_shared_direction_and_sinks():
    wl = gen.WORKLOADS["llama8b_32k"]
    q, k, v = (gen.to_f64(x) for x in gen.chunk_inputs(wl.replace(L=2048), 0))
    kn = np.linalg.norm(k, axis=-1)
    # sinks: first 4 keys are 4x the generator's keys
    base = gen._k_rows_f32(wl, 0, 0, 4, 1)[0]
    assert kn[:, :4].mean() > 3.0 * kn[:, 4:].mean()
    # per-head shared direction: background cosine between keys of one head is high
    kh = k[0, 4:] / kn[0, 4:, None]
    assert (kh[:100] @ kh[100:200].T).mean() > 0.8
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    assert base.shape == (128,)


def test_needles_are_aligned_with_their_queries():
    wl = gen.WORKLOADS["gqa_128k"].replace(L=4096 * 6, needles=8)
    nds = gen.needles(wl)
    assert len(nds) == 8
    for nd in nds:
        assert 3 <= nd.chunk < wl.n_chunks and 4 <= nd.pos < nd.chunk * wl.C
    nd = nds[0]
    q = gen.to_f64(gen.chunk_inputs(wl, nd.chunk)[0])[nd.head, nd.token]
    kc = gen.to_f64(gen.chunk_inputs(wl, nd.pos // wl.C)[1])[nd.head // wl.G, nd.pos % wl.C]
    cos = q @ kc / np.linalg.norm(q) / np.linalg.norm(kc)
    assert abs(cos - 0.9) < 0.01


def test_decode_paged_layout():
    wl = gen.WORKLOADS["decode_paged"].replace(batch=3, decode_len_lo=20, decode_len_hi=70, H_q=4, H_kv=2, d=16)
    di = gen.decode_inputs(wl)
    assert di.prior_len.shape == (3,) and di.q.shape == (3, 4, 1, 16)
    used = di.block_table[di.block_table >= 0]
    assert sorted(used.tolist()) == list(range(di.k_pool.shape[0]))      # a permutation of the pool
    for b in range(3):
        T = int(di.prior_len[b])
        k, v = di.logical_kv(b, wl.block_size)
        assert k.shape == (2, T, 16)
        ref = gen.f32_to_bf16_bits(gen._k_rows_f32(wl, 1, b, 0, T + 1))
        assert np.array_equal(k[1], ref[:T]) and np.array_equal(di.k_new[b, 1, 0], ref[T])
