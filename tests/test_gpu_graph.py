"""The library's launches under HIP graph capture: a whole chunked prompt
(every kvsel_prefill_chunk call, selecting and non-selecting chunks) captured
once and replayed several times, with eager work and synchronisations between
the replays, each replay bit for bit equal to the eager run (the path is
deterministic and issues no memset or host synchronisation)."""
import numpy as np
import pytest
import torch

from chunked_prefill_kv_amd import gen, runner
from chunked_prefill_kv_amd import kvsel as K

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.load()


@pytest.mark.parametrize("name", ["packed", "gathering"])
def test_graph_replay_matches_eager(name):
    base = gen.WORKLOADS["llama8b_32k"]
    wl = {"packed": base.replace(L=2048, C=512, H_q=8, H_kv=2, n_q=64, B=700),
          "gathering": base.replace(L=640, C=32, H_q=8, H_kv=2, n_q=8, B=200)}[name]
    print(f"[case] graph replay {name}", flush=True)
    r = runner.PromptRunner(wl, out_dtype=torch.float32)
    r.load(keep_idx=True)
    r.reset()
    r.run()
    torch.cuda.synchronize()
    eager_out = [o.clone() for o in r.outs]
    eager_idx = [i.clone() for i in r.idx]
    eager_k = r.kc.clone()
    # capture on a side stream after a warm-up there (the graph records the
    # library's launches of one whole prompt)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r.reset()
        r.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.run()
    for rep in range(3):
        r.reset()                                   # eager work between replays
        for o in r.outs:
            o.fill_(float("nan"))
        for i in r.idx:
            i.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, e) in enumerate(zip(r.outs, eager_out)):
            assert torch.equal(o, e), f"replay {rep}: chunk {k} output differs from the eager run"
        for k, (i, e) in enumerate(zip(r.idx, eager_idx)):
            assert torch.equal(i, e), f"replay {rep}: chunk {k} kept set differs"
        assert torch.equal(r.kc, eager_k), f"replay {rep}: cache differs"


def test_graph_replay_decode_matches_eager():
    """A ragged paged decode step (listed scan and top-B grids, gathering
    attention) captured and replayed."""
    wl = gen.WORKLOADS["decode_paged"].replace(batch=12, decode_len_lo=100, decode_len_hi=3000, B=256)
    print("[case] graph replay decode", flush=True)
    dr = runner.DecodeRunner(wl, gen.decode_inputs(wl), out_dtype=torch.float32)
    dr.run()
    torch.cuda.synchronize()
    eager_out, eager_idx = dr.out.clone(), dr.idx.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dr.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dr.run()
    for rep in range(3):
        dr.out.fill_(float("nan"))
        dr.idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dr.out, eager_out), f"replay {rep}: output differs from the eager run"
        assert torch.equal(dr.idx, eager_idx), f"replay {rep}: kept set differs"
