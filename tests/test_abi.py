"""The C-ABI library loads, exports every symbol include/kvsel.h declares, and
rejects bad arguments on the host before enqueuing anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

from chunked_prefill_kv_amd import kvsel as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")

pytestmark = pytest.mark.skipif(not os.path.exists(K.LIB_PATH), reason="libkvsel.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(K.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(K.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert K.version() == 102


def _bad(h=None, b=None, p=None):
    h = h or K.heads(32, 8, 128, K.KVSEL_BF16)
    b = b or K.batch([4096], 2048, None)
    p = p or K.Params(256, 4096)
    return h, b, p


def _status(h, b, p):
    n = ctypes.c_size_t()
    b.prior_len_dev = 256          # a fake device address: size queries never dereference it
    return K.load().kvsel_workspace_size(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,code", [
    (dict(h=K.heads(30, 8, 128, K.KVSEL_BF16)), K.KVSEL_ERR_INVALID_ARG),    # h_q % h_kv
    (dict(h=K.heads(32, 0, 128, K.KVSEL_BF16)), K.KVSEL_ERR_INVALID_ARG),
    (dict(h=K.heads(32, 8, 96, K.KVSEL_BF16)), K.KVSEL_ERR_UNSUPPORTED),     # d
    (dict(p=K.Params(256, 4096, 2)), K.KVSEL_ERR_INVALID_ARG),                # pooling
    (dict(h=K.heads(32, 8, 128, 7)), K.KVSEL_ERR_INVALID_ARG),               # dtype
    (dict(h=K.heads(32, 8, 128, K.KVSEL_BF16, -1.0)), K.KVSEL_ERR_INVALID_ARG),
    (dict(p=K.Params(0, 4096)), K.KVSEL_ERR_INVALID_ARG),                     # n_q
    (dict(p=K.Params(8, 0)), K.KVSEL_ERR_INVALID_ARG),                        # budget
    (dict(b=K.batch([-1], 16, None)), K.KVSEL_ERR_INVALID_ARG),               # prior length
    (dict(b=K.batch([0], 0, None)), K.KVSEL_ERR_INVALID_ARG),                 # chunk length
])
def test_argument_errors(kw, code):
    st, _ = _status(*_bad(**kw))
    assert st == code
    assert K.last_error()


def test_workspace_size_grows_with_context():
    h, b, p = _bad()
    st, small = _status(h, b, p)
    assert st == K.KVSEL_OK and small > 0
    st, big = _status(h, K.batch([30720], 2048, None), p)
    assert st == K.KVSEL_OK and big > small


def test_calls_reject_before_enqueue():
    """Errors found on the host return before any HIP call (this host has no GPU)."""
    lib = K.load()
    h, p = K.heads(32, 8, 128, K.KVSEL_BF16), K.Params(256, 4096)
    b = K.batch([8192], 2048, None)
    b.prior_len_dev = 256
    fake = 1 << 20
    c = K.Cache(fake, fake, 4096, 0, 0, None)        # capacity 4096 < 8192 + 2048
    st = lib.kvsel_prefill_chunk(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake, fake, fake,
                                 ctypes.byref(c), fake, K.KVSEL_F32, None, fake, 1 << 30, None)
    assert st == K.KVSEL_ERR_INVALID_ARG and "capacity" in K.last_error()
    c = K.Cache(fake, fake, 16384, 0, 0, None)
    st = lib.kvsel_prefill_chunk(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake, fake, fake,
                                 ctypes.byref(c), fake, K.KVSEL_F32, None, fake, 16, None)
    assert st == K.KVSEL_ERR_WORKSPACE
    st = lib.kvsel_prefill_chunk(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake + 2, fake, fake,
                                 ctypes.byref(c), fake, K.KVSEL_F32, None, fake, 1 << 30, None)
    assert st == K.KVSEL_ERR_INVALID_ARG and "aligned" in K.last_error()
    # paged cache whose block table is too short
    c = K.Cache(fake, fake, 4096, 16, 8, fake)
    st = lib.kvsel_select(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake, ctypes.byref(c), fake,
                          None, None, None, None, fake, 1 << 30, None)
    assert st == K.KVSEL_ERR_INVALID_ARG and "blocks" in K.last_error()
    # sparse_attn: bad out dtype
    st = lib.kvsel_sparse_attn(ctypes.byref(h), ctypes.byref(b), fake, fake, fake, fake, 16, fake, fake, fake, 9,
                               fake, 1 << 30, None)
    assert st == K.KVSEL_ERR_INVALID_ARG


@pytest.mark.parametrize("T,B", [(1 << 21, 4096), ((1 << 21) + 1, 4096), (2048, (1 << 21) + 1), (100, 1 << 22)])
def test_selection_limit_rejected_on_host(T, B):
    """Prior lengths or budgets above 2^21 keys cannot be selected from (the
    top-B's per-segment counters live on chip): every sizing or launching
    entry point refuses them with UNSUPPORTED before anything is enqueued;
    2^21 itself is accepted."""
    h, p = K.heads(32, 8, 128, K.KVSEL_BF16), K.Params(256, B)
    b = K.batch([T], 2048, None)
    st, _ = _status(h, b, p)
    ok = max(T, B) <= (1 << 21)
    assert st == (K.KVSEL_OK if ok else K.KVSEL_ERR_UNSUPPORTED), K.last_error()
    if ok:
        return
    assert "2097152" in K.last_error()
    lib, fake = K.load(), 1 << 20
    c = K.Cache(fake, fake, T + 4096, 0, 0, None)
    for call in ("select", "prefill"):
        if call == "select":
            st = lib.kvsel_select(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake, ctypes.byref(c), fake,
                                  None, None, None, None, fake, 1 << 40, None)
        else:
            st = lib.kvsel_prefill_chunk(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake, fake, fake,
                                         ctypes.byref(c), fake, K.KVSEL_BF16, None, fake, 1 << 40, None)
        assert st == K.KVSEL_ERR_UNSUPPORTED, (call, K.last_error())


def test_compacted_view_host_arithmetic():
    """The compacted lists sit inside the workspace, after the selection's
    buffers; the gathering attention (one 128-row block per KV head) builds
    none."""
    h, p = K.heads(32, 8, 128, K.KVSEL_BF16), K.Params(256, 4096)
    b = K.batch([30720], 2048, None)
    b.prior_len_dev = 256
    fake = 1 << 20
    c = K.Cache(fake, fake, 32768, 0, 0, None)
    v = K.compacted_view(h, b, p, c)
    st, ws = _status(h, K.batch([30720], 2048, None), p)
    assert v is not None and v["v_transposed"] and v["slots"] == 4096 + 2048
    assert v["k_offset"] % 256 == 0 and v["v_offset"] >= v["k_offset"] + 8 * v["slots"] * 128 * 2
    assert v["v_offset"] + 8 * v["slots"] * 128 * 2 <= ws
    b1 = K.batch([4096] * 4, 1, None)
    b1.prior_len_dev = 256
    assert K.compacted_view(h, b1, K.Params(1, 2048), K.Cache(fake, fake, 8192, 0, 0, None)) is None


def test_decode_reuse_rejects_on_host():
    """kvsel_decode_reuse: NULL selected-entry cache, fp32, a budget above 8192 and
    a chunk too long for the gathering attention are refused before any launch."""
    lib, fake = K.load(), 1 << 20
    c = K.Cache(fake, fake, 4096, 16, 512, fake)
    sel = K.SelCache(fake, fake, fake, None)

    def call(h, b, p, s):
        b.prior_len_dev = 256
        return lib.kvsel_decode_reuse(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p), fake, fake, fake,
                                      ctypes.byref(c), s, fake, K.KVSEL_F32, None, fake, 1 << 40, None)
    h, p = K.heads(32, 8, 128, K.KVSEL_BF16), K.Params(1, 2048)
    assert call(h, K.batch([5000] * 4, 1, None), p, None) == K.KVSEL_ERR_INVALID_ARG
    assert call(K.heads(32, 8, 128, K.KVSEL_F32), K.batch([5000] * 4, 1, None), p, ctypes.byref(sel)) == K.KVSEL_ERR_UNSUPPORTED
    assert call(h, K.batch([5000] * 4, 1, None), K.Params(1, 9000), ctypes.byref(sel)) == K.KVSEL_ERR_UNSUPPORTED
    assert call(h, K.batch([5000] * 4, 64, None), p, ctypes.byref(sel)) == K.KVSEL_ERR_UNSUPPORTED
    assert "128" in K.last_error()
