"""Seeded synthetic inputs for the QuoKA chunked-prefill workloads.

This module only draws and lays out input tensors. It holds none of the
method's arithmetic (no cosine, no selection, no attention), so the CPU oracle
and the HIP path can both consume what it produces without sharing code.

Every draw uses ``numpy.random.default_rng([0x5EED, workload_id, tag, ...])``
so that each tensor, chunk and head can be regenerated on its own.

Floating-point inputs are drawn in fp32 and, for bf16 workloads, rounded to
bf16 by round-to-nearest-even; the bf16 bit patterns (uint16) are the canonical
inputs that both sides read.

Workload shapes (one attention layer each):

* ``tiny_f32``  fp32, L=1024, C=128, H_q=8, H_kv=2, d=64, N_q=32, B=128, i.i.d. N(0,1).
* ``llama8b_32k`` bf16, L=32768, C=2048, H_q=32, H_kv=8, d=128, N_q=256, B=4096.
* ``gqa_128k``  bf16, L=131072, C=4096, H_q=64, H_kv=8, d=128, N_q=512, B=8192, 64 needles.
* ``mqa_64k``   bf16, L=65536, C=2048, H_q=16, H_kv=1, d=128, N_q=256, B=8192.
* ``decode_paged`` bf16, 64 sequences, prior lengths U{4096..65536}, C=1, N_q=1,
  B=2048, H_q=32, H_kv=8, d=128, paged cache (block 16, shuffled block table).

The bf16 generator ("shared direction"): one direction b ~ N(0, I_d) per query
head and, independently, per KV head; Q = 0.5*N(0,1) + 2*b_h, K = 0.5*N(0,1) + 2*b_g;
the keys at absolute positions 0..3 are multiplied by 4 (attention sinks); V ~ N(0,1).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

SEED = 0x5EED

# tensor tags for the seed sequence
TAG_Q, TAG_K, TAG_V, TAG_BQ, TAG_BK, TAG_NEEDLE, TAG_LEN, TAG_PERM = 1, 2, 3, 4, 5, 6, 7, 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed id of the workload
    dtype: str          # "f32" or "bf16"
    L: int              # prompt length (prefill) or 0 for decode
    C: int              # chunk length
    H_q: int
    H_kv: int
    d: int
    n_q: int
    B: int
    gen: str            # "iid" or "shared_dir"
    needles: int = 0
    batch: int = 1
    decode_len_lo: int = 0
    decode_len_hi: int = 0
    block_size: int = 0  # 0 = contiguous cache

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def n_chunks(self) -> int:
        return (self.L + self.C - 1) // self.C if self.L else 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, "f32", 1024, 128, 8, 2, 64, 32, 128, "iid"),
    "llama8b_32k": Workload("llama8b_32k", 2, "bf16", 32768, 2048, 32, 8, 128, 256, 4096, "shared_dir"),
    "gqa_128k": Workload("gqa_128k", 3, "bf16", 131072, 4096, 64, 8, 128, 512, 8192, "shared_dir", needles=64),
    "mqa_64k": Workload("mqa_64k", 4, "bf16", 65536, 2048, 16, 1, 128, 256, 8192, "shared_dir"),
    "decode_paged": Workload("decode_paged", 5, "bf16", 0, 1, 32, 8, 128, 1, 2048, "shared_dir",
                             batch=64, decode_len_lo=4096, decode_len_hi=65536, block_size=16),
}
# order in which the five workloads are listed (configs 1..5)
WORKLOAD_ORDER = ["tiny_f32", "llama8b_32k", "gqa_128k", "mqa_64k", "decode_paged"]


def _rng(*ids: int) -> np.random.Generator:
    return np.random.default_rng([SEED, *ids])


# ----------------------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact fp64 view of an input tensor (uint16 = bf16 bits, or fp32)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _finish(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


# ----------------------------------------------------------------------------- directions

def _dir_q(wl: Workload, h: int) -> np.ndarray:
    return _rng(wl.wid, TAG_BQ, h).standard_normal(wl.d, dtype=np.float32)


def _dir_k(wl: Workload, g: int) -> np.ndarray:
    return _rng(wl.wid, TAG_BK, g).standard_normal(wl.d, dtype=np.float32)


# ----------------------------------------------------------------------------- prefill rows

def _q_rows_f32(wl: Workload, h: int, stream: int, start: int, n: int) -> np.ndarray:
    """fp32 query rows [n, d] of head h for absolute positions [start, start+n) of stream `stream`.

    Rows are drawn per (stream, head, 1024-token block) so any sub-range regenerates identically.
    """
    return _rows(wl, TAG_Q, h, stream, start, n, _dir_q(wl, h) if wl.gen == "shared_dir" else None, 2.0)


def _k_rows_f32(wl: Workload, g: int, stream: int, start: int, n: int) -> np.ndarray:
    x = _rows(wl, TAG_K, g, stream, start, n, _dir_k(wl, g) if wl.gen == "shared_dir" else None, 2.0)
    if wl.gen == "shared_dir" and start < 4:
        x[: max(0, 4 - start)] *= np.float32(4.0)
    return x


def _v_rows_f32(wl: Workload, g: int, stream: int, start: int, n: int) -> np.ndarray:
    return _rows(wl, TAG_V, g, stream, start, n, None, 0.0, noise=1.0)


_BLK = 1024  # rows per seeded block


def _rows(wl: Workload, tag: int, head: int, stream: int, start: int, n: int,
          direction: Optional[np.ndarray], dir_scale: float, noise: Optional[float] = None) -> np.ndarray:
    if noise is None:
        noise = 0.5 if wl.gen == "shared_dir" else 1.0
    out = np.empty((n, wl.d), dtype=np.float32)
    b0, b1 = start // _BLK, (start + n - 1) // _BLK if n else start // _BLK - 1
    for blk in range(b0, b1 + 1):
        z = _rng(wl.wid, tag, head, stream, blk).standard_normal((_BLK, wl.d), dtype=np.float32)
        if noise != 1.0:
            z *= np.float32(noise)
        if direction is not None:
            z += np.float32(dir_scale) * direction[None, :]
        lo = max(start, blk * _BLK)
        hi = min(start + n, (blk + 1) * _BLK)
        out[lo - start: hi - start] = z[lo - blk * _BLK: hi - blk * _BLK]
    return out


# ----------------------------------------------------------------------------- needles

@dataclasses.dataclass(frozen=True)
class Needle:
    chunk: int      # chunk c_n whose query the key is aligned with
    head: int       # query head h_n
    token: int      # token i_n within chunk c_n
    pos: int        # absolute cache position p_n < c_n*C of the planted key


def needles(wl: Workload) -> List[Needle]:
    """The planted needle table: chunk in [3, n_chunks-1], position in [4, chunk*C), distinct per KV head."""
    if not wl.needles:
        return []
    rng = _rng(wl.wid, TAG_NEEDLE)
    out: List[Needle] = []
    used = set()
    hi_chunk = min(31, wl.n_chunks - 1)
    while len(out) < wl.needles:
        c = int(rng.integers(3, hi_chunk + 1))
        h = int(rng.integers(0, wl.H_q))
        i = int(rng.integers(0, wl.C))
        p = int(rng.integers(4, c * wl.C))
        if (h // wl.G, p) in used:
            continue
        used.add((h // wl.G, p))
        out.append(Needle(c, h, i, p))
    return out


def _needle_key(wl: Workload, nd: Needle, k_orig: np.ndarray, idx: int) -> np.ndarray:
    """Key of norm |k_orig| at cosine 0.9 to the needle's (bf16-rounded) query."""
    q = _q_rows_f32(wl, nd.head, 0, nd.chunk * wl.C + nd.token, 1)[0]
    if wl.dtype == "bf16":
        q = bf16_bits_to_f32(f32_to_bf16_bits(q))
    q = q.astype(np.float64)
    qh = q / np.linalg.norm(q)
    u = _rng(wl.wid, TAG_NEEDLE, 1000 + idx).standard_normal(wl.d)
    u -= (u @ qh) * qh
    u /= np.linalg.norm(u)
    k = np.linalg.norm(k_orig.astype(np.float64)) * (0.9 * qh + math.sqrt(0.19) * u)
    return k.astype(np.float32)


# ----------------------------------------------------------------------------- prefill API

def chunk_inputs(wl: Workload, k: int, seq: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Inputs of chunk k of sequence `seq`: Q_c [H_q][C][d], K_c, V_c [H_kv][C][d].

    Returned as uint16 bf16 bits (bf16 workloads) or fp32.  The last chunk is
    shorter when C does not divide L.
    """
    T = k * wl.C
    n = min(wl.C, wl.L - T) if wl.L else wl.C
    Q = np.stack([_q_rows_f32(wl, h, seq, T, n) for h in range(wl.H_q)])
    K = np.stack([_k_rows_f32(wl, g, seq, T, n) for g in range(wl.H_kv)])
    V = np.stack([_v_rows_f32(wl, g, seq, T, n) for g in range(wl.H_kv)])
    for j, nd in enumerate(needles(wl)):
        if seq == 0 and T <= nd.pos < T + n:
            g = nd.head // wl.G
            K[g, nd.pos - T] = _needle_key(wl, nd, K[g, nd.pos - T], j)
    return _finish(Q, wl.dtype), _finish(K, wl.dtype), _finish(V, wl.dtype)


def chunk_lengths(wl: Workload) -> List[int]:
    return [min(wl.C, wl.L - k * wl.C) for k in range(wl.n_chunks)]


# ----------------------------------------------------------------------------- decode API

@dataclasses.dataclass
class DecodeInputs:
    prior_len: np.ndarray          # [batch] int64, T_b
    q: np.ndarray                  # [batch][H_q][1][d]
    k_new: np.ndarray              # [batch][H_kv][1][d] (key of the token at position T_b)
    v_new: np.ndarray
    block_table: np.ndarray        # [batch][max_blocks] int32 (physical block ids; -1 unused)
    k_pool: np.ndarray             # [num_blocks][H_kv][block][d] (prior tokens filled, rest 0)
    v_pool: np.ndarray
    # consecutive steps (decode_inputs(..., steps=S)): step t is the token at
    # position T_b + t; step 0 is q / k_new / v_new above
    q_steps: Optional[np.ndarray] = None       # [S][batch][H_q][1][d]
    k_steps: Optional[np.ndarray] = None       # [S][batch][H_kv][1][d]
    v_steps: Optional[np.ndarray] = None

    def logical_kv(self, b: int, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
        """Prior K, V of sequence b as [H_kv][T_b][d] read back from the pool (layout helper)."""
        T = int(self.prior_len[b])
        nb = (T + block_size - 1) // block_size
        ids = self.block_table[b, :nb]
        k = self.k_pool[ids].transpose(1, 0, 2, 3).reshape(self.k_pool.shape[1], nb * block_size, -1)[:, :T]
        v = self.v_pool[ids].transpose(1, 0, 2, 3).reshape(self.v_pool.shape[1], nb * block_size, -1)[:, :T]
        return k, v


def decode_lengths(wl: Workload) -> np.ndarray:
    return _rng(wl.wid, TAG_LEN).integers(wl.decode_len_lo, wl.decode_len_hi + 1, size=wl.batch).astype(np.int64)


def decode_inputs(wl: Workload, lengths: Optional[np.ndarray] = None, steps: int = 1) -> DecodeInputs:
    """Ragged decode step: sequence b has T_b prior tokens in a paged pool and one new token at T_b.
    With steps = S the pool has room for S new tokens per sequence and q_steps / k_steps /
    v_steps hold the generator's tokens at positions T_b .. T_b + S - 1 (consecutive steps)."""
    bs = wl.block_size
    lens = decode_lengths(wl) if lengths is None else np.asarray(lengths, dtype=np.int64)
    batch = len(lens)
    nblk = [(int(t) + steps + bs - 1) // bs for t in lens]      # room for the new tokens too
    total = int(sum(nblk))
    perm = _rng(wl.wid, TAG_PERM).permutation(total).astype(np.int32)
    maxb = max(nblk)
    table = np.full((batch, maxb), -1, dtype=np.int32)
    pos = 0
    for b in range(batch):
        table[b, : nblk[b]] = perm[pos: pos + nblk[b]]
        pos += nblk[b]
    store = np.uint16 if wl.dtype == "bf16" else np.float32
    k_pool = np.zeros((total, wl.H_kv, bs, wl.d), dtype=store)
    v_pool = np.zeros((total, wl.H_kv, bs, wl.d), dtype=store)
    q_s = np.empty((steps, batch, wl.H_q, 1, wl.d), dtype=store)
    k_s = np.empty((steps, batch, wl.H_kv, 1, wl.d), dtype=store)
    v_s = np.empty((steps, batch, wl.H_kv, 1, wl.d), dtype=store)
    for b in range(batch):
        T = int(lens[b])
        for g in range(wl.H_kv):
            kk = _finish(_k_rows_f32(wl, g, b, 0, T + steps), wl.dtype)
            vv = _finish(_v_rows_f32(wl, g, b, 0, T + steps), wl.dtype)
            padded = nblk[b] * bs
            kp = np.zeros((padded, wl.d), dtype=store)
            vp = np.zeros((padded, wl.d), dtype=store)
            kp[:T] = kk[:T]
            vp[:T] = vv[:T]
            k_pool[table[b, : nblk[b]], g] = kp.reshape(nblk[b], bs, wl.d)
            v_pool[table[b, : nblk[b]], g] = vp.reshape(nblk[b], bs, wl.d)
            k_s[:, b, g, 0] = kk[T:T + steps]
            v_s[:, b, g, 0] = vv[T:T + steps]
        for h in range(wl.H_q):
            q_s[:, b, h, 0] = _finish(_q_rows_f32(wl, h, b, T, steps), wl.dtype)
    return DecodeInputs(lens, q_s[0].copy(), k_s[0].copy(), v_s[0].copy(), table, k_pool, v_pool,
                        q_s if steps > 1 else None, k_s if steps > 1 else None, v_s if steps > 1 else None)


def describe(wl: Workload) -> dict:
    return {k: v for k, v in dataclasses.asdict(wl).items() if v not in (0, None) or k in ("L", "C")}
