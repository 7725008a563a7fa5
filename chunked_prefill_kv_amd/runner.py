"""Drivers that keep a workload's tensors resident on the GPU and issue the
C-ABI calls: the chunk loop of a whole prompt (chunked prefill) and one ragged
paged decode step.  Marshalling only - every step runs in the HIP kernels.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from . import gen
from . import kvsel as K


def to_device(x: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bits -> torch.bfloat16, fp32 -> torch.float32, int -> same (no value changes)."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Inverse of to_device for bf16 (bit patterns as uint16) and fp32."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class PromptRunner:
    """Chunked prefill of one prompt (batch 1) with a contiguous KV cache of capacity L."""

    def __init__(self, wl: gen.Workload, device="cuda", out_dtype=torch.bfloat16, pooling: int = K.KVSEL_POOL_HEAD):
        self.wl = wl
        self.device = device
        self.dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.out_dtype = out_dtype
        self.lens = gen.chunk_lengths(wl)
        self.starts = [k * wl.C for k in range(len(self.lens))]
        self.kc = torch.zeros(1, wl.H_kv, wl.L, wl.d, dtype=self.dt, device=device)
        self.vc = torch.zeros_like(self.kc)
        self.h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16 if wl.dtype == "bf16" else K.KVSEL_F32)
        self.p = K.Params(wl.n_q, wl.B, pooling)
        self.cache = K.cache(self.kc, self.vc, wl.L)
        self.prior = torch.tensor(self.starts, dtype=torch.int64, device=device)
        self.batches = [K.batch([t], c, self.prior[i:i + 1]) for i, (t, c) in enumerate(zip(self.starts, self.lens))]
        ws = max(K.workspace_size(self.h, b, self.p) for b in self.batches)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=device)
        self.chunks: List[tuple] = []
        self.outs: List[torch.Tensor] = []
        self.idx: List[Optional[torch.Tensor]] = []

    def load(self, chunks: Optional[Sequence[tuple]] = None, keep_idx: bool = False) -> None:
        """Upload every chunk's (Q_c, K_c, V_c) (generated if not given) and allocate outputs."""
        wl = self.wl
        self.chunks = []
        for k in range(len(self.lens)):
            c = chunks[k] if chunks is not None else gen.chunk_inputs(wl, k)
            self.chunks.append(tuple(to_device(x[None], self.device) for x in c))
        self.outs = [torch.empty(1, wl.H_q, c, wl.d, dtype=self.out_dtype, device=self.device) for c in self.lens]
        self.idx = [torch.empty(1, wl.H_kv, wl.B, dtype=torch.int32, device=self.device) if keep_idx else None
                    for _ in self.lens]

    def reset(self) -> None:
        """Forget the cache contents (the next run starts from T = 0)."""
        self.kc.zero_()
        self.vc.zero_()

    def run_chunk(self, k: int) -> None:
        q, kc, vc = self.chunks[k]
        K.kvsel_prefill_chunk(self.h, self.batches[k], self.p, q, kc, vc, self.cache, self.outs[k], self.idx[k],
                              self.ws)

    def run(self) -> None:
        for k in range(len(self.lens)):
            self.run_chunk(k)


class DecodeRunner:
    """One ragged decode step (chunk of 1 per sequence) over a paged KV cache."""

    def __init__(self, wl: gen.Workload, inputs: gen.DecodeInputs, device="cuda", out_dtype=torch.bfloat16,
                 pooling: int = K.KVSEL_POOL_HEAD):
        self.wl = wl
        self.inp = inputs
        self.device = device
        bs = wl.block_size
        self.k_pool = to_device(inputs.k_pool, device)
        self.v_pool = to_device(inputs.v_pool, device)
        self.k_pool0 = None
        self.table = to_device(inputs.block_table, device)
        self.q = to_device(inputs.q, device)
        self.k_new = to_device(inputs.k_new, device)
        self.v_new = to_device(inputs.v_new, device)
        self.prior = to_device(inputs.prior_len, device)
        self.h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16 if wl.dtype == "bf16" else K.KVSEL_F32)
        self.p = K.Params(wl.n_q, wl.B, pooling)
        self.b = K.batch(inputs.prior_len.tolist(), 1, self.prior)
        self.cache = K.cache(self.k_pool, self.v_pool, self.k_pool.shape[0], bs, self.table)
        self.ws = torch.empty(K.workspace_size(self.h, self.b, self.p), dtype=torch.uint8, device=device)
        self.out = torch.empty(len(inputs.prior_len), wl.H_q, 1, wl.d, dtype=out_dtype, device=device)
        self.idx = torch.empty(len(inputs.prior_len), wl.H_kv, wl.B, dtype=torch.int32, device=device)

    def run(self) -> None:
        K.kvsel_prefill_chunk(self.h, self.b, self.p, self.q, self.k_new, self.v_new, self.cache, self.out,
                              self.idx, self.ws)


class DecodeStepsRunner:
    """Consecutive decode steps of a ragged paged batch (step t: the token at T_b + t),
    either plain (kvsel_prefill_chunk) or with the selected-entry cache
    (kvsel_decode_reuse).  `inputs` must come from gen.decode_inputs(..., steps=S)."""

    def __init__(self, wl: gen.Workload, inputs: gen.DecodeInputs, device="cuda", out_dtype=torch.bfloat16):
        assert inputs.q_steps is not None, "decode_inputs(..., steps=S) with S > 1"
        self.wl = wl
        self.S = inputs.q_steps.shape[0]
        self.device = device
        self.k_pool = to_device(inputs.k_pool, device)
        self.v_pool = to_device(inputs.v_pool, device)
        self.table = to_device(inputs.block_table, device)
        self.q = [to_device(x, device) for x in inputs.q_steps]
        self.k_new = [to_device(x, device) for x in inputs.k_steps]
        self.v_new = [to_device(x, device) for x in inputs.v_steps]
        self.h = K.heads(wl.H_q, wl.H_kv, wl.d, K.KVSEL_BF16)
        self.p = K.Params(wl.n_q, wl.B)
        T0 = inputs.prior_len.astype(np.int64)
        self.prior = [torch.tensor(T0 + t, dtype=torch.int64, device=device) for t in range(self.S)]
        self.batches = [K.batch((T0 + t).tolist(), 1, self.prior[t]) for t in range(self.S)]
        self.cache = K.cache(self.k_pool, self.v_pool, self.k_pool.shape[0], wl.block_size, self.table)
        self.ws = torch.empty(max(K.workspace_size(self.h, b, self.p) for b in self.batches), dtype=torch.uint8,
                              device=device)
        nb = len(T0)
        self.out = torch.empty(nb, wl.H_q, 1, wl.d, dtype=out_dtype, device=device)
        self.idx = torch.empty(nb, wl.H_kv, wl.B, dtype=torch.int32, device=device)
        self.sel_k = torch.empty(nb, wl.H_kv, wl.B, wl.d, dtype=torch.bfloat16, device=device)
        self.sel_v = torch.empty_like(self.sel_k)
        self.pos = torch.full((nb, wl.H_kv, wl.B), -1, dtype=torch.int32, device=device)
        self.counts = torch.zeros(nb, wl.H_kv, 2, dtype=torch.int32, device=device)
        self.sel = K.sel_cache(self.sel_k, self.sel_v, self.pos, self.counts)

    def reset(self) -> None:
        """Empty the selected-entry cache (a new sequence per batch entry)."""
        self.pos.fill_(-1)

    def step(self, t: int, reuse: bool) -> None:
        if reuse:
            K.kvsel_decode_reuse(self.h, self.batches[t], self.p, self.q[t], self.k_new[t], self.v_new[t], self.cache,
                                 self.sel, self.out, self.idx, self.ws)
        else:
            K.kvsel_prefill_chunk(self.h, self.batches[t], self.p, self.q[t], self.k_new[t], self.v_new[t],
                                  self.cache, self.out, self.idx, self.ws)
