"""Seeded synthetic inputs for the KDA prefill and decode workloads.

This module holds random draws only -- none of the method's arithmetic -- so
that the HIP path and the fp64 oracle can be fed the very same tensors.

Workloads (the head size dk = dv = 128 and the 128 x 128 state per head are
the ones the page "Kimi Delta Attention" reports in §05; the chunk size 64 is
the block size of the "Kimi Linear Guide" page's hardware-chunking section):

=============  =====  ====  =====================  ======  =====  ==========
name           N      H     tokens                 d       dtype  log-decay u
=============  =====  ====  =====================  ======  =====  ==========
tiny           1      1     256                    64      f32    U(-4, 0)
prefill_8k     1      32    8192                   128     bf16   U(-5, 0)
varlen_16      16     32    U_int[512, 32768] each 128     bf16   U(-5, 0)
long_1m        1      16    1,048,576              128     bf16   U(-8, -2)
decode_256     256    32    512 decode steps       128     bf16   U(-5, 0)
=============  =====  ====  =====================  ======  =====  ==========

Recipe (one ``torch.Generator`` per workload, seeded with the workload's seed,
draws taken in this order: lengths, q, k, v, log_alpha, beta, initial state):

* q, k: standard normal in fp32, divided by their L2 norm over the head
  dimension (per token and head), then cast to the input dtype;
* v: standard normal, cast;
* log_alpha: ``-exp(u)`` with u uniform in the workload's range, fp32;
* beta: ``sigmoid(standard normal)``, cast;
* initial state: ``0.02 * standard normal`` in fp32 (varlen and decode), or
  zeros; stored ``[N, H, dv, dk]``.

Large workloads are drawn on the GPU with a device generator; the oracle
then consumes host copies of those same tensors.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class KdaWorkload:
    name: str
    num_seqs: int
    heads: int
    dk: int
    dv: int
    dtype: str                 # "f32" or "bf16" for q, k, v, beta and o
    seq_len: int = 0           # fixed length of every sequence (prefill)
    len_range: tuple = ()      # (lo, hi) inclusive: varlen lengths
    u_range: tuple = (-5.0, 0.0)
    init_std: float = 0.0      # 0 -> zero initial state
    seed: int = 0
    decode_steps: int = 0      # > 0 -> a decode workload

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "KdaWorkload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": KdaWorkload("tiny", 1, 1, 64, 64, "f32", seq_len=256,
                        u_range=(-4.0, 0.0), seed=0),
    "prefill_8k": KdaWorkload("prefill_8k", 1, 32, 128, 128, "bf16", seq_len=8192,
                              u_range=(-5.0, 0.0), seed=1),
    "varlen_16": KdaWorkload("varlen_16", 16, 32, 128, 128, "bf16",
                             len_range=(512, 32768), u_range=(-5.0, 0.0),
                             init_std=0.02, seed=2),
    "long_1m": KdaWorkload("long_1m", 1, 16, 128, 128, "bf16", seq_len=1 << 20,
                           u_range=(-8.0, -2.0), seed=3),
    "decode_256": KdaWorkload("decode_256", 256, 32, 128, 128, "bf16",
                              u_range=(-5.0, 0.0), init_std=0.02, seed=4,
                              decode_steps=512),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(shape, g, device, dtype):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    return x.to(dtype)


def _token_tensors(wl: KdaWorkload, lead: tuple, g, device):
    """q, k, v, log_alpha, beta for a block of tokens with leading shape ``lead``."""
    dt = wl.torch_dtype
    H = wl.heads
    q = _unit_rows(lead + (H, wl.dk), g, device, dt)
    k = _unit_rows(lead + (H, wl.dk), g, device, dt)
    v = torch.randn(lead + (H, wl.dv), generator=g, device=device, dtype=torch.float32).to(dt)
    lo, hi = wl.u_range
    u = torch.rand(lead + (H, wl.dk), generator=g, device=device, dtype=torch.float32)
    log_alpha = -torch.exp(lo + (hi - lo) * u)
    beta = torch.sigmoid(torch.randn(lead + (H,), generator=g, device=device,
                                     dtype=torch.float32)).to(dt)
    return q, k, v, log_alpha, beta


def seq_lengths(wl: KdaWorkload, g=None, device="cpu") -> list:
    if wl.len_range:
        g = g if g is not None else _gen(device, wl.seed)
        lo, hi = wl.len_range
        return [int(x) for x in torch.randint(lo, hi + 1, (wl.num_seqs,), generator=g,
                                              device=device)]
    return [wl.seq_len] * wl.num_seqs


def prefill_inputs(wl: KdaWorkload, device="cpu") -> dict:
    """Packed varlen prefill inputs: q, k, v, log_alpha, beta, cu_seqlens (int32),
    init_state (or None), plus ``lengths``."""
    g = _gen(device, wl.seed)
    lengths = seq_lengths(wl, g, device)
    T = sum(lengths)
    q, k, v, log_alpha, beta = _token_tensors(wl, (T,), g, device)
    init = None
    if wl.init_std > 0:
        init = wl.init_std * torch.randn((wl.num_seqs, wl.heads, wl.dv, wl.dk), generator=g,
                                         device=device, dtype=torch.float32)
    cu = torch.zeros(wl.num_seqs + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta,
                cu_seqlens=cu.to(device), init_state=init, lengths=lengths)


def decode_inputs(wl: KdaWorkload, device="cpu", steps: int | None = None) -> dict:
    """Decode inputs: per-step q, k ``[S,N,H,dk]``, v ``[S,N,H,dv]``, log_alpha
    ``[S,N,H,dk]``, beta ``[S,N,H]`` and the initial state ``[N,H,dv,dk]``."""
    g = _gen(device, wl.seed)
    S = wl.decode_steps if steps is None else steps
    q, k, v, log_alpha, beta = _token_tensors(wl, (S, wl.num_seqs), g, device)
    if wl.init_std > 0:
        state = wl.init_std * torch.randn((wl.num_seqs, wl.heads, wl.dv, wl.dk), generator=g,
                                          device=device, dtype=torch.float32)
    else:
        state = torch.zeros((wl.num_seqs, wl.heads, wl.dv, wl.dk), device=device,
                            dtype=torch.float32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, state=state)
