"""Seeded synthetic workloads for the KDA entry points.

This module draws inputs only: it holds none of the recurrence's arithmetic and imports
nothing from the library or from the CPU oracle, so both sides can share it. Every tensor is
drawn in float32 from one seeded ``torch.Generator`` in a fixed order, transformed in float32
into the configuration's distribution, then cast to the device dtype (round to nearest even
for bf16). The oracle receives exact upcasts of the same bits.

Shapes follow the workloads the pages describe: 96 heads with head dimension 128 (Kimi K3's
KDA layers), 12 heads per GPU for an 8-way tensor-parallel share, long prefills, a draft
window of 7 plus one bonus token.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = ["CONFIGS", "prefill_inputs", "raw_prefill_inputs", "varlen_lengths", "decode_inputs",
           "DecodeWorkload"]


# name -> parameters. "kind" tells which entry point the configuration exercises.
CONFIGS = {
    # fp32 parity case small enough for the per-token oracle in seconds
    "tiny_f32": dict(kind="prefill", T=256, H=2, dk=64, dv=64, dtype="f32", h0_std=0.0, seed=0),
    # long prefill over all 96 heads of one layer, bf16 inputs, restored fp32 state
    "prefill_8k": dict(kind="prefill", T=8192, H=96, dk=128, dv=128, dtype="bf16", h0_std=0.02,
                       seed=1),
    # ultra-long prefill over one GPU's 12-head share: segment-parallel entry point
    "ultralong_256k": dict(kind="segment", T=262144, H=12, dk=128, dv=128, dtype="bf16",
                           h0_std=0.0, seed=2),
    # 64 packed sequences, lengths uniform in [512, 16384], per-sequence restored state
    "varlen_64": dict(kind="prefill", n_seqs=64, len_lo=512, len_hi=16384, H=96, dk=128, dv=128,
                      dtype="bf16", h0_std=0.02, seed=3),
    # speculative verify: 256 requests, 96 heads, window of 7 drafts + 1 bonus, conv width 4
    "decode_verify": dict(kind="decode", R=256, H=96, dk=128, dv=128, conv_width=4, n_new=8,
                          window=8, seed=4),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(x):
    # uniform direction on the sphere: a normal draw divided by its length (per token, head)
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def varlen_lengths(n_seqs, lo, hi, seed):
    """Sequence lengths uniform in [lo, hi] (inclusive), drawn on the CPU."""
    g = _gen(seed * 7919 + 17, "cpu")
    return torch.randint(lo, hi + 1, (n_seqs,), generator=g, dtype=torch.int64).tolist()


def prefill_inputs(T=None, H=2, dk=64, dv=64, dtype="f32", seed=0, h0_std=0.0, lengths=None,
                   device="cpu", floor_stress=False, g_fill=None, beta_fill=None):
    """Inputs for the chunked prefill.

    q, k ~ N(0, 1) scaled to unit length per (token, head); v ~ N(0, 1);
    beta = sigmoid(N(0, 1)); g = max(-softplus(N(0, 1)), -5) (with ``floor_stress`` the
    normal draw is multiplied by 10 and the floor is NOT applied here, so the kernel's floor
    is exercised); h0 ~ N(0, h0_std^2) per sequence and head (None when h0_std == 0).
    ``lengths`` packs several sequences (cu_seqlens), otherwise one sequence of T tokens.
    ``g_fill`` / ``beta_fill`` replace g / beta by a constant (special-case tests).
    Returns a dict of tensors on ``device`` plus 'cu_seqlens' (int32, CPU) and 'lengths'.
    """
    if lengths is None:
        lengths = [int(T)]
    lengths = [int(x) for x in lengths]
    total = sum(lengths)
    gen = _gen(seed, device)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    q = _unit_rows(torch.randn(total, H, dk, **f32))
    k = _unit_rows(torch.randn(total, H, dk, **f32))
    v = torch.randn(total, H, dv, **f32)
    g_raw = torch.randn(total, H, dk, **f32)
    if floor_stress:
        g = -torch.nn.functional.softplus(10.0 * g_raw)
    else:
        g = torch.clamp(-torch.nn.functional.softplus(g_raw), min=-5.0)
    beta = torch.sigmoid(torch.randn(total, H, **f32))
    h0 = None
    if h0_std > 0:
        h0 = h0_std * torch.randn(len(lengths), H, dk, dv, **f32)
    if g_fill is not None:
        g = torch.full_like(g, float(g_fill))
    if beta_fill is not None:
        beta = torch.full_like(beta, float(beta_fill))
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    io = _DT[dtype]
    return dict(q=q.to(io), k=k.to(io), v=v.to(io), g=g.contiguous(), beta=beta.contiguous(),
                h0=h0, cu_seqlens=cu, lengths=lengths)


@dataclass
class DecodeWorkload:
    R: int
    H: int
    dk: int
    dv: int
    conv_width: int
    n_new: int
    window: int
    n_acc: torch.Tensor            # [R] int32
    prev: dict                     # raw projected inputs of the previous window
    new: dict                      # raw projected inputs of this window (with 'z')
    conv_w: torch.Tensor           # [H, 2 dk + dv, W] fp32
    norm_w: torch.Tensor           # [dv] fp32
    state: torch.Tensor            # [R, H, dk, dv] fp32
    conv_tail: torch.Tensor        # [R, H, 2 dk + dv, W - 1] fp32
    extra: dict = field(default_factory=dict)


def decode_inputs(R=256, H=96, dk=128, dv=128, conv_width=4, n_new=8, window=8, seed=4,
                  device="cpu", max_acc: Optional[int] = None, n_acc_fill=None):
    """Speculative-verify inputs: raw q, k, v, g, beta, z ~ N(0, 1) in bf16 for both windows;
    conv taps 0.5 N(0, 1); RMSNorm weight 1 + 0.1 N(0, 1); committed state N(0, 0.02^2);
    conv tail N(0, 1); accepted drafts n_acc uniform in {0, ..., window - 1}."""
    gen = _gen(seed, device)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    C = 2 * dk + dv

    def window_tensors(slots, with_z):
        t = dict(q=torch.randn(R, slots, H, dk, **f32), k=torch.randn(R, slots, H, dk, **f32),
                 v=torch.randn(R, slots, H, dv, **f32), g=torch.randn(R, slots, H, dk, **f32),
                 beta=torch.randn(R, slots, H, **f32))
        t["z"] = torch.randn(R, slots, H, dv, **f32) if with_z else None
        return {n: (x.to(torch.bfloat16) if x is not None else None) for n, x in t.items()}

    prev = window_tensors(window, False)
    new = window_tensors(n_new, True)
    conv_w = 0.5 * torch.randn(H, C, conv_width, **f32)
    norm_w = 1.0 + 0.1 * torch.randn(dv, **f32)
    state = 0.02 * torch.randn(R, H, dk, dv, **f32)
    tail = torch.randn(R, H, C, conv_width - 1, **f32)
    hi = window - 1 if max_acc is None else max_acc
    n_acc = torch.randint(0, hi + 1, (R,), generator=gen, device=device, dtype=torch.int64)
    if n_acc_fill is not None:
        n_acc = torch.full_like(n_acc, int(n_acc_fill))
    return DecodeWorkload(R=R, H=H, dk=dk, dv=dv, conv_width=conv_width, n_new=n_new,
                          window=window, n_acc=n_acc.to(torch.int32), prev=prev, new=new,
                          conv_w=conv_w, norm_w=norm_w, state=state, conv_tail=tail)


def raw_prefill_inputs(T=None, H=2, dk=128, dv=128, conv_width=4, seed=0, h0_std=0.0,
                       lengths=None, with_tail=True, device="cpu"):
    """Raw projections for the prefill with the fused token stage, drawn like the decode's:
    q, k, v, g, beta ~ N(0, 1) in bf16; conv taps 0.5 N(0, 1); entering conv tails N(0, 1)
    (or none); h0 ~ N(0, h0_std^2) per sequence. Returns a dict with 'cu_seqlens' (CPU)."""
    if lengths is None:
        lengths = [int(T)]
    lengths = [int(x) for x in lengths]
    total = sum(lengths)
    gen = _gen(seed, device)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    bf = lambda *shape: torch.randn(*shape, **f32).to(torch.bfloat16)
    C = 2 * dk + dv
    out = dict(q=bf(total, H, dk), k=bf(total, H, dk), v=bf(total, H, dv), g=bf(total, H, dk),
               beta=bf(total, H))
    out["conv_w"] = 0.5 * torch.randn(H, C, conv_width, **f32)
    out["conv_tail"] = (torch.randn(len(lengths), H, C, conv_width - 1, **f32)
                        if with_tail and conv_width > 1 else None)
    out["h0"] = (h0_std * torch.randn(len(lengths), H, dk, dv, **f32) if h0_std > 0 else None)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    out["cu_seqlens"] = cu
    out["lengths"] = lengths
    return out
