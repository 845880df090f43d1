"""kda_chunk_bwd (HIP) against the oracle's backward (recurrence_bwd: the chain rule applied
to the per-token definition, pinned in test_oracle_backward.py by central differences),
element by element, for all six gradients."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import kda_oracle as ko
from kda_testutil import TOL_BF16, TOL_F32, np64, rel_max_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _grads_vs_oracle(inp, do, dht, varlen, scale=1.0):
    d = to_dev(inp)
    cu = d["cu_seqlens"] if varlen else None
    got = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do.cuda(),
                        dht=None if dht is None else dht.cuda(), h0=d["h0"], cu_seqlens=cu,
                        scale=scale)
    torch.cuda.synchronize()
    ref = ko.recurrence_bwd(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["g"]),
                            np64(inp["beta"]), np64(do), dht=np64(dht), h0=np64(inp["h0"]),
                            cu_seqlens=inp["cu_seqlens"].numpy() if varlen else None,
                            scale=scale)
    return {n: rel_max_err(np64(got[n]), ref[n]) for n in NAMES}, got


def test_backward_tiny_f32_config():
    """The tiny fp32 configuration (T=256, H=2, d=64, seed 0) with random output and
    final-state gradients, at the fp32 bar of 1e-4 x RMS on every gradient."""
    cfg = wl.CONFIGS["tiny_f32"]
    print(f"case backward tiny_f32 T={cfg['T']} H={cfg['H']} d={cfg['dk']}", flush=True)
    inp = wl.prefill_inputs(T=cfg["T"], H=cfg["H"], dk=cfg["dk"], dv=cfg["dv"], dtype="f32",
                            seed=cfg["seed"], h0_std=0.0)
    gen = torch.Generator().manual_seed(11)
    do = torch.randn(cfg["T"], cfg["H"], cfg["dv"], generator=gen)
    dht = torch.randn(1, cfg["H"], cfg["dk"], cfg["dv"], generator=gen)
    errs, _ = _grads_vs_oracle(inp, do, dht, varlen=False)
    print(" ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL_F32, n


@pytest.mark.parametrize("dk", [128, 64])
def test_backward_bf16_varlen_with_h0(dk):
    """1024 tokens x 4 heads in ragged packed sequences (one empty, one of a single token),
    bf16 inputs, h0 per sequence, scale 0.8: the bf16 bar of 2e-2 x RMS."""
    lengths = [300, 1, 0, 523, 200]
    assert sum(lengths) == 1024
    print(f"case backward bf16 varlen dk={dk} lengths={lengths}", flush=True)
    inp = wl.prefill_inputs(H=4, dk=dk, dv=dk, dtype="bf16", seed=40 + dk, h0_std=0.02,
                            lengths=lengths)
    gen = torch.Generator().manual_seed(12)
    do = torch.randn(1024, 4, dk, generator=gen).to(torch.bfloat16)
    dht = torch.randn(len(lengths), 4, dk, dk, generator=gen)
    errs, got = _grads_vs_oracle(inp, do, dht, varlen=True, scale=0.8)
    print(" ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL_BF16, n
    # the empty sequence passes its final-state gradient through
    assert torch.equal(got["dh0"][2].cpu(), dht[2])


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_backward_pairs_of_chunks(dtype, dk):
    """Sequences whose last 16-token chunk is odd (full, or ragged down to one token) or even:
    the gradient pass rebuilds the state of one chunk of each pair from its neighbour (an odd
    chunk's entering state from the chunk before, an even chunk's leaving-state gradient from
    the chunk after, also where that one is a ragged last chunk)."""
    lengths = [20, 50, 32, 17, 16, 33, 111]
    T = sum(lengths)
    print(f"case backward pairs {dtype} dk={dk} lengths={lengths}", flush=True)
    inp = wl.prefill_inputs(H=3, dk=dk, dv=dk, dtype=dtype, seed=60 + dk, h0_std=0.02,
                            lengths=lengths)
    gen = torch.Generator().manual_seed(14)
    do = torch.randn(T, 3, dk, generator=gen)
    if dtype == "bf16":
        do = do.to(torch.bfloat16)
    dht = torch.randn(len(lengths), 3, dk, dk, generator=gen)
    errs, _ = _grads_vs_oracle(inp, do, dht, varlen=True, scale=0.9)
    print(" ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for n, e in errs.items():
        assert e <= tol, n


def test_backward_floor_and_determinism():
    """Raw g x 10 (the floor at -5 bites on part of the channels, where dg must be exactly 0),
    no final-state gradient, fp32; two calls give the same bits."""
    print("case backward floor stress T=150 H=2 d=128 f32", flush=True)
    inp = wl.prefill_inputs(T=150, H=2, dk=128, dv=128, dtype="f32", seed=9, h0_std=0.02,
                            floor_stress=True)
    g = inp["g"]
    assert (g < -5.0).any() and (g > -5.0).any()
    gen = torch.Generator().manual_seed(13)
    do = torch.randn(150, 2, 128, generator=gen)
    errs, got = _grads_vs_oracle(inp, do, None, varlen=False)
    print(" ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL_F32, n
    floored = (g <= -5.0)
    assert torch.all(got["dg"].cpu()[floored] == 0)
    _, again = _grads_vs_oracle(inp, do, None, varlen=False)
    for n in NAMES:
        assert torch.equal(got[n], again[n]), n
