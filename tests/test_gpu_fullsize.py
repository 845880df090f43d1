"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each test runs the entry point on the whole workload exactly as the benchmark does (bf16
output), runs it again with fp32 output, and checks:
  * the bf16 output is bit-for-bit the round-to-nearest-even of the fp32 output (so the timed
    launch carries the verified arithmetic);
  * the fp32 output and the final states match the fp64 oracle, element by element, on a
    sample of heads / sequences / requests the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import c_recurrence_fwd
from oracle import kda_oracle as ko
from kda_testutil import TOL_BF16, TOL_F32, np64, rel_max_err

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-5


def _host_heads(x, heads):
    return x[:, heads].detach().to("cpu", torch.float32).numpy()


def _check_rounding(o16, o32):
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o32.to(torch.bfloat16), o16)


def test_prefill_8k_full():
    cfg = wl.CONFIGS["prefill_8k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    print(f"case prefill_8k T={T} H={H} d={dk}", flush=True)
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dv, dtype=cfg["dtype"], seed=cfg["seed"],
                            h0_std=cfg["h0_std"], device="cuda")
    args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
    # the automatic path choice, as the benchmark calls it (two launches at this shape)
    o16, ht16 = kda.chunk_fwd(*args, h0=inp["h0"])
    o32, ht32 = kda.chunk_fwd(*args, h0=inp["h0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_rounding(o16, o32)
    assert torch.equal(ht16, ht32)
    # the one-launch path gives the same bits
    o1, ht1 = kda.chunk_fwd(*args, h0=inp["h0"], out_dtype=torch.float32, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o32) and torch.equal(ht1, ht32)
    del o1, ht1
    # every head (the threaded C oracle takes about a second for all 96)
    heads = list(range(H))
    o_ref, ht_ref = c_recurrence_fwd(*[_host_heads(x, heads) for x in args],
                                     h0=_host_heads(inp["h0"], heads))
    e_o = rel_max_err(_host_heads(o32, heads), o_ref)
    e_s = rel_max_err(_host_heads(ht32, heads), ht_ref)
    print(f"all {H} heads: err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_prefill_8k_full_f32():
    """The prefill_8k shape with fp32 inputs (the 16-token chunk form on fp32 matrix cores at
    d = 128), every head against the oracle at the fp32 bar."""
    cfg = wl.CONFIGS["prefill_8k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    print(f"case prefill_8k fp32 T={T} H={H} d={dk}", flush=True)
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dv, dtype="f32", seed=cfg["seed"],
                            h0_std=cfg["h0_std"], device="cuda")
    args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
    o32, ht32 = kda.chunk_fwd(*args, h0=inp["h0"])
    torch.cuda.synchronize()
    heads = list(range(H))
    o_ref, ht_ref = c_recurrence_fwd(*[_host_heads(x, heads) for x in args],
                                     h0=_host_heads(inp["h0"], heads))
    e_o = rel_max_err(_host_heads(o32, heads), o_ref)
    e_s = rel_max_err(_host_heads(ht32, heads), ht_ref)
    print(f"all {H} heads: err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_F32 and e_s <= TOL_F32


def test_backward_8k_full_sampled_heads():
    """kda_chunk_bwd on the backward leg's workload (8192 tokens x 96 heads, d = 128, bf16,
    the same seeded inputs, output and final-state gradients), every gradient of heads 0 and
    95 against the oracle's per-token backward (one head at a time: it keeps every token's
    state)."""
    cfg = wl.CONFIGS["prefill_8k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    print(f"case backward 8k full T={T} H={H} d={dk}", flush=True)
    dev = torch.device("cuda")
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dv, dtype=cfg["dtype"], seed=cfg["seed"],
                            h0_std=cfg["h0_std"], device=dev)
    gen = torch.Generator(device=dev).manual_seed(7)
    do = torch.randn(T, H, dv, device=dev, generator=gen).to(torch.bfloat16)
    dht = torch.randn(1, H, dk, dv, device=dev, generator=gen)
    args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
    got = kda.chunk_bwd(*args, do, dht=dht, h0=inp["h0"])
    torch.cuda.synchronize()
    for h in (0, H - 1):
        sl = [h]
        ref = ko.recurrence_bwd(*[_host_heads(x, sl) for x in args], _host_heads(do, sl),
                                dht=_host_heads(dht, sl), h0=_host_heads(inp["h0"], sl))
        for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
            e = rel_max_err(_host_heads(got[name], sl), ref[name])
            print(f"head {h} {name}: err {e:.3e}", flush=True)
            assert e <= TOL_BF16, (h, name)


_ULTRALONG = {}


def _ultralong_inputs_and_oracle(heads):
    """The ultralong workload on the device and the oracle on the sampled heads, computed
    once for the segment counts below."""
    if not _ULTRALONG:
        cfg = wl.CONFIGS["ultralong_256k"]
        inp = wl.prefill_inputs(T=cfg["T"], H=cfg["H"], dk=cfg["dk"], dv=cfg["dv"],
                                dtype=cfg["dtype"], seed=cfg["seed"], h0_std=cfg["h0_std"],
                                device="cuda")
        args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
        _ULTRALONG["args"] = args
        _ULTRALONG["ref"] = c_recurrence_fwd(*[_host_heads(x, heads) for x in args])
    return _ULTRALONG["args"], _ULTRALONG["ref"]


@pytest.mark.parametrize("n_segments", [0, 64, 256])
def test_ultralong_256k_segment_cp_full(n_segments):
    """T = 262144, H = 12 through the segment-parallel path: the automatic segment count (as
    the benchmark runs it) and the two ends of the 64..256 range of the workload."""
    cfg = wl.CONFIGS["ultralong_256k"]
    print(f"case ultralong_256k T={cfg['T']} H={cfg['H']} d={cfg['dk']} "
          f"n_segments={n_segments or 'automatic'}", flush=True)
    heads = list(range(cfg["H"]))   # every head
    args, (o_ref, ht_ref) = _ultralong_inputs_and_oracle(heads)
    o16, ht16 = kda.segment_cp_fwd(*args, n_segments=n_segments)
    o32, ht32 = kda.segment_cp_fwd(*args, n_segments=n_segments, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_rounding(o16, o32)
    assert torch.equal(ht16, ht32)
    e_o = rel_max_err(_host_heads(o32, heads), o_ref)
    e_s = rel_max_err(_host_heads(ht32, heads), ht_ref)
    print(f"all {len(heads)} heads: err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    del o16, o32
    torch.cuda.empty_cache()


def test_varlen_64_full():
    cfg = wl.CONFIGS["varlen_64"]
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    lengths = wl.varlen_lengths(cfg["n_seqs"], cfg["len_lo"], cfg["len_hi"], cfg["seed"])
    print(f"case varlen_64 {len(lengths)} sequences, {sum(lengths)} tokens, H={H}", flush=True)
    inp = wl.prefill_inputs(H=H, dk=dk, dv=dv, dtype=cfg["dtype"], seed=cfg["seed"],
                            h0_std=cfg["h0_std"], lengths=lengths, device="cuda")
    args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
    cu = inp["cu_seqlens"]
    o32, ht32 = kda.chunk_fwd(*args, h0=inp["h0"], cu_seqlens=cu, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cu_h = cu.tolist()
    # the first and the last sequence, the shortest and the longest, and four in between;
    # 13 heads each (every eighth and the last)
    order = np.argsort(lengths)
    n_s = len(lengths)
    seqs = sorted({0, n_s - 1, int(order[0]), int(order[-1]), int(order[n_s // 2]), 7, 21, 42})
    assert len(seqs) >= 8
    heads = list(range(0, H, 8)) + [H - 1]
    for n in seqs:
        a, b = cu_h[n], cu_h[n + 1]
        sl = [x[a:b] for x in args]
        o_ref, ht_ref = c_recurrence_fwd(*[_host_heads(x, heads) for x in sl],
                                         h0=_host_heads(inp["h0"][n:n + 1], heads))
        e_o = rel_max_err(_host_heads(o32[a:b], heads), o_ref)
        e_s = rel_max_err(_host_heads(ht32[n:n + 1], heads), ht_ref)
        print(f"seq {n} (length {b - a}) heads {heads}: err_o={e_o:.3e} err_state={e_s:.3e}")
        assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    del o32
    torch.cuda.empty_cache()
    o16, ht16 = kda.chunk_fwd(*args, h0=inp["h0"], cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(ht16, ht32)


def test_decode_verify_full():
    cfg = wl.CONFIGS["decode_verify"]
    R, H, D, W, n_new = cfg["R"], cfg["H"], cfg["dk"], cfg["conv_width"], cfg["n_new"]
    print(f"case decode_verify R={R} H={H} d={D}", flush=True)
    w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, conv_width=W, n_new=n_new, window=cfg["window"],
                         seed=cfg["seed"], device="cuda")
    outs = {}
    for odt in (torch.bfloat16, torch.float32):
        state, tail = w.state.clone(), w.conv_tail.clone()
        o, acc = kda.decode_replay(state, tail, w.n_acc, w.prev, w.new, w.conv_w, w.norm_w,
                                   out_dtype=odt)
        torch.cuda.synchronize()
        outs[odt] = (o, state, acc, tail)
    o16, s16, a16, t16 = outs[torch.bfloat16]
    o32, s32, a32, t32 = outs[torch.float32]
    _check_rounding(o16, o32)
    assert torch.equal(s16, s32) and torch.equal(a16, a32) and torch.equal(t16, t32)
    n_acc = w.n_acc.cpu()
    # requests with no, some and all accepted drafts: the fewest and the most, and every
    # seventeenth request (16 or more in all, the first and the last included)
    rs = sorted({int(torch.argmin(n_acc)), int(torch.argmax(n_acc)), R - 1,
                 *range(0, R, 17)})
    assert len(rs) >= 16
    host = lambda x: None if x is None else x[rs].double().cpu().numpy()
    ref = ko.decode_replay(host(w.state), host(w.conv_tail), n_acc[rs].numpy(),
                           {k: host(v) for k, v in w.prev.items()},
                           {k: host(v) for k, v in w.new.items()},
                           w.conv_w.double().cpu().numpy(), w.norm_w.double().cpu().numpy())
    e_state = np.abs(np64(s32[rs]) - ref["state"]).max()
    e_acc = np.abs(np64(a32[rs]) - ref["state_acc"]).max()
    e_tail = np.abs(np64(t32[rs]) - ref["conv_tail"]).max()
    e_o = rel_max_err(np64(o32[rs]), ref["o"])
    print(f"requests {rs} (n_acc {n_acc[rs].tolist()}): err_state={e_state:.2e} "
          f"err_acc={e_acc:.2e} err_tail={e_tail:.2e} err_o={e_o:.2e}")
    assert e_state <= STATE_TOL and e_acc <= STATE_TOL and e_tail <= STATE_TOL
    assert e_o <= TOL_BF16
