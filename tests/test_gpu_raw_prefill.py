"""kda_chunk_fwd_raw (raw projections in: short convolution, SiLU, L2 input norms and gate
activations fused into the prep pass) against the fp64 oracle's token stage plus recurrence."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import kda_oracle as ko
from kda_testutil import np64, to_dev

# The raw-projection prefill once read q and k rows past the end of a ragged last chunk and
# faulted the GPU; tests/test_raw_addressing.py replays every access of its kernels on the CPU.
pytestmark = pytest.mark.gpu

# The bf16 bar of the other prefill paths: max |err| <= 2e-2 x RMS(ref), on o and on the final
# state. The raw path's outputs are heavier-tailed (max |o| reaches 17-33 x RMS, against 11-13
# x for the workloads': the convolved, SiLU-activated keys share a positive direction), which
# is what the pair operands of M's off-diagonal blocks are for.
TOL = 2e-2


def _errs(got, ref):
    """(max |err| / max |ref|, RMS(err) / RMS(ref), max |err| / RMS(ref))."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = got - ref
    rms = np.sqrt(np.mean(ref * ref))
    return (np.abs(err).max() / np.abs(ref).max(), np.sqrt(np.mean(err * err)) / rms,
            np.abs(err).max() / rms)


def _run(inp, varlen, act=1, scale=1.0):
    d = to_dev(inp)
    o, ht, tail = kda.chunk_fwd_raw(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"],
                                    conv_tail=d["conv_tail"], h0=d["h0"],
                                    cu_seqlens=d["cu_seqlens"] if varlen else None,
                                    act=act, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return o, ht, tail


def _oracle(inp, varlen, act=1, scale=1.0):
    return ko.prefill_raw_fwd(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["g"]),
                              np64(inp["beta"]), np64(inp["conv_w"]),
                              conv_tail=np64(inp["conv_tail"]), h0=np64(inp["h0"]),
                              cu_seqlens=inp["cu_seqlens"].numpy() if varlen else None,
                              scale=scale, act=act)


@pytest.mark.parametrize("T,H,dk,W,act", [(1000, 3, 128, 4, 1), (300, 2, 64, 4, 0),
                                          (130, 2, 128, 2, 1), (200, 2, 128, 1, 1)])
def test_raw_prefill_matches_oracle(T, H, dk, W, act):
    print(f"case raw prefill T={T} H={H} dk={dk} W={W} act={act}", flush=True)
    inp = wl.raw_prefill_inputs(T=T, H=H, dk=dk, dv=dk, conv_width=W, seed=T + W, h0_std=0.02)
    o, ht, tail = _run(inp, False, act=act, scale=0.9)
    o_ref, ht_ref, tail_ref = _oracle(inp, False, act=act, scale=0.9)
    eo, es = _errs(np64(o), o_ref), _errs(np64(ht), ht_ref)
    print(f"o: max/max {eo[0]:.2e} rms/rms {eo[1]:.2e} max/rms {eo[2]:.2e} (tail "
          f"{np.abs(o_ref).max() / np.sqrt(np.mean(o_ref ** 2)):.1f}); state: {es[0]:.2e} "
          f"{es[1]:.2e} {es[2]:.2e}")
    assert eo[2] <= TOL and es[2] <= TOL
    if W > 1:
        # the leaving tail holds raw inputs: exact
        assert np.array_equal(np64(tail), tail_ref)


@pytest.mark.parametrize("dk,W", [(128, 4), (64, 3)])
def test_raw_prefill_varlen_and_short_sequences(dk, W):
    """Packed sequences, some shorter than the convolution tail (their leaving tail keeps
    shifted entries of the entering one) and one empty (its tail passes through)."""
    lengths = [1, 2, 64, 65, 0, 300, 3, 129]
    print(f"case raw prefill varlen dk={dk} W={W} lengths={lengths}", flush=True)
    inp = wl.raw_prefill_inputs(H=2, dk=dk, dv=dk, conv_width=W, seed=80 + W, h0_std=0.02,
                                lengths=lengths)
    o, ht, tail = _run(inp, True)
    o_ref, ht_ref, tail_ref = _oracle(inp, True)
    eo, es = _errs(np64(o), o_ref), _errs(np64(ht), ht_ref)
    print(f"o: max/max {eo[0]:.2e} rms/rms {eo[1]:.2e} max/rms {eo[2]:.2e} (tail "
          f"{np.abs(o_ref).max() / np.sqrt(np.mean(o_ref ** 2)):.1f}); state: {es[0]:.2e} "
          f"{es[1]:.2e} {es[2]:.2e}")
    assert np.array_equal(np64(tail), tail_ref)
    assert eo[2] <= TOL and es[2] <= TOL


def test_raw_prefill_without_entering_tail():
    print("case raw prefill T=200 H=2 dk=128 W=4 without entering tail", flush=True)
    inp = wl.raw_prefill_inputs(T=200, H=2, dk=128, dv=128, conv_width=4, seed=88,
                                with_tail=False)
    o, ht, tail = _run(inp, False)
    o_ref, ht_ref, tail_ref = _oracle(inp, False)
    for e in (_errs(np64(o), o_ref), _errs(np64(ht), ht_ref)):
        assert e[2] <= TOL
    assert np.array_equal(np64(tail), tail_ref)


@pytest.mark.parametrize("dk", [64, 128])
def test_raw_grouped_sequences_bit_identical(dk):
    """A workspace smaller than the whole batch needs (here the least it accepts: the longest
    sequence's convolved values and slots) runs groups of whole sequences: the same bits as
    the whole batch at once, outputs, final states and leaving tails included."""
    lengths = [300, 0, 640, 129, 1024, 64, 1, 500]
    print(f"case raw grouped sequences dk={dk} lengths={lengths}", flush=True)
    inp = wl.raw_prefill_inputs(lengths=lengths, H=3, dk=dk, dv=dk, conv_width=4, seed=61 + dk,
                                h0_std=0.02)
    d = to_dev(inp)
    need_min = kda.chunk_fwd_raw_workspace_size(1, max(lengths), 1, 3, dk, dk)
    need_all = kda.chunk_fwd_raw_workspace_size(1, sum(lengths), len(lengths), 3, dk, dk)
    assert need_min < need_all
    res = []
    for nbytes in (need_all, need_min):
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
        res.append(kda.chunk_fwd_raw(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"],
                                     conv_tail=d["conv_tail"], h0=d["h0"],
                                     cu_seqlens=d["cu_seqlens"], out_dtype=torch.float32,
                                     workspace=ws))
        torch.cuda.synchronize()
    for a, b, name in zip(res[0], res[1], ("o", "ht", "tail_out")):
        assert torch.equal(a, b), name
    with pytest.raises(kda.KDAError) as ei:
        kda.chunk_fwd_raw(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"],
                          conv_tail=d["conv_tail"], h0=d["h0"], cu_seqlens=d["cu_seqlens"],
                          workspace=torch.empty(need_min - 16, dtype=torch.uint8,
                                                device="cuda"))
    assert ei.value.status == -6
