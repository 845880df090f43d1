"""Parity of kda_segment_cp_fwd (HIP, through the C ABI) with the fp64 CPU oracle and with
kda_chunk_fwd."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import c_recurrence_fwd
from kda_testutil import TOL_BF16, TOL_F32, np64, rel_max_err, to_dev

pytestmark = pytest.mark.gpu


def _oracle(inp, varlen, scale=1.0):
    cu = inp["cu_seqlens"].numpy() if varlen else None
    return c_recurrence_fwd(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["g"]),
                            np64(inp["beta"]), h0=np64(inp["h0"]), cu_seqlens=cu, scale=scale)


def _seg(inp, n_seg, varlen=False, out_dtype=torch.float32, scale=1.0):
    d = to_dev(inp)
    o, ht = kda.segment_cp_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"],
                               cu_seqlens=d["cu_seqlens"] if varlen else None,
                               n_segments=n_seg, out_dtype=out_dtype, scale=scale)
    torch.cuda.synchronize()
    return o, ht


@pytest.mark.parametrize("T,n_seg", [(1000, 1), (1000, 3), (1000, 7), (4096, 16), (130, 8)])
def test_segments_match_oracle(T, n_seg):
    print(f"case segment T={T} n_seg={n_seg}", flush=True)
    inp = wl.prefill_inputs(T=T, H=2, dk=128, dv=128, dtype="bf16", seed=T + n_seg, h0_std=0.02)
    o, ht = _seg(inp, n_seg, scale=0.9)
    o_ref, ht_ref = _oracle(inp, varlen=False, scale=0.9)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_segments_agree_with_chunk_fwd():
    """Any segment count reaches the same result as the single-pass kernel."""
    inp = wl.prefill_inputs(T=3000, H=3, dk=128, dv=128, dtype="bf16", seed=8, h0_std=0.02)
    d = to_dev(inp)
    o1, h1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"],
                           out_dtype=torch.float32)
    for n_seg in (2, 5, 47):
        o2, h2 = _seg(inp, n_seg)
        e_o = rel_max_err(np64(o2), np64(o1))
        e_s = rel_max_err(np64(h2), np64(h1))
        print(f"n_seg={n_seg} vs chunk_fwd: err_o={e_o:.3e} err_state={e_s:.3e}")
        assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_segments_varlen():
    lengths = [1, 64, 65, 300, 0, 1000, 129]
    print(f"case segment varlen {lengths}", flush=True)
    inp = wl.prefill_inputs(H=2, dk=128, dv=128, dtype="bf16", seed=4, h0_std=0.02,
                            lengths=lengths)
    o, ht = _seg(inp, 4, varlen=True)
    o_ref, ht_ref = _oracle(inp, varlen=True)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    assert torch.equal(ht[4].cpu(), inp["h0"][4])


def test_segments_f32():
    inp = wl.prefill_inputs(T=700, H=2, dk=64, dv=64, dtype="f32", seed=3, h0_std=0.02)
    o, ht = _seg(inp, 5)
    o_ref, ht_ref = _oracle(inp, varlen=False)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"f32 err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_F32 and e_s <= TOL_F32


@pytest.mark.parametrize("n_seg", [64, 256])
def test_segments_f32_many_segments(n_seg):
    """fp32 inputs across the workload's 64..256 segment range (16384 tokens, so that 256
    segments still hold one chunk each): the ordered scan's products run in fp32, so the
    composition of 256 summaries stays within the fp32 bar of 1e-4 x RMS."""
    T = 16384
    print(f"case segment f32 T={T} H=2 d=64 n_seg={n_seg}", flush=True)
    inp = wl.prefill_inputs(T=T, H=2, dk=64, dv=64, dtype="f32", seed=60 + n_seg, h0_std=0.02)
    o, ht = _seg(inp, n_seg, scale=0.9)
    o_ref, ht_ref = _oracle(inp, varlen=False, scale=0.9)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"f32 n_seg={n_seg}: err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_F32 and e_s <= TOL_F32


def test_workspace_too_small_is_rejected():
    inp = to_dev(wl.prefill_inputs(T=256, H=2, dk=128, dv=128, dtype="bf16", seed=1))
    # below the segment summaries themselves (the size the query gives for fp32 inputs)
    need = kda.segment_cp_workspace_size(1, 256, 1, 2, 128, 128, io_dtype=kda.KDA_F32,
                                         n_segments=4)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        kda.segment_cp_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], n_segments=4,
                           workspace=ws)
    assert ei.value.status == -6


def test_automatic_segment_count():
    """n_segments = 0: the library picks the count from its cost model (a few segments for
    two heads of 1000 tokens) and matches the oracle."""
    inp = wl.prefill_inputs(T=1000, H=2, dk=128, dv=128, dtype="bf16", seed=21, h0_std=0.02)
    o, ht = _seg(inp, 0)
    o_ref, ht_ref = _oracle(inp, varlen=False)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"auto: err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_automatic_single_segment_is_the_forward_pass():
    """With enough heads to fill the device the model picks one segment, which runs the
    forward kernel itself: the result equals kda_chunk_fwd bit for bit."""
    inp = wl.prefill_inputs(T=300, H=96, dk=128, dv=128, dtype="bf16", seed=22, h0_std=0.02)
    d = to_dev(inp)
    o1, h1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"],
                           out_dtype=torch.float32)
    o2, h2 = _seg(inp, 0)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("n_segments,lengths", [(4, None), (0, None), (3, [100, 0, 700, 64, 1])])
def test_two_launch_form_is_bit_identical(n_segments, lengths):
    """A workspace holding the operand slots runs the prep pass and the transition and
    replay walks; one holding only the segment summaries runs the one-launch kernel for both.
    The two forms compute the same products in the same order: identical o and final state."""
    print(f"case segment two-launch vs one-launch n_segments={n_segments} lengths={lengths}",
          flush=True)
    if lengths is None:
        inp = wl.prefill_inputs(T=1500, H=3, dk=128, dv=128, dtype="bf16", seed=33, h0_std=0.02)
    else:
        inp = wl.prefill_inputs(H=2, dk=128, dv=128, dtype="bf16", seed=34, h0_std=0.02,
                                lengths=lengths)
    d = to_dev(inp)
    cu = d["cu_seqlens"] if lengths is not None else None
    T = int(d["q"].shape[0])
    N = len(lengths) if lengths is not None else 1
    H = int(d["q"].shape[1])
    full = kda.segment_cp_workspace_size(1, T, N, H, 128, 128, kda.KDA_BF16, n_segments)
    small = kda.segment_cp_workspace_size(1, T, N, H, 128, 128, kda.KDA_F32, n_segments)
    assert full > small
    res = []
    for nbytes in (full, small):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        res.append(kda.segment_cp_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"],
                                      cu_seqlens=cu, n_segments=n_segments, workspace=ws,
                                      out_dtype=torch.float32))
        torch.cuda.synchronize()
    (o1, h1), (o2, h2) = res
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o_ref, ht_ref = _oracle(inp, varlen=lengths is not None)
    e_o, e_s = rel_max_err(np64(o1), o_ref), rel_max_err(np64(h1), ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
