"""kda_chunk_fwd with fp32 inputs at d_k = d_v = 128 (the 16-token chunk form on fp32 matrix
cores, through a workspace of per-chunk operand blocks) against the fp64 oracle at the fp32
bar, with its ragged, varlen, floor, checkpoint, grouping and in-place cases."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import c_recurrence_fwd
from kda_testutil import TOL_F32, np64, rel_max_err, to_dev

pytestmark = pytest.mark.gpu


def _args(d):
    return [d[n] for n in ("q", "k", "v", "g", "beta")]


def _oracle(inp, scale=1.0, varlen=False):
    cu = inp["cu_seqlens"].numpy() if varlen else None
    return c_recurrence_fwd(*[np64(x) for x in _args(inp)], h0=np64(inp["h0"]), cu_seqlens=cu,
                            scale=scale)


@pytest.mark.parametrize("T,H,h0_std,scale", [(256, 2, 0.0, 1.0), (200, 3, 0.02, 0.7),
                                              (1, 2, 0.02, 1.0), (16, 1, 0.02, 1.0)])
def test_f32_d128_matches_oracle(T, H, h0_std, scale):
    print(f"case f32 d=128 T={T} H={H} h0_std={h0_std}", flush=True)
    inp = wl.prefill_inputs(T=T, H=H, dk=128, dv=128, dtype="f32", seed=T + 7, h0_std=h0_std)
    d = to_dev(inp)
    o, ht = kda.chunk_fwd(*_args(d), h0=d["h0"], scale=scale)
    torch.cuda.synchronize()
    o_ref, ht_ref = _oracle(inp, scale=scale)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_F32 and e_s <= TOL_F32


def test_f32_d128_varlen_with_h0():
    lengths = [1, 64, 65, 130, 0, 17, 256, 33]
    print(f"case f32 d=128 varlen lengths={lengths}", flush=True)
    inp = wl.prefill_inputs(H=2, dk=128, dv=128, dtype="f32", seed=21, h0_std=0.02,
                            lengths=lengths)
    d = to_dev(inp)
    o, ht = kda.chunk_fwd(*_args(d), h0=d["h0"], cu_seqlens=d["cu_seqlens"], scale=0.9)
    torch.cuda.synchronize()
    o_ref, ht_ref = _oracle(inp, scale=0.9, varlen=True)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_F32 and e_s <= TOL_F32
    # a length-0 sequence hands its entering state through unchanged
    assert torch.equal(ht[4].cpu(), inp["h0"][4])


@pytest.mark.parametrize("mode", ["floor_stress", "g_min_everywhere", "overwrite"])
def test_f32_d128_decay_extremes(mode):
    print(f"case f32 d=128 extremes {mode}", flush=True)
    kw = dict(T=300, H=2, dk=128, dv=128, dtype="f32", seed=5, h0_std=0.02)
    if mode == "floor_stress":
        inp = wl.prefill_inputs(floor_stress=True, **kw)
    elif mode == "g_min_everywhere":
        inp = wl.prefill_inputs(g_fill=-5.0, **kw)
    else:
        inp = wl.prefill_inputs(g_fill=0.0, beta_fill=1.0, **kw)
    d = to_dev(inp)
    o, ht = kda.chunk_fwd(*_args(d), h0=d["h0"])
    torch.cuda.synchronize()
    o_ref, ht_ref = _oracle(inp)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert np.isfinite(np64(o)).all()
    assert e_o <= TOL_F32 and e_s <= TOL_F32


def test_f32_d128_groups_and_in_place_state():
    """The smallest workspace (groups of whole sequences) gives the same bits as the whole
    batch's; the final state written over h0 in place gives the same bits too; two calls
    agree bit for bit."""
    lengths = [300, 0, 640, 129, 47, 64]
    print(f"case f32 d=128 groups lengths={lengths}", flush=True)
    inp = wl.prefill_inputs(H=3, dk=128, dv=128, dtype="f32", seed=23, h0_std=0.02,
                            lengths=lengths)
    d = to_dev(inp)
    kw = dict(h0=d["h0"], cu_seqlens=d["cu_seqlens"])
    o1, h1 = kda.chunk_fwd(*_args(d), workspace="two_pass", **kw)
    o2, h2 = kda.chunk_fwd(*_args(d), workspace="min", **kw)
    o3, h3 = kda.chunk_fwd(*_args(d), workspace="two_pass", **kw)
    state = d["h0"].clone()
    o4, _ = kda.chunk_fwd(*_args(d), h0=state, ht=state, cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    assert torch.equal(o1, o3) and torch.equal(h1, h3)
    assert torch.equal(o1, o4) and torch.equal(h1, state)
    o_ref, ht_ref = _oracle(inp, varlen=True)
    assert rel_max_err(np64(o1), o_ref) <= TOL_F32
    assert rel_max_err(np64(h1), ht_ref) <= TOL_F32


def test_f32_d128_checkpoints_and_resume():
    """Checkpoints every 128 tokens of packed sequences against the oracle's prefix states
    (slot floor(bos_n / every) + j; unreached slots untouched), and a resume from one
    reproducing the rest of its sequence bit for bit."""
    lengths, every = [300, 0, 640, 129, 64], 128
    print(f"case f32 d=128 checkpoints lengths={lengths} every={every}", flush=True)
    inp = wl.prefill_inputs(H=2, dk=128, dv=128, dtype="f32", seed=25, h0_std=0.02,
                            lengths=lengths)
    d = to_dev(inp)
    T = sum(lengths)
    ck = torch.full((T // every, 2, 128, 128), float("nan"), device="cuda")
    o, ht, _ = kda.chunk_fwd(*_args(d), h0=d["h0"], cu_seqlens=d["cu_seqlens"],
                             ckpt_every=every, ckpt=ck)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    host = [np64(x) for x in _args(inp)]
    written = set()
    for n, length in enumerate(lengths):
        a = cu[n]
        for j in range(length // every):
            slot = a // every + j
            written.add(slot)
            t = (j + 1) * every
            _, s_ref = c_recurrence_fwd(*[x[a:a + t] for x in host], h0=np64(inp["h0"][n:n + 1]))
            e = rel_max_err(np64(ck[slot:slot + 1]), s_ref)
            print(f"sequence {n} checkpoint {j} -> slot {slot}: err {e:.3e}")
            assert e <= TOL_F32
    for slot in range(T // every):
        if slot not in written:
            assert torch.isnan(ck[slot]).all()
    # resume sequence 2 (640 tokens) from its second checkpoint (after 256 tokens)
    a, cut = cu[2], 256
    slot = a // every + cut // every - 1
    rest = [x[a + cut:a + 640].contiguous() for x in _args(d)]
    o_r, ht_r = kda.chunk_fwd(*rest, h0=ck[slot:slot + 1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o_r, o[a + cut:a + 640])
    assert torch.equal(ht_r, ht[2:3])
