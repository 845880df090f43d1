"""The two-launch prefill of kda_chunk_fwd (prep pass over every chunk and head, then the
serial walk) against the one-launch kernel, bit for bit, and against the fp64 oracle."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import c_recurrence_fwd
from kda_testutil import TOL_BF16, np64, rel_max_err, to_dev

pytestmark = pytest.mark.gpu


def _args(d):
    return [d[n] for n in ("q", "k", "v", "g", "beta")]


def _both(inp, varlen=False, out_dtype=torch.float32, scale=1.0, h0=True):
    """(one-launch, two-launch) results of the same call."""
    d = to_dev(inp)
    cu = d["cu_seqlens"] if varlen else None
    res = []
    for ws in (None, "two_pass"):
        o, ht = kda.chunk_fwd(*_args(d), h0=d["h0"] if h0 else None, cu_seqlens=cu,
                              scale=scale, out_dtype=out_dtype, workspace=ws)
        torch.cuda.synchronize()
        res.append((o, ht))
    return res


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,H,dk", [(1000, 3, 128), (64, 2, 64), (1, 2, 128), (1061, 2, 128),
                                    (600, 5, 64)])
def test_two_pass_bit_identical_to_one_launch(T, H, dk, out_dtype):
    """Same operands, same products in the same order: o and the final state agree exactly
    (1061 tokens = 16 full chunks, two prep groups of eight, and a ragged 37-token chunk)."""
    print(f"case two-pass vs one-launch T={T} H={H} dk={dk} out={out_dtype}", flush=True)
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dk, dtype="bf16", seed=T + H, h0_std=0.02)
    (o1, h1), (o2, h2) = _both(inp, out_dtype=out_dtype, scale=0.8)
    assert torch.equal(o1, o2)
    assert torch.equal(h1, h2)


@pytest.mark.parametrize("dk", [64, 128])
def test_two_pass_varlen_bit_identical(dk):
    """Packed sequences, including empty ones, one-token ones and sequence starts that are
    not multiples of 64 (the operand slots of neighbouring sequences must not collide)."""
    lengths = [1, 64, 65, 130, 0, 17, 256, 700, 0, 3]
    print(f"case two-pass varlen dk={dk} lengths={lengths}", flush=True)
    inp = wl.prefill_inputs(H=3, dk=dk, dv=dk, dtype="bf16", seed=40 + dk, h0_std=0.02,
                            lengths=lengths)
    (o1, h1), (o2, h2) = _both(inp, varlen=True)
    assert torch.equal(o1, o2)
    assert torch.equal(h1, h2)
    assert torch.equal(h2[4].cpu(), inp["h0"][4]) and torch.equal(h2[8].cpu(), inp["h0"][8])


def test_two_pass_matches_oracle():
    print("case two-pass oracle T=1000 H=3 dk=128", flush=True)
    inp = wl.prefill_inputs(T=1000, H=3, dk=128, dv=128, dtype="bf16", seed=77, h0_std=0.02)
    _, (o, ht) = _both(inp, scale=0.9)
    o_ref, ht_ref = c_recurrence_fwd(*[np64(x) for x in _args(inp)], h0=np64(inp["h0"]),
                                     scale=0.9)
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht)[0:1], ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_two_pass_fixed_length_batch_without_h0():
    """A [B, T, H, d] batch (no cu_seqlens) with zero entering states."""
    B, T, H, dk = 3, 200, 2, 128
    print(f"case two-pass batch B={B} T={T} H={H}", flush=True)
    inp = wl.prefill_inputs(H=H, dk=dk, dv=dk, dtype="bf16", seed=9, lengths=[T] * B)
    d = to_dev(inp)
    args = [x.reshape(B, T, *x.shape[1:]) for x in _args(d)]
    o1, h1 = kda.chunk_fwd(*args, out_dtype=torch.float32, workspace=None)
    o2, h2 = kda.chunk_fwd(*args, out_dtype=torch.float32, workspace="two_pass")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o_ref, ht_ref = c_recurrence_fwd(*[np64(x) for x in _args(inp)],
                                     cu_seqlens=inp["cu_seqlens"].numpy())
    e_o = rel_max_err(np64(o2).reshape(B * T, H, dk), o_ref)
    e_s = rel_max_err(np64(h2), ht_ref)
    print(f"err_o={e_o:.3e} err_state={e_s:.3e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_workspace_contents_do_not_matter():
    """Every operand the walk reads is written by the prep pass of the same call: a
    workspace full of NaN bytes gives the same result as a zeroed one."""
    inp = wl.prefill_inputs(T=777, H=2, dk=128, dv=128, dtype="bf16", seed=12, h0_std=0.02)
    d = to_dev(inp)
    need = kda.chunk_fwd_workspace_size(1, 777, 1, 2, 128, 128,
                                        policy=kda.KDA_CHUNK_WS_TWO_PASS)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        outs.append(kda.chunk_fwd(*_args(d), h0=d["h0"], out_dtype=torch.float32, workspace=ws))
        torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert np.isfinite(np64(outs[1][0])).all()


def test_automatic_path_choice():
    """The automatic policy takes the whole batch in two launches when the one-launch
    workgroups would not fill the device (8192 tokens x 96 heads: 192 workgroups), and groups
    of sequences through an 8 GiB workspace when they would (64 sequences x 96 heads)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"compute units {cus}", flush=True)
    n_small = kda.chunk_fwd_workspace_size(1, 8192, 1, 96, 128, 128)
    if 96 * 2 <= cus:
        assert n_small == kda.chunk_fwd_workspace_size(
            1, 8192, 1, 96, 128, 128, policy=kda.KDA_CHUNK_WS_TWO_PASS) > 0
    cu = torch.tensor([0] + [8192 * (i + 1) for i in range(64)], dtype=torch.int32)
    n_large = kda.chunk_fwd_workspace_size(1, 8192 * 64, 64, 96, 128, 128, cu_seqlens_host=cu)
    assert n_large == 8 << 30


@pytest.mark.parametrize("dk", [64, 128])
def test_grouped_sequences_bit_identical(dk):
    """A workspace smaller than the batch needs runs groups of whole sequences (here the
    least it accepts: the longest sequence's slots, so most groups hold one or two
    sequences): same bits as the one-launch kernel, checkpoints included."""
    lengths = [300, 0, 640, 129, 1024, 64, 1, 500]
    print(f"case grouped sequences dk={dk} lengths={lengths}", flush=True)
    inp = wl.prefill_inputs(H=3, dk=dk, dv=dk, dtype="bf16", seed=57 + dk, h0_std=0.02,
                            lengths=lengths)
    d = to_dev(inp)
    cu = d["cu_seqlens"]
    T = sum(lengths)
    need_min = kda.chunk_fwd_workspace_size(1, T, len(lengths), 3, dk, dk,
                                            policy=kda.KDA_CHUNK_WS_MIN,
                                            cu_seqlens_host=inp["cu_seqlens"])
    need_all = kda.chunk_fwd_workspace_size(1, T, len(lengths), 3, dk, dk,
                                            policy=kda.KDA_CHUNK_WS_TWO_PASS)
    assert need_min < need_all
    res = []
    for ws in (None, torch.empty(need_min, dtype=torch.uint8, device="cuda")):
        ck = torch.full((T // 128, 3, dk, dk), float("nan"), device="cuda")
        res.append(kda.chunk_fwd(*_args(d), h0=d["h0"], cu_seqlens=cu, out_dtype=torch.float32,
                                 workspace=ws, ckpt_every=128, ckpt=ck))
        torch.cuda.synchronize()
    (o1, h1, c1), (o2, h2, c2) = res
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    assert torch.equal(torch.isnan(c1), torch.isnan(c2))
    written = ~torch.isnan(c1)
    assert torch.equal(c1[written], c2[written])
    with pytest.raises(kda.KDAError) as ei:
        kda.chunk_fwd(*_args(d), h0=d["h0"], cu_seqlens=cu,
                      workspace=torch.empty(need_min - 16, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == -6


def test_two_tiles_per_workgroup_bit_identical():
    """With more (sequence, head, tile) units than compute units the walk packs both value
    tiles of a head into one eight-wave workgroup: still the same bits as the one-launch
    kernel (3 sequences x 96 heads x 2 tiles = 576 tiles)."""
    lengths = [200, 64, 130]
    print(f"case two tiles per workgroup lengths={lengths} H=96", flush=True)
    inp = wl.prefill_inputs(H=96, dk=128, dv=128, dtype="bf16", seed=55, h0_std=0.02,
                            lengths=lengths)
    (o1, h1), (o2, h2) = _both(inp, varlen=True)
    assert torch.equal(o1, o2)
    assert torch.equal(h1, h2)


def test_segment_walks_two_tiles_per_workgroup_bit_identical():
    """The segment path's transition walk (96 heads x 2 segments x 4 tiles) and replay walk
    (x 2 tiles) with eight-wave workgroups, against the one-launch passes."""
    print("case segment walks with two tiles per workgroup T=256 H=96 n_segments=2", flush=True)
    inp = wl.prefill_inputs(T=256, H=96, dk=128, dv=128, dtype="bf16", seed=56, h0_std=0.02)
    d = to_dev(inp)
    full = kda.segment_cp_workspace_size(1, 256, 1, 96, 128, 128, kda.KDA_BF16, 2)
    small = kda.segment_cp_workspace_size(1, 256, 1, 96, 128, 128, kda.KDA_F32, 2)
    res = []
    for nbytes in (full, small):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        res.append(kda.segment_cp_fwd(*_args(d), h0=d["h0"], n_segments=2, workspace=ws,
                                      out_dtype=torch.float32))
        torch.cuda.synchronize()
    (o1, h1), (o2, h2) = res
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_many_sequences_keep_their_order_bit_identical():
    """Walks take a group's sequences longest first when the group has at most 256 (the other
    tests here); a group of 300 keeps sequence order. Both give the one-launch kernel's bits."""
    g = torch.Generator().manual_seed(58)
    lengths = torch.randint(0, 90, (300,), generator=g).tolist()
    print(f"case 300 short sequences, {sum(lengths)} tokens", flush=True)
    inp = wl.prefill_inputs(H=2, dk=64, dv=64, dtype="bf16", seed=58, h0_std=0.02,
                            lengths=lengths)
    (o1, h1), (o2, h2) = _both(inp, varlen=True)
    assert torch.equal(o1, o2)
    assert torch.equal(h1, h2)
