"""State checkpoints of kda_chunk_fwd (prefix-cache resume points): every checkpoint against
the fp64 oracle's state after the same prefix, and a resume from a checkpoint reproducing the
rest of the original call bit for bit, on the one-launch and the two-launch paths."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import c_recurrence_fwd
from kda_testutil import TOL_BF16, np64, rel_max_err, to_dev

pytestmark = pytest.mark.gpu

PATHS = [None, "two_pass"]


def _args(d):
    return [d[n] for n in ("q", "k", "v", "g", "beta")]


@pytest.mark.parametrize("workspace", PATHS)
@pytest.mark.parametrize("dk,every", [(128, 256), (64, 128)])
def test_checkpoints_match_oracle_prefix_states(workspace, dk, every):
    T, H = 1000, 3
    print(f"case checkpoints T={T} H={H} dk={dk} every={every} path={workspace}", flush=True)
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dk, dtype="bf16", seed=61, h0_std=0.02)
    d = to_dev(inp)
    o, ht, ck = kda.chunk_fwd(*_args(d), h0=d["h0"], out_dtype=torch.float32,
                              workspace=workspace, ckpt_every=every)
    torch.cuda.synchronize()
    assert ck.shape == (T // every, H, dk, dk)
    host = [np64(x) for x in _args(inp)]
    for j in range(T // every):
        t = (j + 1) * every
        _, s_ref = c_recurrence_fwd(*[x[:t] for x in host], h0=np64(inp["h0"]))
        e = rel_max_err(np64(ck[j:j + 1]), s_ref)
        print(f"checkpoint {j} (after {t} tokens): err {e:.3e}")
        assert e <= TOL_BF16


@pytest.mark.parametrize("workspace", PATHS)
def test_varlen_checkpoint_slots(workspace):
    """Packed sequences: sequence n's j-th checkpoint lands in slot floor(bos_n / every) + j;
    slots no sequence reaches keep their contents."""
    lengths, every = [300, 0, 640, 129, 1024, 64], 128
    print(f"case varlen checkpoints lengths={lengths} every={every} path={workspace}", flush=True)
    inp = wl.prefill_inputs(H=2, dk=128, dv=128, dtype="bf16", seed=62, h0_std=0.02,
                            lengths=lengths)
    d = to_dev(inp)
    T = sum(lengths)
    ck = torch.full((T // every, 2, 128, 128), float("nan"), device="cuda")
    kda.chunk_fwd(*_args(d), h0=d["h0"], cu_seqlens=d["cu_seqlens"], out_dtype=torch.float32,
                  workspace=workspace, ckpt_every=every, ckpt=ck)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    host = [np64(x) for x in _args(inp)]
    written = set()
    for n, length in enumerate(lengths):
        a = cu[n]
        for j in range(length // every):
            slot = a // every + j
            assert slot not in written
            written.add(slot)
            t = (j + 1) * every
            _, s_ref = c_recurrence_fwd(*[x[a:a + t] for x in host], h0=np64(inp["h0"][n:n + 1]))
            e = rel_max_err(np64(ck[slot:slot + 1]), s_ref)
            print(f"sequence {n} checkpoint {j} -> slot {slot}: err {e:.3e}")
            assert e <= TOL_BF16
    for slot in range(T // every):
        if slot not in written:
            assert torch.isnan(ck[slot]).all()


@pytest.mark.parametrize("workspace", PATHS)
def test_resume_from_checkpoint_is_bit_exact(workspace):
    """A checkpoint passed as h0 for the rest of the sequence gives the rest of the original
    output and the same final state, bit for bit (chunk boundaries line up)."""
    T, H, every = 1000, 3, 256
    print(f"case resume T={T} H={H} every={every} path={workspace}", flush=True)
    inp = wl.prefill_inputs(T=T, H=H, dk=128, dv=128, dtype="bf16", seed=63, h0_std=0.02)
    d = to_dev(inp)
    o, ht, ck = kda.chunk_fwd(*_args(d), h0=d["h0"], workspace=workspace, ckpt_every=every)
    for j in range(T // every):
        t = (j + 1) * every
        o2, ht2 = kda.chunk_fwd(*[x[t:] for x in _args(d)], h0=ck[j:j + 1].contiguous(),
                                workspace=workspace)
        torch.cuda.synchronize()
        assert torch.equal(o2, o[t:]), f"resume after {t} tokens"
        assert torch.equal(ht2, ht)


def test_checkpoint_interval_beyond_the_sequence():
    """An interval longer than every sequence writes nothing and needs no buffer."""
    inp = wl.prefill_inputs(T=200, H=2, dk=128, dv=128, dtype="bf16", seed=64)
    d = to_dev(inp)
    o, ht, ck = kda.chunk_fwd(*_args(d), ckpt_every=256)
    torch.cuda.synchronize()
    assert ck.shape[0] == 0
    o_ref, _ = kda.chunk_fwd(*_args(d))
    assert torch.equal(o, o_ref)
