"""Parity of kda_decode_replay (HIP, through the C ABI) with the fp64 CPU oracle, and
bit-identity of replayed states with one-token-at-a-time launches."""
import dataclasses

import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import kda_oracle as ko
from kda_testutil import TOL_BF16, np64, rel_max_err

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-5   # absolute, fp32 arithmetic against the fp64 oracle


def _dev_window(win):
    return {k: (v.cuda() if v is not None else None) for k, v in win.items()}


def _np_window(win):
    return {k: np64(v) for k, v in win.items()}


def _run_gpu(w, n_new=None, act=1, scale=1.0, out_dtype=torch.float32):
    state = w.state.cuda().clone()
    tail = w.conv_tail.cuda().clone()
    o, acc = kda.decode_replay(state, tail, w.n_acc.cuda(), _dev_window(w.prev),
                               _dev_window(w.new), w.conv_w.cuda(), w.norm_w.cuda(),
                               n_new=n_new, act=act, scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, state, acc, tail


def _run_oracle(w, n_new=None, act=1, scale=1.0):
    new = _np_window(w.new)
    if n_new is not None:
        new = {k: (v[:, :n_new] if v is not None else None) for k, v in new.items()}
    return ko.decode_replay(np64(w.state), np64(w.conv_tail), w.n_acc.numpy(),
                            _np_window(w.prev), new, np64(w.conv_w), np64(w.norm_w),
                            scale=scale, act=act)


@pytest.mark.parametrize("D,W,n_new,act", [(128, 4, 8, 1), (64, 4, 8, 1), (128, 2, 3, 0),
                                           (128, 4, 1, 1), (64, 1, 5, 1)])
def test_decode_matches_oracle(D, W, n_new, act):
    print(f"case decode D={D} W={W} n_new={n_new} act={act}", flush=True)
    w = wl.decode_inputs(R=5, H=3, dk=D, dv=D, conv_width=W, n_new=8, window=8, seed=D + W)
    o, state, acc, tail = _run_gpu(w, n_new=n_new, act=act, scale=0.8)
    ref = _run_oracle(w, n_new=n_new, act=act, scale=0.8)
    e_state = np.abs(np64(state) - ref["state"]).max()
    e_acc = np.abs(np64(acc) - ref["state_acc"]).max()
    e_tail = np.abs(np64(tail) - ref["conv_tail"]).max() if tail.numel() else 0.0
    e_o = rel_max_err(np64(o), ref["o"])
    print(f"n_acc={w.n_acc.tolist()} err_state={e_state:.2e} err_acc={e_acc:.2e} "
          f"err_tail={e_tail:.2e} err_o={e_o:.2e}")
    assert e_state <= STATE_TOL and e_acc <= STATE_TOL and e_tail <= STATE_TOL
    assert e_o <= TOL_BF16


@pytest.mark.parametrize("a", [0, 3, 7])
def test_replay_bit_identical_to_single_token_launches(a):
    """One launch replaying a accepted drafts then the bonus equals a + 1 launches that each
    take a single token (n_acc = 0, n_new = 1): states, tails and the bonus output match
    bit for bit."""
    print(f"case bit-identity a={a}", flush=True)
    R, H, D = 4, 3, 128
    w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, n_new=8, window=8, seed=40 + a, n_acc_fill=a)
    o_a, s_a, acc_a, tail_a = _run_gpu(w, n_new=1)

    state = w.state.cuda().clone()
    tail = w.conv_tail.cuda().clone()
    zeros_acc = torch.zeros(R, dtype=torch.int32, device="cuda")
    prev = _dev_window(w.prev)
    for j in range(1, a + 1):
        one = {k: (prev[k][:, j:j + 1].contiguous() if prev[k] is not None else None)
               for k in ("q", "k", "v", "g", "beta")}
        one["z"] = torch.zeros(R, 1, H, D, dtype=torch.bfloat16, device="cuda")
        kda.decode_replay(state, tail, zeros_acc, prev, one, w.conv_w.cuda(), w.norm_w.cuda(),
                          n_new=1, write_state_acc=False, out_dtype=torch.float32)
    acc_seq = state.clone()
    new = _dev_window(w.new)
    bonus = {k: (new[k][:, :1].contiguous() if new[k] is not None else None) for k in new}
    o_b, _ = kda.decode_replay(state, tail, zeros_acc, prev, bonus, w.conv_w.cuda(),
                               w.norm_w.cuda(), n_new=1, write_state_acc=False,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(acc_a, acc_seq)
    assert torch.equal(s_a, state)
    assert torch.equal(tail_a, tail)
    assert torch.equal(o_a[:, 0], o_b[:, 0])


@pytest.mark.parametrize("D", [128, 64])
def test_small_batch_waves_bit_identical(D):
    """A launch gives each (request, head) workgroup 8 waves when the pairs would leave most
    compute units idle, and 4 otherwise. Every lane keeps the same key rows and every sum the
    same order, so requests run inside a large batch (4 waves) and alone in a small one
    (8 waves, first block fetched before the accepted count is known) agree bit for bit,
    with accepted counts 0 and above among them."""
    R, H = 64, 12
    print(f"case decode widths D={D}: {R}x{H} against 3x{H}", flush=True)
    w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, conv_width=4, n_new=4, window=8, seed=77 + D)
    w.n_acc[0] = 0
    w.n_acc[5] = 6
    pick = [0, 5, 63]
    big = _run_gpu(w)                                   # 768 pairs: 4 waves
    sel = lambda x: None if x is None else x[pick].clone()
    sub = dataclasses.replace(w, R=len(pick), n_acc=w.n_acc[pick].clone(),
                              prev={k: sel(v) for k, v in w.prev.items()},
                              new={k: sel(v) for k, v in w.new.items()},
                              state=w.state[pick].clone(), conv_tail=w.conv_tail[pick].clone())
    small = _run_gpu(sub)                               # 36 pairs: 8 waves
    for name, x, y in zip(("o", "state", "state_acc", "tail"), big, small):
        assert torch.equal(x[pick], y), name


def test_speculative_stream_matches_oracle():
    """Four verify steps with random acceptance, each call's window becoming the next call's
    previous window: the committed state tracks the oracle's stream throughout."""
    R, H, D = 3, 2, 128
    w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, n_new=8, window=8, seed=77)
    state, tail = w.state.cuda().clone(), w.conv_tail.cuda().clone()
    s_ref, t_ref = np64(w.state), np64(w.conv_tail)
    prev = w.prev
    n_acc = torch.zeros(R, dtype=torch.int32)
    gen = torch.Generator().manual_seed(5)
    for step in range(4):
        new = wl.decode_inputs(R=R, H=H, dk=D, dv=D, n_new=8, window=8, seed=100 + step).new
        o, _ = kda.decode_replay(state, tail, n_acc.cuda(), _dev_window(prev),
                                 _dev_window(new), w.conv_w.cuda(), w.norm_w.cuda(),
                                 out_dtype=torch.float32)
        ref = ko.decode_replay(s_ref, t_ref, n_acc.numpy(), _np_window(prev), _np_window(new),
                               np64(w.conv_w), np64(w.norm_w))
        torch.cuda.synchronize()
        s_ref, t_ref = ref["state"], ref["conv_tail"]
        e = np.abs(np64(state) - s_ref).max()
        print(f"step {step} n_acc={n_acc.tolist()} err_state={e:.2e}")
        assert e <= STATE_TOL
        assert rel_max_err(np64(o), ref["o"]) <= TOL_BF16
        prev = new
        n_acc = torch.randint(0, 8, (R,), generator=gen, dtype=torch.int32)


def test_decode_validation_errors():
    w = wl.decode_inputs(R=2, H=2, dk=128, dv=128, n_new=8, window=8, seed=1)
    state, tail = w.state.cuda(), w.conv_tail.cuda()
    with pytest.raises(kda.KDAError) as ei:   # n_new above the window
        kda.decode_replay(state, tail, w.n_acc.cuda(), _dev_window(w.prev), _dev_window(w.new),
                          w.conv_w.cuda(), w.norm_w.cuda(), n_new=9)
    assert ei.value.status == -2


def test_decode_bf16_output_is_rounded_fp32_output():
    """The bf16 output is exactly the round-to-nearest-even of the fp32 output of the same
    arithmetic (outputs after the gated RMSNorm reach ~8x their RMS, so bf16's own half-ulp
    is ~2.6% of the RMS at the largest elements: the tolerance is checked on fp32)."""
    w = wl.decode_inputs(R=6, H=3, dk=128, dv=128, n_new=8, window=8, seed=9)
    o32, s32, a32, t32 = _run_gpu(w, out_dtype=torch.float32)
    o16, s16, a16, t16 = _run_gpu(w, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(s32, s16) and torch.equal(a32, a16) and torch.equal(t32, t16)


@pytest.mark.parametrize("D", [128, 64])
def test_irregular_draft_windows(D):
    """Requests with different new-token counts in one launch: each request's outputs match
    the oracle run over its own window, rows past its count stay untouched, and the
    committed states equal those of the uniform launch bit for bit (they only depend on the
    accepted drafts and the bonus token)."""
    R, H = 6, 3
    w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, conv_width=4, n_new=8, window=8, seed=70 + D)
    nn = torch.tensor([1, 8, 3, 5, 2, 7], dtype=torch.int32)
    print(f"case irregular windows D={D} n_acc={w.n_acc.tolist()} n_new={nn.tolist()}",
          flush=True)
    state, tail = w.state.cuda().clone(), w.conv_tail.cuda().clone()
    o = torch.full((R, 8, H, D), float("nan"), device="cuda")
    _, acc = kda.decode_replay(state, tail, w.n_acc.cuda(), _dev_window(w.prev),
                               _dev_window(w.new), w.conv_w.cuda(), w.norm_w.cuda(), o=o,
                               n_new_per_request=nn.cuda())
    torch.cuda.synchronize()
    o_u, state_u, acc_u, tail_u = _run_gpu(w)
    assert torch.equal(state, state_u) and torch.equal(acc, acc_u) and torch.equal(tail, tail_u)
    for r in range(R):
        k = int(nn[r])
        assert torch.equal(o[r, :k], o_u[r, :k])
        assert torch.isnan(o[r, k:]).all()
        ref = ko.decode_replay(np64(w.state[r:r + 1]), np64(w.conv_tail[r:r + 1]),
                               w.n_acc[r:r + 1].numpy(),
                               {x: (np64(v[r:r + 1]) if v is not None else None)
                                for x, v in w.prev.items()},
                               {x: (np64(v[r:r + 1, :k]) if v is not None else None)
                                for x, v in w.new.items()},
                               np64(w.conv_w), np64(w.norm_w))
        e_o = rel_max_err(np64(o[r:r + 1, :k]), ref["o"])
        e_s = np.abs(np64(state[r:r + 1]) - ref["state"]).max()
        print(f"request {r} (n_acc {int(w.n_acc[r])}, n_new {k}): err_o={e_o:.2e} "
              f"err_state={e_s:.2e}")
        assert e_o <= TOL_BF16 and e_s <= STATE_TOL
