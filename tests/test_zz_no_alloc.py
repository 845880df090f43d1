"""kda_chunk_fwd_noalloc through the C ABI against kda_chunk_fwd: the same bits, on two calls in
a row (the second smaller), with nothing allocated by the calls. The first call's packed batch
needs more operand slots than the 256 MiB static scratch holds, so it runs in groups of whole
sequences; kda_chunk_fwd gets a workspace for the whole batch and runs it in one group."""
import ctypes

import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl

pytestmark = pytest.mark.gpu

F32, BF16 = 0, 1
SCRATCH = 256 << 20


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(fn, inp, cu_dev, cu_host, o, ht, T, N, H, d, ws=None, io=BF16):
    lib = kda.library()
    args = [_p(inp["q"]), _p(inp["k"]), _p(inp["v"]), _p(inp["g"]), _p(inp["beta"]),
            _p(inp["h0"]), _p(cu_dev),
            None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr()),
            1, T, N, H, d, d, io, io, 1.0, -5.0, _p(o), _p(ht), 0, None]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if fn == "noalloc":
        return lib.kda_chunk_fwd_noalloc(*args, stream)
    return lib.kda_chunk_fwd(*args, _p(ws), 0 if ws is None else ws.numel(), stream)


def _run_case(lengths, H, d, seed):
    dev = torch.device("cuda")
    print(f"case noalloc lengths={lengths} H={H} d={d}", flush=True)
    inp = wl.prefill_inputs(H=H, dk=d, dv=d, dtype="bf16", seed=seed, h0_std=0.02,
                            lengths=lengths, device=dev)
    cu_host = inp["cu_seqlens"].to("cpu", torch.int32).contiguous()
    cu_dev = cu_host.to(dev)
    T, N = int(cu_host[-1]), len(lengths)
    slots = (T // 64 + N + 1) * H * (74752 if d == 128 else 50176)
    need = kda.chunk_fwd_workspace_size(1, T, N, H, d, d, policy=kda.KDA_CHUNK_WS_TWO_PASS,
                                        cu_seqlens_host=cu_host)
    assert need == slots
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o_ref = torch.empty(T, H, d, dtype=torch.bfloat16, device=dev)
    ht_ref = torch.empty(N, H, d, d, dtype=torch.float32, device=dev)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    assert _call("ws", inp, cu_dev, cu_host, o_ref, ht_ref, T, N, H, d, ws) == 0
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    assert _call("noalloc", inp, cu_dev, cu_host, o, ht, T, N, H, d) == 0
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(o, o_ref)
    assert torch.equal(ht, ht_ref)
    return slots


def test_noalloc_matches_chunk_fwd_on_two_calls():
    # the first batch's slots exceed the scratch (groups of sequences), the second is smaller
    big = _run_case([2000, 1500, 0, 700, 2303, 65], 96, 128, seed=31)
    assert big > SCRATCH
    small = _run_case([500], 4, 64, seed=32)
    assert small < big


def test_noalloc_fp32_d128_matches_chunk_fwd_on_two_calls():
    """fp32 at d = 128 (operand blocks of the 16-token chunk form in the scratch): the same
    bits as kda_chunk_fwd with a whole-batch workspace, on two calls in a row, the first in
    groups of sequences, the second smaller."""
    dev = torch.device("cuda")
    block = 27200
    sizes = []
    for lengths, H, seed in (([1500, 900, 0, 1615, 30], 96, 33), ([300, 17], 4, 34)):
        print(f"case noalloc fp32 d=128 lengths={lengths} H={H}", flush=True)
        inp = wl.prefill_inputs(H=H, dk=128, dv=128, dtype="f32", seed=seed, h0_std=0.02,
                                lengths=lengths, device=dev)
        cu_host = inp["cu_seqlens"].to("cpu", torch.int32).contiguous()
        cu_dev = cu_host.to(dev)
        T, N = int(cu_host[-1]), len(lengths)
        need = kda.chunk_fwd_workspace_size(1, T, N, H, 128, 128, io_dtype=F32,
                                            policy=kda.KDA_CHUNK_WS_TWO_PASS,
                                            cu_seqlens_host=cu_host)
        assert need == (T // 16 + N + 1) * H * block
        sizes.append(need)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        o_ref = torch.empty(T, H, 128, dtype=torch.float32, device=dev)
        ht_ref = torch.empty(N, H, 128, 128, dtype=torch.float32, device=dev)
        o = torch.full_like(o_ref, float("nan"))
        ht = torch.full_like(ht_ref, float("nan"))
        assert _call("ws", inp, cu_dev, cu_host, o_ref, ht_ref, T, N, H, 128, ws, io=F32) == 0
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        assert _call("noalloc", inp, cu_dev, cu_host, o, ht, T, N, H, 128, io=F32) == 0
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(o, o_ref)
        assert torch.equal(ht, ht_ref)
        del inp, ws, o_ref, ht_ref, o, ht
    assert sizes[0] > SCRATCH and sizes[1] < sizes[0]


def test_noalloc_rejects_a_sequence_beyond_the_scratch():
    dev = torch.device("cuda")
    H, d, T = 96, 128, 2304
    print(f"case noalloc rejection T={T} H={H} d={d}", flush=True)
    # rejected before any launch: the tensors are never read
    q = torch.empty(T, H, d, dtype=torch.bfloat16, device=dev)
    g = torch.empty(T, H, d, dtype=torch.float32, device=dev)
    beta = torch.empty(T, H, dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lib = kda.library()
    st = lib.kda_chunk_fwd_noalloc(_p(q), _p(q), _p(q), _p(g), _p(beta), None, None, None, 1, T,
                                   1, H, d, d, BF16, BF16, 1.0, -5.0, _p(o), None, 0, None,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -11
