"""The library's launches inside HIP graphs (torch.cuda.CUDAGraph is a HIP graph on ROCm):
the calls allocate nothing, clear nothing with memsets and synchronise nothing, so they can
be captured; every replay, with eager work and synchronisation between replays, must give
the eager result bit for bit."""
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from kda_testutil import to_dev

pytestmark = pytest.mark.gpu


def test_two_launch_prefill_in_a_graph():
    print("case graph: two-launch prefill T=700 H=4 d=128", flush=True)
    d = to_dev(wl.prefill_inputs(T=700, H=4, dk=128, dv=128, dtype="bf16", seed=101,
                                 h0_std=0.02))
    args = [d[n] for n in ("q", "k", "v", "g", "beta")]
    need = kda.chunk_fwd_workspace_size(1, 700, 1, 4, 128, 128,
                                        policy=kda.KDA_CHUNK_WS_TWO_PASS)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty(700, 4, 128, dtype=torch.bfloat16, device="cuda")
    ht = torch.empty(1, 4, 128, 128, dtype=torch.float32, device="cuda")
    o_ref, ht_ref = kda.chunk_fwd(*args, h0=d["h0"], workspace=ws)
    o_ref, ht_ref = o_ref.clone(), ht_ref.clone()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        kda.chunk_fwd(*args, h0=d["h0"], o=o, ht=ht, workspace=ws,
                      stream=torch.cuda.current_stream())
    for i in range(4):
        o.zero_()
        ht.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref), f"replay {i}"


def test_decode_verify_in_a_graph():
    """The page-shaped tiny verify (1 request, 12 heads, 4 new tokens): the graph restores the
    committed state and tail with device copies, then runs the fused verify."""
    print("case graph: decode verify R=1 H=12 n_new=4", flush=True)
    w = wl.decode_inputs(R=1, H=12, dk=128, dv=128, n_new=4, window=4, seed=102,
                         device="cuda")
    state, tail = w.state.clone(), w.conv_tail.clone()
    acc = torch.empty_like(state)
    o = torch.empty(1, 4, 12, 128, dtype=torch.bfloat16, device="cuda")
    o_ref, acc_ref = kda.decode_replay(state, tail, w.n_acc, w.prev, w.new, w.conv_w, w.norm_w)
    o_ref, acc_ref, s_ref, t_ref = o_ref.clone(), acc_ref.clone(), state.clone(), tail.clone()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        state.copy_(w.state)
        tail.copy_(w.conv_tail)
        kda.decode_replay(state, tail, w.n_acc, w.prev, w.new, w.conv_w, w.norm_w,
                          state_acc=acc, o=o, stream=torch.cuda.current_stream())
    for i in range(4):
        o.zero_()
        acc.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(acc, acc_ref), f"replay {i}"
        assert torch.equal(state, s_ref) and torch.equal(tail, t_ref), f"replay {i}"


def _replays_match(graph, outs, refs, n=4):
    for i in range(n):
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs, refs):
            assert torch.equal(x, y), f"replay {i}"


def test_segment_path_in_a_graph():
    """Prep pass, transition walk, ordered scan and replay walk (4 launches) in one graph."""
    print("case graph: segment path T=2048 H=2 n_segments=4", flush=True)
    d = to_dev(wl.prefill_inputs(T=2048, H=2, dk=128, dv=128, dtype="bf16", seed=103,
                                 h0_std=0.02))
    args = [d[n] for n in ("q", "k", "v", "g", "beta")]
    need = kda.segment_cp_workspace_size(1, 2048, 1, 2, 128, 128, kda.KDA_BF16, 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty(2048, 2, 128, dtype=torch.bfloat16, device="cuda")
    ht = torch.empty(1, 2, 128, 128, dtype=torch.float32, device="cuda")
    o_ref, ht_ref = kda.segment_cp_fwd(*args, h0=d["h0"], n_segments=4, workspace=ws)
    o_ref, ht_ref = o_ref.clone(), ht_ref.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        kda.segment_cp_fwd(*args, h0=d["h0"], n_segments=4, workspace=ws, o=o, ht=ht,
                           stream=torch.cuda.current_stream())
    _replays_match(graph, (o, ht), (o_ref, ht_ref))


def test_raw_prefill_in_a_graph():
    """The raw-projection prefill (token stage in the prep pass, then the walk) in a graph:
    outputs, final states and leaving conv tails of every replay equal the eager call's."""
    lengths = [200, 70, 333]
    print(f"case graph: raw prefill lengths={lengths} H=2", flush=True)
    d = to_dev(wl.raw_prefill_inputs(lengths=lengths, H=2, dk=128, dv=128, conv_width=4,
                                     seed=104, h0_std=0.02))
    raw = [d[n] for n in ("q", "k", "v", "g", "beta", "conv_w")]
    T = sum(lengths)
    ws = torch.empty(kda.chunk_fwd_raw_workspace_size(1, T, len(lengths), 2, 128, 128),
                     dtype=torch.uint8, device="cuda")
    cu_host = d["cu_seqlens"].cpu().to(torch.int32)
    cu_dev = cu_host.cuda()
    o_ref, ht_ref, tail_ref = kda.chunk_fwd_raw(*raw, conv_tail=d["conv_tail"], h0=d["h0"],
                                                cu_seqlens=cu_dev, cu_seqlens_host=cu_host,
                                                workspace=ws)
    o_ref, ht_ref, tail_ref = o_ref.clone(), ht_ref.clone(), tail_ref.clone()
    o, ht, tail = torch.empty_like(o_ref), torch.empty_like(ht_ref), torch.empty_like(tail_ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        kda.chunk_fwd_raw(*raw, conv_tail=d["conv_tail"], h0=d["h0"], cu_seqlens=cu_dev,
                          cu_seqlens_host=cu_host, workspace=ws, o=o, ht=ht,
                          conv_tail_out=tail, stream=torch.cuda.current_stream())
    _replays_match(graph, (o, ht, tail), (o_ref, ht_ref, tail_ref))


def test_backward_in_a_graph():
    """kda_chunk_bwd (four launches) captured: every replay gives the eager gradients."""
    print("case graph: backward T=300 H=2 d=128 packed", flush=True)
    lengths = [200, 0, 100]
    d = to_dev(wl.prefill_inputs(H=2, dk=128, dv=128, dtype="bf16", seed=103, h0_std=0.02,
                                 lengths=lengths))
    args = [d[n] for n in ("q", "k", "v", "g", "beta")]
    gen = torch.Generator(device="cuda").manual_seed(104)
    do = torch.randn(300, 2, 128, device="cuda", generator=gen).to(torch.bfloat16)
    dht = torch.randn(3, 2, 128, 128, device="cuda", generator=gen)
    cu = d["cu_seqlens"]
    cu_host = cu.to("cpu")
    ws = torch.empty(kda.chunk_bwd_workspace_size(1, 300, 3, 2, 128, 128), dtype=torch.uint8,
                     device="cuda")
    ref = kda.chunk_bwd(*args, do, dht=dht, h0=d["h0"], cu_seqlens=cu, workspace=ws,
                        cu_seqlens_host=cu_host)
    ref = {n: x.clone() for n, x in ref.items()}
    outs = {n: torch.empty_like(x) for n, x in ref.items()}
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        got = kda.chunk_bwd(*args, do, dht=dht, h0=d["h0"], cu_seqlens=cu, workspace=ws,
                            cu_seqlens_host=cu_host, stream=torch.cuda.current_stream())
        for n in outs:
            outs[n].copy_(got[n])
    names = sorted(ref)
    _replays_match(graph, [outs[n] for n in names], [ref[n] for n in names])


def test_fp32_wide_prefill_in_a_graph():
    """kda_chunk_fwd with fp32 inputs at d = 128 (operand pass and walk) captured."""
    print("case graph: fp32 prefill T=300 H=2 d=128", flush=True)
    d = to_dev(wl.prefill_inputs(T=300, H=2, dk=128, dv=128, dtype="f32", seed=105,
                                 h0_std=0.02))
    args = [d[n] for n in ("q", "k", "v", "g", "beta")]
    ws = torch.empty(kda.chunk_fwd_workspace_size(1, 300, 1, 2, 128, 128,
                                                  io_dtype=kda.KDA_F32),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty(300, 2, 128, dtype=torch.float32, device="cuda")
    ht = torch.empty(1, 2, 128, 128, dtype=torch.float32, device="cuda")
    o_ref, ht_ref = kda.chunk_fwd(*args, h0=d["h0"], workspace=ws)
    o_ref, ht_ref = o_ref.clone(), ht_ref.clone()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        kda.chunk_fwd(*args, h0=d["h0"], o=o, ht=ht, workspace=ws,
                      stream=torch.cuda.current_stream())
    _replays_match(graph, [o, ht], [o_ref, ht_ref])
