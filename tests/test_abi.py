"""The C ABI without a GPU: every symbol include/kda.h declares is exported, and host-side
validation returns its status codes before anything is launched. Device pointers here are
fake addresses: validation never dereferences them, and no case reaches a launch."""
import ctypes
import os
import re

import pytest

import linear_attention_recurrence_chunk_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, DTYPE, ALIGN, SEQ, WS, UNSUP, LAUNCH, ALIAS, VALUE = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(kda.library_path())
    names = declared_functions()
    assert {"kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_segment_cp_fwd",
            "kda_segment_cp_workspace_size",
            "kda_decode_replay", "kda_status_string", "kda_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert kda.version() == 1
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, SEQ, WS, UNSUP, LAUNCH, ALIAS, VALUE):
        s = kda.status_string(code)
        assert s and s != "unknown status"
    assert kda.status_string(-99) == "unknown status"


# ----------------------------------------------------------------------------- prefill
BASE = 1 << 40          # fake, 16-byte aligned device addresses far apart
GiB = 1 << 30


def ptrs(n=9):
    return [ctypes.c_void_p(BASE + i * 64 * GiB) for i in range(n)]


def chunk(q=True, k=True, v=True, g=True, beta=True, h0=None, cu=None, cu_host=None, batch=1,
          seq_len=256, n_seqs=1, H=2, dk=128, dv=128, io=BF16, out=None, scale=1.0,
          g_min=-5.0, o=True, ht=None, override=None):
    P = ptrs()
    args = dict(q=P[0] if q else None, k=P[1] if k else None, v=P[2] if v else None,
                g=P[3] if g else None, beta=P[4] if beta else None, h0=h0, cu=cu,
                cu_host=cu_host, o=P[5] if o else None, ht=ht)
    if override:
        args.update(override)
    return kda.library().kda_chunk_fwd(
        args["q"], args["k"], args["v"], args["g"], args["beta"], args["h0"], args["cu"],
        args["cu_host"], batch, seq_len, n_seqs, H, dk, dv, io, io if out is None else out,
        scale, g_min, args["o"], args["ht"], args.get("ckpt_every", 0), args.get("ckpt"),
        args.get("ws"), args.get("ws_bytes", 0), None)


def host_cu(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def test_chunk_null_arguments():
    for name in ("q", "k", "v", "g", "beta", "o"):
        assert chunk(**{name: False}) == NULL


def test_chunk_dtype_shape_value_checks():
    assert chunk(io=7) == DTYPE
    assert chunk(io=F32, out=BF16, dk=64, dv=64) == DTYPE       # bf16 output of fp32 input
    assert chunk(H=0) == SHAPE
    assert chunk(seq_len=-1) == SHAPE
    assert chunk(n_seqs=2) == SHAPE                             # batch 1 without cu_seqlens
    assert chunk(dk=96, dv=96) == UNSUP
    assert chunk(dk=128, dv=64) == UNSUP
    assert chunk(io=F32, dk=128, dv=64) == UNSUP
    assert chunk(io=F32, dk=128, dv=128) == WS                  # fp32 at d = 128 needs a workspace
    assert chunk(g_min=-6.0) == VALUE
    assert chunk(g_min=0.5) == VALUE
    assert chunk(scale=float("nan")) == VALUE


def test_chunk_alignment_and_aliasing():
    P = ptrs()
    assert chunk(override={"q": ctypes.c_void_p(BASE + 8)}) == ALIGN
    assert chunk(override={"o": P[0]}) == ALIAS                 # o on top of q
    assert chunk(override={"o": ctypes.c_void_p(P[1].value + 64)}) == ALIAS  # inside k
    h0 = ctypes.c_void_p(BASE + 7 * 64 * GiB)
    ht_bad = ctypes.c_void_p(h0.value + 256)
    assert chunk(h0=h0, ht=ht_bad) == ALIAS                     # partial overlap of ht and h0


def test_chunk_cu_seqlens_checks():
    dev_cu = ctypes.c_void_p(BASE + 8 * 64 * GiB)
    arr, cu_host = host_cu([0, 100, 50, 300])                   # decreasing
    assert chunk(cu=dev_cu, cu_host=cu_host, seq_len=300, n_seqs=3) == SEQ
    arr, cu_host = host_cu([1, 100, 300])                       # not starting at 0
    assert chunk(cu=dev_cu, cu_host=cu_host, seq_len=300, n_seqs=2) == SEQ
    arr, cu_host = host_cu([0, 100, 299])                       # not ending at T
    assert chunk(cu=dev_cu, cu_host=cu_host, seq_len=300, n_seqs=2) == SEQ
    arr, cu_host = host_cu([0, 100, 300])
    assert chunk(cu=dev_cu, cu_host=None, seq_len=300, n_seqs=2) == NULL   # host copy missing
    assert chunk(cu=dev_cu, cu_host=cu_host, seq_len=300, n_seqs=2, batch=2) == SHAPE
    assert chunk(cu=ctypes.c_void_p(dev_cu.value + 4), cu_host=cu_host, seq_len=300,
                 n_seqs=2) == ALIGN


def chunk_ws_size(batch=1, seq_len=8192, n_seqs=1, H=96, dk=128, dv=128, io=BF16, policy=1,
                  cu=None):
    out = ctypes.c_size_t(123)
    st = kda.library().kda_chunk_fwd_workspace_size(batch, seq_len, n_seqs, cu, H, dk, dv, io,
                                                    policy, ctypes.byref(out))
    return st, out.value


def test_chunk_workspace_size():
    """Two-launch workspace: (T / 64 + N + 1) chunk slots x heads x one slot, a slot being
    the MFMA fragments of one chunk's serial-step operands (1 KiB each) plus its decay."""
    slot128 = (8 * 4 + 24 + 2 * 8 + 1) * 1024
    slot64 = (8 * 2 + 24 + 2 * 4 + 1) * 1024
    assert chunk_ws_size() == (OK, (8192 // 64 + 1 + 1) * 96 * slot128)
    # packed sequences: seq_len is the token total, n_seqs the sequence count
    assert chunk_ws_size(seq_len=1000, n_seqs=5, H=3) == (OK, (1000 // 64 + 5 + 1) * 3 * slot128)
    assert chunk_ws_size(batch=4, seq_len=300, n_seqs=4, H=2, dk=64, dv=64) == (
        OK, (1200 // 64 + 4 + 1) * 2 * slot64)
    # fp32 at d = 128: operand blocks of the 16-token chunk form, (T / 16 + N + 1) x heads x
    # (three 16 x 128 tiles, two 16 x 16 matrices, 128 decay factors, 16 betas) fp32
    block = (3 * 16 * 128 + 2 * 256 + 128 + 16) * 4
    assert chunk_ws_size(io=F32) == (OK, (8192 // 16 + 1 + 1) * 96 * block)
    arr, cu = host_cu([0, 100, 1100, 1300])
    assert chunk_ws_size(io=F32, seq_len=1300, n_seqs=3, H=3, policy=2, cu=cu) == (
        OK, (1000 // 16 + 1 + 1) * 3 * block)
    assert chunk_ws_size(io=F32, seq_len=1300, n_seqs=3, H=3, policy=0, cu=cu) == (
        OK, (1300 // 16 + 3 + 1) * 3 * block)
    # fp32 at d = 64 and unsupported widths never take a two-launch path
    assert chunk_ws_size(io=F32, dk=64, dv=64) == (OK, 0)
    assert chunk_ws_size(io=F32, dk=64, dv=64, policy=0) == (OK, 0)
    assert chunk_ws_size(dk=96, dv=96) == (OK, 0)
    assert chunk_ws_size(policy=3)[0] == VALUE
    # the least the two-launch path accepts: the longest sequence's slots
    arr, cu = host_cu([0, 100, 1100, 1300])
    assert chunk_ws_size(seq_len=1300, n_seqs=3, H=3, policy=2, cu=cu) == (
        OK, (1000 // 64 + 1 + 1) * 3 * slot128)
    assert chunk_ws_size(batch=4, seq_len=300, n_seqs=4, H=2, policy=2) == (
        OK, (300 // 64 + 1 + 1) * 2 * slot128)
    assert chunk_ws_size(io=5)[0] == DTYPE
    assert chunk_ws_size(H=0)[0] == SHAPE
    assert kda.library().kda_chunk_fwd_workspace_size(1, 64, 1, None, 2, 128, 128, BF16, 1,
                                                      None) == NULL


def test_chunk_workspace_checks():
    P = ptrs()
    _, need = chunk_ws_size(seq_len=256, H=2)
    ws = ctypes.c_void_p(BASE + 20 * 64 * GiB)
    assert chunk(override=dict(ws=ctypes.c_void_p(ws.value + 8), ws_bytes=need)) == ALIGN
    assert chunk(override=dict(ws=ws, ws_bytes=need - 16)) == WS     # one sequence: all of it
    assert chunk(override=dict(ws=P[2], ws_bytes=need)) == ALIAS          # overlaps v
    assert chunk(override=dict(ws=ctypes.c_void_p(P[5].value - 1024), ws_bytes=need)) == ALIAS
    # an fp32 call at d = 64 ignores the workspace, as documented
    assert chunk(io=F32, dk=64, dv=64, q=False, override=dict(ws=ws, ws_bytes=0)) == NULL
    # fp32 at d = 128: the workspace is required, aligned, large enough, and overlaps nothing
    _, need32 = chunk_ws_size(seq_len=256, H=2, io=F32)
    assert chunk(io=F32, override=dict(ws=ws, ws_bytes=need32 - 16)) == WS
    assert chunk(io=F32, override=dict(ws=ctypes.c_void_p(ws.value + 8), ws_bytes=need32)) == ALIGN
    assert chunk(io=F32, override=dict(ws=P[2], ws_bytes=need32)) == ALIAS


def test_chunk_checkpoint_checks():
    P = ptrs()
    ck = ctypes.c_void_p(BASE + 30 * 64 * GiB)
    assert chunk(override=dict(ckpt_every=100, ckpt=ck)) == SHAPE        # not a multiple of 64
    assert chunk(override=dict(ckpt_every=-64, ckpt=ck)) == SHAPE
    assert chunk(override=dict(ckpt_every=128, ckpt=None)) == NULL
    assert chunk(override=dict(ckpt_every=128, ckpt=ctypes.c_void_p(ck.value + 4))) == ALIGN
    assert chunk(override=dict(ckpt_every=128, ckpt=P[3])) == ALIAS       # on top of g
    assert chunk(override=dict(ckpt_every=128, ckpt=ctypes.c_void_p(P[5].value + 64))) == ALIAS


def test_segment_workspace_size():
    lib = kda.library()
    out = ctypes.c_size_t(0)

    def size(n_seg, io=F32, batch=1, seq_len=262144, n_seqs=1, H=12):
        st = lib.kda_segment_cp_workspace_size(batch, seq_len, n_seqs, H, 128, 128, io, n_seg,
                                               ctypes.byref(out))
        return st, out.value
    # [P | Q] summaries plus entering states: N * n_seg * H * d_k * (d_k + 2 d_v) fp32
    seg64 = 1 * 64 * 12 * 128 * (128 + 256) * 4
    assert size(64) == (OK, seg64)
    assert size(0) == (OK, seg64)                              # automatic choice: 64 segments
    # bf16 inputs add the two-launch operand slots: (T / 64 + N + 1) x H x 74752 B
    assert size(64, io=BF16) == (OK, seg64 + (262144 // 64 + 2) * 12 * 74752)
    assert size(257)[0] == SHAPE
    assert size(4, io=9)[0] == DTYPE
    assert lib.kda_segment_cp_workspace_size(1, 256, 1, 12, 128, 128, F32, 4, None) == NULL


def test_segment_workspace_checks():
    lib = kda.library()
    P = ptrs()
    need = 1 * 4 * 2 * 128 * 384 * 4
    ws = ctypes.c_void_p(BASE + 8 * 64 * GiB)

    def seg(n_seg=4, ws_ptr=ws, ws_bytes=need, o=P[5]):
        return lib.kda_segment_cp_fwd(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, 256, 1,
                                      2, 128, 128, BF16, BF16, 1.0, -5.0, o, None, n_seg,
                                      ws_ptr, ws_bytes, None)
    assert seg(ws_bytes=need - 1) == WS
    assert seg(ws_ptr=None) == NULL
    assert seg(ws_ptr=ctypes.c_void_p(ws.value + 4)) == ALIGN
    assert seg(ws_ptr=P[0]) == ALIAS                            # workspace on top of q
    assert seg(n_seg=-1) == SHAPE
    assert seg(o=None) == NULL


# ----------------------------------------------------------------------------- decode
def window(slots, with_z=True, base=0):
    P = [ctypes.c_void_p(BASE + (20 + base + i) * 64 * GiB) for i in range(6)]
    return kda.TokenWindow(P[0], P[1], P[2], P[3], P[4], P[5] if with_z else None, slots)


def decode(R=4, H=2, D=128, W=4, n_new=8, prev=None, cur=None, act=1, g_min=-5.0,
           eps_l2=1e-6, eps_rms=1e-6, out=BF16, override=None):
    P = [ctypes.c_void_p(BASE + (40 + i) * 64 * GiB) for i in range(7)]
    a = dict(n_acc=P[0], conv_w=P[1], norm_w=P[2], state=P[3], state_acc=P[4], tail=P[5], o=P[6])
    if override:
        a.update(override)
    prev = prev if prev is not None else window(8, with_z=False)
    cur = cur if cur is not None else window(8, base=10)
    return kda.library().kda_decode_replay(
        R, H, D, D, W, n_new, a["n_acc"], a.get("n_new_r"), ctypes.byref(prev), ctypes.byref(cur),
        a["conv_w"],
        a["norm_w"], 1.0, g_min, eps_l2, eps_rms, act, a["state"], a["state_acc"], a["tail"],
        a["o"], out, None)


def test_decode_checks():
    assert decode(override={"state": None}) == NULL
    assert decode(override={"tail": None}) == NULL              # width 4 needs a tail
    assert decode(cur=window(8, with_z=False, base=10)) == NULL  # z of the current window
    assert decode(W=5) == SHAPE
    assert decode(n_new=9) == SHAPE                              # more new tokens than slots
    assert decode(n_new=0) == SHAPE
    assert decode(prev=window(17, with_z=False)) == SHAPE
    assert decode(D=96) == UNSUP
    assert decode(act=2) == VALUE
    assert decode(eps_l2=0.0) == VALUE
    assert decode(g_min=1.0) == VALUE
    assert decode(out=5) == DTYPE
    assert decode(override={"o": ctypes.c_void_p(BASE + (40 + 6) * 64 * GiB + 2)}) == ALIGN
    same = ctypes.c_void_p(BASE + 43 * 64 * GiB)
    assert decode(override={"state_acc": same}) == ALIAS        # state_acc on top of state
    # per-request new-token counts: aligned, and never written over by an output
    assert decode(override={"n_new_r": ctypes.c_void_p(BASE + 50 * 64 * GiB + 4)}) == ALIGN
    assert decode(override={"n_new_r": ctypes.c_void_p(BASE + (40 + 6) * 64 * GiB)}) == ALIAS


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """No silent fallback: with the shared library absent, a call raises."""
    monkeypatch.setattr(kda, "_LIB", None)
    monkeypatch.setattr(kda, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="libkda.so not found"):
        kda.library()


def raw_call(W=4, act=1, eps=1e-6, dk=128, dv=128, conv_w=True, tail_in=None, tail_out=None,
             ws=True, ws_bytes=None, T=256, H=2):
    P = [ctypes.c_void_p(BASE + (60 + i) * 64 * GiB) for i in range(12)]
    need = ctypes.c_size_t(0)
    kda.library().kda_chunk_fwd_raw_workspace_size(1, T, 1, H, dk, dk, ctypes.byref(need))
    return kda.library().kda_chunk_fwd_raw(
        P[0], P[1], P[2], P[3], P[4], P[5] if conv_w else None, tail_in, tail_out, None, None,
        None, 1, T, 1, H, dk, dv, W, act, eps, 1.0, -5.0, P[6], None, BF16,
        P[7] if ws else None, need.value if ws_bytes is None else ws_bytes, None)


def test_raw_prefill_checks():
    out = ctypes.c_size_t(0)
    assert kda.library().kda_chunk_fwd_raw_workspace_size(1, 256, 1, 2, 128, 128,
                                                          ctypes.byref(out)) == OK
    # fp32 convolved values plus the operand slots
    assert out.value == 256 * 2 * 128 * 4 + (256 // 64 + 2) * 2 * 74752
    assert raw_call(conv_w=False) == NULL
    assert raw_call(ws=False) == NULL
    assert raw_call(W=5) == SHAPE
    assert raw_call(W=0) == SHAPE
    assert raw_call(act=2) == VALUE
    assert raw_call(eps=0.0) == VALUE
    assert raw_call(dv=64) == UNSUP
    assert raw_call(ws_bytes=16) == WS
    same = ctypes.c_void_p(BASE + 80 * 64 * GiB)
    assert raw_call(tail_in=same, tail_out=same) == ALIAS          # tails must not overlap
    assert raw_call(tail_out=ctypes.c_void_p(BASE + 60 * 64 * GiB)) == ALIAS   # on top of q


# ----------------------------------------------------------------- no-allocation prefill
def noalloc(seq_len=256, H=2, dk=128, io=BF16, cu=None, cu_host=None, n_seqs=1, o=True):
    P = ptrs()
    return kda.library().kda_chunk_fwd_noalloc(
        P[0], P[1], P[2], P[3], P[4], None, cu, cu_host, 1, seq_len, n_seqs, H, dk, dk, io, io,
        1.0, -5.0, P[5] if o else None, None, 0, None, None)


def test_noalloc_rejects_what_its_scratch_cannot_hold():
    """kda_chunk_fwd_noalloc validates like kda_chunk_fwd, then rejects a sequence whose
    operand slots exceed the 256 MiB static scratch, all before any HIP call: a sequence of T
    tokens takes floor(T / 64) + 2 slots of 74752 B per head (d = 128), so at 96 heads it holds
    (floor(2^28 / (74752 x 96)) - 1) x 64 - 1 = 2303 tokens at most."""
    too_small = -11
    assert kda.status_string(too_small) != "unknown status"
    slots = (256 << 20) // (74752 * 96)
    limit = (slots - 1) * 64 - 1
    assert limit == 2303 and (limit // 64 + 2) * 74752 * 96 <= 256 << 20
    assert ((limit + 1) // 64 + 2) * 74752 * 96 > 256 << 20
    assert noalloc(seq_len=limit + 1, H=96) == too_small
    # packed sequences: the longest one counts, not the total
    arr, cu_host = host_cu([0, 2000, 2000 + limit + 1])
    assert noalloc(seq_len=2000 + limit + 1, H=96, n_seqs=2, cu=ctypes.c_void_p(BASE + 8 * GiB),
                   cu_host=cu_host) == too_small
    # ordinary validation comes first
    assert noalloc(o=False) == NULL
    assert noalloc(dk=96) == UNSUP


# ----------------------------------------------------------------------------- backward
def bwd(io=BF16, dk=128, H=2, seq_len=256, ws_bytes=None, override=None):
    P = ptrs(16)
    a = dict(q=P[0], k=P[1], v=P[2], g=P[3], beta=P[4], do=P[5], dq=P[6], dk=P[7], dv=P[8],
             dg=P[9], dbeta=P[10], dh0=None, ws=P[11])
    if override:
        a.update(override)
    need = ctypes.c_size_t(1 << 30)
    kda.library().kda_chunk_bwd_workspace_size(1, seq_len, 1, H, dk, dk, ctypes.byref(need))
    return kda.library().kda_chunk_bwd(
        a["q"], a["k"], a["v"], a["g"], a["beta"], None, None, None, 1, seq_len, 1, H, dk, dk,
        io, 1.0, -5.0, a["do"], None, a["dq"], a["dk"], a["dv"], a["dg"], a["dbeta"], a["dh0"],
        a["ws"], need.value if ws_bytes is None else ws_bytes, None)


def test_backward_validation():
    for name in ("do", "dq", "dk", "dv", "dg", "dbeta", "ws"):
        assert bwd(override={name: None}) == NULL
    assert bwd(io=5) == DTYPE
    assert bwd(dk=96) == UNSUP
    assert bwd(ws_bytes=1024) == WS
    assert bwd(override={"dq": ctypes.c_void_p(BASE + 0 * 64 * GiB)}) == ALIAS   # dq on q
    assert bwd(override={"dk": ctypes.c_void_p(BASE + 6 * 64 * GiB)}) == ALIAS   # dk on dq
    assert bwd(override={"dg": ctypes.c_void_p(BASE + 9 * 64 * GiB + 4)}) == ALIGN
    need = ctypes.c_size_t(0)
    assert kda.library().kda_chunk_bwd_workspace_size(1, 1024, 1, 4, 128, 128,
                                                       ctypes.byref(need)) == OK
    # per 16-token chunk slot (1024 / 16 + 1 sequence + 1) and head: the entering state and
    # the leaving state's gradient (d_k x d_v each), four 16 x d_v row blocks, and the operand
    # block (three 16 x d_k tiles, two 16 x 16 matrices, d_k decay factors, 16 betas)
    slots = 1024 // 16 + 2
    op_block = 3 * 16 * 128 + 2 * 256 + 128 + 16
    assert need.value == slots * 4 * (2 * 128 * 128 + 4 * 16 * 128 + op_block) * 4
