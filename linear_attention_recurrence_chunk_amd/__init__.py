"""Python binding of libkda (the KDA gated delta-rule recurrence on MI355X).

Argument marshalling only: torch tensors are turned into device pointers and the current
HIP stream, and every step runs in the library's HIP kernels. There is no fallback: if
libkda.so is missing or fails to load, every call raises.

Entry points mirror include/kda.h: ``chunk_fwd``, ``chunk_fwd_workspace_size``,
``segment_cp_fwd``, ``segment_cp_workspace_size``, ``decode_replay``.
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["KDAError", "library", "library_path", "chunk_fwd", "chunk_fwd_workspace_size",
           "chunk_fwd_raw",
           "segment_cp_fwd",
           "segment_cp_workspace_size", "decode_replay", "status_string", "version"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

KDA_F32 = 0
KDA_BF16 = 1
KDA_CHUNK_WS_AUTO = 0
KDA_CHUNK_WS_TWO_PASS = 1
KDA_CHUNK_WS_MIN = 2


class KDAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: libkda status {status} ({status_string(status)})")


class TokenWindow(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("slots", ctypes.c_int)]


def library_path():
    return os.path.join(_HERE, "libkda.so")


def library():
    """Load libkda.so (raises if it is not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libkda.so not found at {path}: build it with "
                           "`python -m linear_attention_recurrence_chunk_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, F, P, P, I,
                                  P, P, ctypes.c_size_t, P]
    lib.kda_chunk_fwd.restype = I
    lib.kda_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, F,
                                          P, P, I, P, P]
    lib.kda_chunk_fwd_noalloc.restype = I
    lib.kda_chunk_bwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, F, P, P, P, P,
                                  P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_chunk_bwd.restype = I
    lib.kda_chunk_bwd_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_chunk_bwd_workspace_size.restype = I
    lib.kda_chunk_fwd_workspace_size.argtypes = [I, I, I, P, I, I, I, I, I,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_chunk_fwd_workspace_size.restype = I
    lib.kda_chunk_fwd_raw.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                      F, F, F, P, P, I, P, ctypes.c_size_t, P]
    lib.kda_chunk_fwd_raw.restype = I
    lib.kda_chunk_fwd_raw_workspace_size.argtypes = [I, I, I, I, I, I,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_chunk_fwd_raw_workspace_size.restype = I
    lib.kda_segment_cp_workspace_size.argtypes = [I, I, I, I, I, I, I, I,
                                                  ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_segment_cp_workspace_size.restype = I
    lib.kda_segment_cp_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, F, P,
                                       P, I, P, ctypes.c_size_t, P]
    lib.kda_segment_cp_fwd.restype = I
    lib.kda_decode_replay.argtypes = [I, I, I, I, I, I, P, P, ctypes.POINTER(TokenWindow),
                                      ctypes.POINTER(TokenWindow), P, P, F, F, F, F, I, P, P, P,
                                      P, I, P]
    lib.kda_decode_replay.restype = I
    lib.kda_status_string.argtypes = [I]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.restype = I
    lib.kda_last_launch_error.restype = I
    _LIB = lib
    return lib


def status_string(status):
    try:
        return library().kda_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - only when the library itself is missing
        return "unknown"


def version():
    return int(library().kda_version())


# ------------------------------------------------------------------------------ helpers
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")


def _io_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise ValueError(f"unsupported io dtype {t.dtype}")


def _out_dtype(q, out_dtype):
    torch = _torch()
    if out_dtype is None:
        return q.dtype
    if out_dtype in (torch.float32, "f32", "float32"):
        return torch.float32
    if out_dtype in (torch.bfloat16, "bf16", "bfloat16"):
        return torch.bfloat16
    raise ValueError(f"unsupported out_dtype {out_dtype}")


def _prefill_args(q, k, v, g, beta, h0, cu_seqlens, o, ht, output_final_state, out_dtype,
                  gate_dtype=None, cu_seqlens_host=None):
    torch = _torch()
    gate_dtype = torch.float32 if gate_dtype is None else gate_dtype
    if q.dim() == 4:                 # [B, T, H, d]
        batch, seq_len, H, dk = q.shape
    elif q.dim() == 3:               # [T, H, d]
        batch, (seq_len, H, dk) = 1, q.shape
    else:
        raise ValueError("q must be [B, T, H, d_k] or [T, H, d_k]")
    dv = v.shape[-1]
    dev = q.device
    io = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, io, dev)
    _check(g, "g", gate_dtype, dev)
    _check(beta, "beta", gate_dtype, dev)
    _check(h0, "h0", torch.float32, dev)
    cu_dev = cu_host = None
    if cu_seqlens is not None:
        if batch != 1:
            raise ValueError("cu_seqlens needs batch 1")
        if cu_seqlens_host is not None:
            # both copies given: nothing is copied here, so the call can be graph-captured
            if cu_seqlens_host.device.type != "cpu" or cu_seqlens_host.dtype != torch.int32:
                raise ValueError("cu_seqlens_host must be a CPU int32 tensor")
            cu_host = cu_seqlens_host.contiguous()
            if cu_host.numel() != cu_seqlens.numel():
                raise ValueError("cu_seqlens_host must match cu_seqlens")
        else:
            cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
        cu_dev = cu_seqlens.to(dev, torch.int32).contiguous()
        n_seqs = cu_host.numel() - 1
    else:
        n_seqs = batch
    odt = _out_dtype(q, out_dtype) if o is None else o.dtype
    if o is None:
        o = torch.empty(*q.shape[:-1], dv, dtype=odt, device=dev)
    _check(o, "o", odt, dev)
    if ht is None and output_final_state:
        ht = torch.empty(n_seqs, H, dk, dv, dtype=torch.float32, device=dev)
    _check(ht, "ht", torch.float32, dev)
    return dict(batch=batch, seq_len=seq_len, H=H, dk=dk, dv=dv, io=_io_dtype(q), out=_io_dtype(o),
                cu_dev=cu_dev, cu_host=cu_host, n_seqs=n_seqs, o=o, ht=ht)


def _cu_host_ptr(cu_host):
    return None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr())


# ------------------------------------------------------------------------------ entry points
def chunk_fwd_workspace_size(batch, seq_len, n_seqs, H, dk, dv, io_dtype=KDA_BF16,
                             policy=KDA_CHUNK_WS_AUTO, cu_seqlens_host=None):
    """kda_chunk_fwd_workspace_size: bytes of workspace for the two-launch path (0 under the
    automatic policy when one launch is recommended). cu_seqlens_host: optional int32 CPU
    tensor of packed-sequence offsets."""
    cu = None
    if cu_seqlens_host is not None:
        cu = cu_seqlens_host.detach().to("cpu", _torch().int32).contiguous()
    out = ctypes.c_size_t(0)
    st = library().kda_chunk_fwd_workspace_size(int(batch), int(seq_len), int(n_seqs),
                                                _cu_host_ptr(cu), int(H), int(dk), int(dv),
                                                int(io_dtype), int(policy), ctypes.byref(out))
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_workspace_size")
    return int(out.value)


def chunk_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=1.0, g_min=-5.0, o=None,
              ht=None, output_final_state=True, out_dtype=None, workspace="auto", ckpt_every=0,
              ckpt=None, stream=None, cu_seqlens_host=None):
    """kda_chunk_fwd. q, k: [B, T, H, d_k] or packed [T, H, d_k]; v: [.., d_v];
    g: same shape as k (fp32); beta: [.., H] (fp32); h0: [N, H, d_k, d_v] fp32 or None;
    cu_seqlens: [N + 1] int32 (any device) for packed varlen input; out_dtype: None (same as
    q) or torch.float32. workspace: "auto" (the library's recommended path, allocating the
    workspace it asks for), None (one launch), "two_pass" (two launches over the whole batch),
    "min" (two launches per group of sequences, the smallest workspace) or a uint8 device
    tensor (two launches, grouped when it is smaller than the whole batch needs). ckpt_every > 0 (a multiple of 64) also returns
    the states after every ckpt_every tokens of each sequence, [T // ckpt_every, H, d_k, d_v]
    fp32 (slot floor(bos_n / ckpt_every) + j for sequence n): (o, ht, ckpt). Returns (o, ht)
    otherwise. cu_seqlens_host: the same offsets as a CPU int32 tensor, when the caller has
    them (with cu_seqlens already int32 on the device, nothing is copied: graph capture)."""
    a = _prefill_args(q, k, v, g, beta, h0, cu_seqlens, o, ht, output_final_state, out_dtype,
                      cu_seqlens_host=cu_seqlens_host)
    T_arg = a["seq_len"] if a["cu_dev"] is None else int(a["cu_host"][-1])
    if isinstance(workspace, str):
        policies = {"auto": KDA_CHUNK_WS_AUTO, "two_pass": KDA_CHUNK_WS_TWO_PASS,
                    "min": KDA_CHUNK_WS_MIN}
        if workspace not in policies:
            raise ValueError(f"unknown workspace policy {workspace!r}")
        need = chunk_fwd_workspace_size(a["batch"], T_arg, a["n_seqs"], a["H"], a["dk"],
                                        a["dv"], a["io"], policies[workspace], a["cu_host"])
        workspace = (_torch().empty(need, dtype=_torch().uint8, device=q.device)
                     if need > 0 else None)
    if ckpt_every and ckpt is None:
        total = a["batch"] * T_arg if a["cu_dev"] is None else T_arg
        ckpt = _torch().empty(total // ckpt_every, a["H"], a["dk"], a["dv"],
                              dtype=_torch().float32, device=q.device)
    _check(ckpt, "ckpt", _torch().float32, q.device)
    st = library().kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(a["cu_dev"]),
        _cu_host_ptr(a["cu_host"]), a["batch"], T_arg, a["n_seqs"], a["H"], a["dk"], a["dv"],
        a["io"], a["out"], float(scale), float(g_min), _ptr(a["o"]), _ptr(a["ht"]),
        int(ckpt_every), _ptr(ckpt) if ckpt_every else None,
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd")
    if ckpt_every:
        return a["o"], a["ht"], ckpt
    return a["o"], a["ht"]


def chunk_bwd_workspace_size(batch, seq_len, n_seqs, H, dk, dv):
    out = ctypes.c_size_t(0)
    st = library().kda_chunk_bwd_workspace_size(batch, seq_len, n_seqs, H, dk, dv,
                                                ctypes.byref(out))
    if st != 0:
        raise KDAError(st, "kda_chunk_bwd_workspace_size")
    return out.value


def chunk_bwd(q, k, v, g, beta, do, dht=None, h0=None, cu_seqlens=None, scale=1.0, g_min=-5.0,
              workspace=None, stream=None, cu_seqlens_host=None, want_dh0=True):
    """kda_chunk_bwd: gradients of chunk_fwd's outputs. do: [.., H, d_v] like o (same dtype as
    q); dht: [N, H, d_k, d_v] fp32 or None. Returns a dict of fp32 tensors dq, dk, dv, dg,
    dbeta and dh0 (None when want_dh0 is False)."""
    torch = _torch()
    a = _prefill_args(q, k, v, g, beta, h0, cu_seqlens, do, None, False, None,
                      cu_seqlens_host=cu_seqlens_host)
    if do.dtype != q.dtype:
        raise ValueError("do must have q's dtype")
    _check(dht, "dht", torch.float32, q.device)
    T_arg = a["seq_len"] if a["cu_dev"] is None else int(a["cu_host"][-1])
    f32 = dict(dtype=torch.float32, device=q.device)
    grads = {"dq": torch.empty(*q.shape, **f32), "dk": torch.empty(*k.shape, **f32),
             "dv": torch.empty(*v.shape, **f32), "dg": torch.empty(*g.shape, **f32),
             "dbeta": torch.empty(*beta.shape, **f32),
             "dh0": (torch.empty(a["n_seqs"], a["H"], a["dk"], a["dv"], **f32)
                     if want_dh0 else None)}
    if workspace is None:
        need = chunk_bwd_workspace_size(a["batch"], T_arg, a["n_seqs"], a["H"], a["dk"], a["dv"])
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = library().kda_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(a["cu_dev"]),
        _cu_host_ptr(a["cu_host"]), a["batch"], T_arg, a["n_seqs"], a["H"], a["dk"], a["dv"],
        a["io"], float(scale), float(g_min), _ptr(do), _ptr(dht), _ptr(grads["dq"]),
        _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]), _ptr(grads["dbeta"]),
        _ptr(grads["dh0"]), _ptr(workspace), workspace.numel(), _stream(stream))
    if st != 0:
        raise KDAError(st, "kda_chunk_bwd")
    return grads


NOALLOC_SCRATCH_BYTES = 256 << 20   # KDA_NOALLOC_SCRATCH_BYTES


def chunk_fwd_noalloc(q, k, v, g, beta, o, ht=None, h0=None, cu_seqlens=None,
                      cu_seqlens_host=None, scale=1.0, g_min=-5.0, ckpt_every=0, ckpt=None,
                      stream=None):
    """kda_chunk_fwd_noalloc: kda_chunk_fwd with the two-launch path's operand slots in the
    library's static per-GPU scratch, for callers that cannot allocate. Nothing is allocated or
    copied here either: o (and ht, ckpt when wanted) must be given, and packed sequences need
    cu_seqlens as a contiguous int32 device tensor plus cu_seqlens_host as a CPU int32
    tensor. Returns (o, ht)."""
    torch = _torch()
    if o is None:
        raise ValueError("chunk_fwd_noalloc allocates nothing: pass o")
    if cu_seqlens is not None and (cu_seqlens_host is None or cu_seqlens.dtype != torch.int32
                                   or cu_seqlens.device != q.device
                                   or not cu_seqlens.is_contiguous()):
        raise ValueError("chunk_fwd_noalloc needs cu_seqlens as a contiguous int32 tensor on "
                         "q's device and cu_seqlens_host as a CPU int32 tensor")
    if ckpt_every and ckpt is None:
        raise ValueError("chunk_fwd_noalloc allocates nothing: pass ckpt")
    a = _prefill_args(q, k, v, g, beta, h0, cu_seqlens, o, ht, False, None,
                      cu_seqlens_host=cu_seqlens_host)
    T_arg = a["seq_len"] if a["cu_dev"] is None else int(a["cu_host"][-1])
    _check(ckpt, "ckpt", torch.float32, q.device)
    st = library().kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(a["cu_dev"]),
        _cu_host_ptr(a["cu_host"]), a["batch"], T_arg, a["n_seqs"], a["H"], a["dk"], a["dv"],
        a["io"], a["out"], float(scale), float(g_min), _ptr(a["o"]), _ptr(a["ht"]),
        int(ckpt_every), _ptr(ckpt) if ckpt_every else None, _stream(stream))
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_noalloc")
    return a["o"], a["ht"]


def chunk_fwd_raw_workspace_size(batch, seq_len, n_seqs, H, dk, dv):
    """kda_chunk_fwd_raw_workspace_size: bytes for the whole batch at once. A smaller workspace,
    down to this size for the longest sequence alone (batch = n_seqs = 1), runs groups of
    whole sequences."""
    need = ctypes.c_size_t(0)
    st = library().kda_chunk_fwd_raw_workspace_size(int(batch), int(seq_len), int(n_seqs),
                                                    int(H), int(dk), int(dv), ctypes.byref(need))
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_raw_workspace_size")
    return need.value


def chunk_fwd_raw(q, k, v, g, beta, conv_w, conv_tail=None, h0=None, cu_seqlens=None,
                  scale=1.0, g_min=-5.0, eps_l2=1e-6, act=1, o=None, ht=None,
                  output_final_state=True, out_dtype=None, workspace=None,
                  conv_tail_out=None, stream=None, cu_seqlens_host=None):
    """kda_chunk_fwd_raw: the prefill from raw bf16 projections q, k, g [.., H, d_k], v
    [.., H, d_v], beta [.., H] with the short convolution (taps conv_w [H, 2 d_k + d_v, W]),
    SiLU (act), L2 input norms and gate activations fused into the prep pass. conv_tail: the
    entering raw tails [N, H, 2 d_k + d_v, W - 1] fp32 or None. Returns (o, ht, tail_out)."""
    torch = _torch()
    a = _prefill_args(q, k, v, g, beta, h0, cu_seqlens, o, ht, output_final_state,
                      out_dtype if out_dtype is not None else torch.bfloat16,
                      gate_dtype=torch.bfloat16, cu_seqlens_host=cu_seqlens_host)
    T_arg = a["seq_len"] if a["cu_dev"] is None else int(a["cu_host"][-1])
    dev = q.device
    _check(conv_w, "conv_w", torch.float32, dev)
    _check(conv_tail, "conv_tail", torch.float32, dev)
    W = conv_w.shape[-1]
    if conv_tail_out is None and W > 1:
        conv_tail_out = torch.empty(a["n_seqs"], a["H"], 2 * a["dk"] + a["dv"], W - 1,
                                    dtype=torch.float32, device=dev)
    _check(conv_tail_out, "conv_tail_out", torch.float32, dev)
    if workspace is None:
        need = ctypes.c_size_t(0)
        st = library().kda_chunk_fwd_raw_workspace_size(a["batch"], T_arg, a["n_seqs"], a["H"],
                                                        a["dk"], a["dv"], ctypes.byref(need))
        if st != 0:
            raise KDAError(st, "kda_chunk_fwd_raw_workspace_size")
        workspace = torch.empty(max(int(need.value), 16), dtype=torch.uint8, device=dev)
    st = library().kda_chunk_fwd_raw(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(conv_w), _ptr(conv_tail),
        _ptr(conv_tail_out) if W > 1 else None, _ptr(h0), _ptr(a["cu_dev"]),
        _cu_host_ptr(a["cu_host"]), a["batch"], T_arg, a["n_seqs"], a["H"], a["dk"], a["dv"],
        int(W), int(act), float(eps_l2), float(scale), float(g_min), _ptr(a["o"]),
        _ptr(a["ht"]), a["out"], _ptr(workspace), workspace.numel(), _stream(stream))
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_raw")
    return a["o"], a["ht"], conv_tail_out


def segment_cp_workspace_size(batch, seq_len, n_seqs, H, dk, dv, io_dtype=KDA_BF16,
                              n_segments=0):
    """kda_segment_cp_workspace_size (batch / seq_len / n_seqs as in kda_chunk_fwd)."""
    out = ctypes.c_size_t(0)
    st = library().kda_segment_cp_workspace_size(int(batch), int(seq_len), int(n_seqs), int(H),
                                                  int(dk), int(dv), int(io_dtype),
                                                  int(n_segments), ctypes.byref(out))
    if st != 0:
        raise KDAError(st, "kda_segment_cp_workspace_size")
    return int(out.value)


def segment_cp_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=1.0, g_min=-5.0,
                   n_segments=0, workspace=None, o=None, ht=None, output_final_state=True,
                   out_dtype=None, stream=None, cu_seqlens_host=None):
    """kda_segment_cp_fwd (same tensors as chunk_fwd, cu_seqlens_host included). ``workspace``
    is a uint8 device tensor of at least segment_cp_workspace_size(...) bytes; allocated here
    if None."""
    torch = _torch()
    a = _prefill_args(q, k, v, g, beta, h0, cu_seqlens, o, ht, output_final_state, out_dtype,
                      cu_seqlens_host=cu_seqlens_host)
    T_arg = a["seq_len"] if a["cu_dev"] is None else int(a["cu_host"][-1])
    need = segment_cp_workspace_size(a["batch"], T_arg, a["n_seqs"], a["H"], a["dk"], a["dv"],
                                     a["io"], n_segments)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = library().kda_segment_cp_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(a["cu_dev"]),
        _cu_host_ptr(a["cu_host"]), a["batch"], a["seq_len"] if a["cu_dev"] is None
        else int(a["cu_host"][-1]), a["n_seqs"], a["H"], a["dk"], a["dv"], a["io"], a["out"],
        float(scale), float(g_min), _ptr(a["o"]), _ptr(a["ht"]), int(n_segments),
        _ptr(workspace), workspace.numel(), _stream(stream))
    if st != 0:
        raise KDAError(st, "kda_segment_cp_fwd")
    return a["o"], a["ht"]


def _window(win, slots):
    return TokenWindow(_ptr(win["q"]), _ptr(win["k"]), _ptr(win["v"]), _ptr(win["g"]),
                       _ptr(win["beta"]), _ptr(win.get("z")), int(slots))


def decode_replay(state, conv_tail, n_acc, prev, new, conv_w, norm_w, n_new=None, scale=1.0,
                  g_min=-5.0, eps_l2=1e-6, eps_rms=1e-6, act=1, state_acc=None, o=None,
                  write_state_acc=True, out_dtype=None, n_new_per_request=None, stream=None):
    """kda_decode_replay. ``state`` [R, H, d_k, d_v] and ``conv_tail`` are updated in place;
    prev / new are dicts of bf16 tensors q, k, v, g, beta (and z for new), each
    [R, slots, H, ...]. out_dtype: None (bf16) or torch.float32.
    n_new_per_request: optional [R] int32 device tensor of new tokens per request (clamped
    to [1, n_new]; rows past a request's count are left untouched).
    Returns (o [R, n_new, H, d_v], state_acc or None)."""
    torch = _torch()
    R, H, dk, dv = state.shape
    dev = state.device
    conv_width = conv_w.shape[-1]
    if n_new is None:
        n_new = new["q"].shape[1]
    _check(state, "state", torch.float32, dev)
    _check(conv_tail, "conv_tail", torch.float32, dev)
    _check(conv_w, "conv_w", torch.float32, dev)
    _check(norm_w, "norm_w", torch.float32, dev)
    _check(n_acc, "n_acc", torch.int32, dev)
    _check(n_new_per_request, "n_new_per_request", torch.int32, dev)
    for win, nm in ((prev, "prev"), (new, "new")):
        for key in ("q", "k", "v", "g", "beta", "z"):
            if win.get(key) is not None:
                _check(win[key], f"{nm}.{key}", torch.bfloat16, dev)
    if state_acc is None and write_state_acc:
        state_acc = torch.empty_like(state)
    _check(state_acc, "state_acc", torch.float32, dev)
    if o is None:
        odt = torch.float32 if out_dtype in (torch.float32, "f32", "float32") else torch.bfloat16
        o = torch.empty(R, n_new, H, dv, dtype=odt, device=dev)
    if o.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("o must be bf16 or fp32")
    _check(o, "o", None, dev)
    pw = _window(prev, prev["q"].shape[1])
    nw = _window(new, new["q"].shape[1])
    st = library().kda_decode_replay(
        R, H, dk, dv, conv_width, int(n_new), _ptr(n_acc), _ptr(n_new_per_request),
        ctypes.byref(pw), ctypes.byref(nw),
        _ptr(conv_w), _ptr(norm_w), float(scale), float(g_min), float(eps_l2), float(eps_rms),
        int(act), _ptr(state), _ptr(state_acc),
        _ptr(conv_tail) if conv_tail.numel() else None, _ptr(o), _io_dtype(o), _stream(stream))
    if st != 0:
        raise KDAError(st, "kda_decode_replay")
    return o, state_acc
