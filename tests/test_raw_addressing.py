"""CPU address check of the raw-projection prefill (kda_chunk_fwd_raw).

tests/addrcheck/raw_addr_check.cpp replays every global-memory access of the call's prep pass
(raw mode) and walk, thread by thread, with the row, slot and group arithmetic of
csrc/kda_index.h (the header the kernels call), and checks each against the extent of the
buffer it addresses; the walk's reads of convolved values and operand slots must also land on
what the prep pass wrote.

The path faulted the GPU twice (hipErrorIllegalAddress in test_raw_prefill_without_entering_tail,
then in test_raw_prefill_varlen_and_short_sequences[128-4]). Both times the convolution history
of q and k was loaded for every thread of a ragged last chunk, bounded below by the sequence
start only: threads whose rows lie past the chunk's end read up to 62 rows past it, past the
end of q and k for the batch's last sequence. The legacy-predicate cases below reproduce that
on the CPU (the access lands past the allocation), and the current predicate (history rows
also bounded by the chunk's last row) leaves no access out of bounds.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "addrcheck", "raw_addr_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    lib = str(tmp_path_factory.mktemp("addrcheck") / "raw_addr_check.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall", SRC, "-o", lib],
                   check=True)
    so = ctypes.CDLL(lib)
    f = so.kda_raw_addr_check
    f.restype = ctypes.c_longlong
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_longlong), ctypes.c_char_p, ctypes.c_int]

    def run(lengths=None, T=None, B=1, H=2, dk=128, W=4, tail_in=True, tail_out=True, h0=True,
            ht=True, out_bytes=4, workspace=0, legacy=False):
        if lengths is not None:
            cu = np.zeros(len(lengths) + 1, np.int32)
            cu[1:] = np.cumsum(lengths)
            n, seq_len, cu_p = len(lengths), int(cu[-1]), cu.ctypes.data
        else:
            cu, n, seq_len, cu_p = None, B, T, None
        nacc = ctypes.c_longlong(0)
        rep = ctypes.create_string_buffer(4096)
        bad = f(n, cu_p, seq_len, H, dk, W, int(tail_in), int(tail_out), int(h0), int(ht),
                out_bytes, workspace, int(legacy), ctypes.byref(nacc), rep, len(rep))
        return bad, nacc.value, rep.value.decode()
    return run


def _need(lengths, H, dk):
    """kda_chunk_fwd_raw_workspace_size for one sequence of the longest length (the least a
    call accepts): fp32 values [T, H, d] rounded to 256 bytes plus the operand slots."""
    T = max(lengths)
    slot = (8 * (dk // 32) + 24 + 2 * (dk // 16) + 1) * 1024
    return (T * H * dk * 4 + 255) // 256 * 256 + (T // 64 + 2) * H * slot


# the raw GPU tests' calls, plus edge cases: ragged last chunks, sequences shorter than the
# convolution tail, empty sequences, the last sequence of a packed batch, every width
CASES = [
    dict(T=1000, H=3, dk=128, W=4), dict(T=300, H=2, dk=64, W=4), dict(T=130, H=2, dk=128, W=2),
    dict(T=200, H=2, dk=128, W=1), dict(T=200, H=2, dk=128, W=4, tail_in=False),
    dict(lengths=[1, 2, 64, 65, 0, 300, 3, 129], dk=128, W=4),
    dict(lengths=[1, 2, 64, 65, 0, 300, 3, 129], dk=64, W=3),
    dict(lengths=[300, 0, 640, 129, 1024, 64, 1, 500], H=3, dk=128, W=4),
    dict(lengths=[300, 0, 640, 129, 1024, 64, 1, 500], H=3, dk=64, W=4),
    dict(lengths=[64, 130, 1], H=2, dk=128, W=4),
    dict(lengths=[0, 0, 1, 0], H=1, dk=128, W=4), dict(lengths=[2, 1, 3], H=2, dk=64, W=4),
    dict(lengths=[63, 64, 65, 127, 128, 129], H=2, dk=128, W=3, tail_in=False),
    dict(T=1, B=3, H=2, dk=128, W=4), dict(T=64, B=2, H=2, dk=64, W=2),
    dict(T=4100, H=1, dk=128, W=4, out_bytes=2, h0=False, ht=False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: ",".join(f"{k}={v}" for k, v in c.items()))
def test_every_access_in_bounds(checker, case):
    bad, n, rep = checker(**case)
    assert n > 0
    assert bad == 0, rep


@pytest.mark.parametrize("lengths,H,dk", [([300, 0, 640, 129, 1024, 64, 1, 500], 3, 128),
                                           ([300, 0, 640, 129, 1024, 64, 1, 500], 3, 64),
                                           ([1, 2, 64, 65, 0, 300, 3, 129], 2, 128)])
def test_grouped_workspace_in_bounds(checker, lengths, H, dk):
    """The least workspace the call accepts (the longest sequence's values and slots): groups
    of whole sequences, each inside the workspace, values addressed from a shifted base."""
    bad, n, rep = checker(lengths=lengths, H=H, dk=dk, W=4, workspace=_need(lengths, H, dk))
    assert n > 0
    assert bad == 0, rep


@pytest.mark.parametrize("case", [dict(T=200, H=2, dk=128, W=4, tail_in=False),
                                  dict(lengths=[1, 2, 64, 65, 0, 300, 3, 129], dk=128, W=4)],
                         ids=["without_entering_tail", "varlen_128_4"])
def test_fault_cause_reproduced_on_cpu(checker, case):
    """The two faulting GPU tests under the history predicate of the code that faulted:
    reads of q and k past the end of the inputs (a ragged last chunk of the batch's last
    sequence); under the current predicate none."""
    bad, _, rep = checker(**case, legacy=True)
    assert bad > 0
    assert "out of bounds: q" in rep and "history q" in rep
    # the rows read lie past the end of the allocation, not inside another sequence
    assert checker(**case)[0] == 0
