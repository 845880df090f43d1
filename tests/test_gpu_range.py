"""Where the fp16 operands' range ends (the bound stated in include/kda.h).

Several of the bf16 path's products take fp16 operands (the state among them). In the method's
regime (unit-norm q and k, beta in [0, 1], g <= 0) each token adds at most v_c^2 to the squared
norm of state column c, so |S| <= sqrt(|h0 column|^2 + sum_t v_{t,c}^2); the header names a
sum of about 1e9 as the edge. These cases sit just inside it, with the values or the entering
state scaled up, and both prefill forms must stay finite and within the bf16 bar."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import workloads as wl
from oracle import kda_oracle as ko
from kda_testutil import TOL_BF16, np64, rel_max_err

pytestmark = pytest.mark.gpu


def _column_bound(inp):
    """max over heads and value columns of |h0 column|^2 + sum_t v_{t,c}^2"""
    v = np64(inp["v"])
    s = (v * v).sum(axis=0)                      # [H, dv]
    if inp["h0"] is not None:
        h0 = np64(inp["h0"])[0]
        s = s + (h0 * h0).sum(axis=1)            # [H, dv]: over key rows
    return float(s.max())


@pytest.mark.parametrize("case", ["values", "state"])
@pytest.mark.parametrize("two_launch", [False, True])
def test_near_the_fp16_edge(case, two_launch):
    T, H, d = 512, 2, 128
    print(f"case fp16 edge {case} two_launch={two_launch}", flush=True)
    inp = wl.prefill_inputs(T=T, H=H, dk=d, dv=d, dtype="f32", seed=21, h0_std=0.02)
    if case == "values":
        # per-column sums of v^2 about 5e8
        inp["v"] = inp["v"] * 990.0
    else:
        # an entering state of column norm about 2e4 (elements up to ~1e4)
        inp["h0"] = inp["h0"] * (2.0e4 / (0.02 * np.sqrt(d)))
    inp["q"], inp["k"], inp["v"] = (inp[x].to(torch.bfloat16) for x in ("q", "k", "v"))
    bound = _column_bound(inp)
    assert 2.5e8 <= bound <= 1e9, bound
    dev = {x: (t.cuda() if isinstance(t, torch.Tensor) else t) for x, t in inp.items()}
    ws = None
    if two_launch:
        n = kda.chunk_fwd_workspace_size(1, T, 1, H, d, d, policy=kda.KDA_CHUNK_WS_TWO_PASS)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o, ht = kda.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], h0=dev["h0"],
                          out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ht).all()
    o_ref, ht_ref = ko.recurrence_fwd(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]),
                                      np64(inp["g"]), np64(inp["beta"]), h0=np64(inp["h0"]))
    e_o, e_s = rel_max_err(np64(o), o_ref), rel_max_err(np64(ht), ht_ref)
    print(f"column bound {bound:.2e}: max|S| {np.abs(ht_ref).max():.2e} err_o={e_o:.2e} "
          f"err_state={e_s:.2e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
