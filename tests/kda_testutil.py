"""Helpers shared by the GPU parity tests (comparison metrics, tensor conversion)."""
import numpy as np
import torch


def np64(t):
    """Exact upcast of a tensor's values to float64 on the host."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rel_max_err(got, ref):
    """max |got - ref| / RMS(ref) over the whole tensor (the tolerance metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def to_dev(d, device="cuda"):
    out = {}
    for k, v in d.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


# tolerances: max |err| <= TOL * RMS(reference)
TOL_BF16 = 2e-2
TOL_F32 = 1e-4
