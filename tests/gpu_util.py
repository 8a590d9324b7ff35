"""Helpers shared by the GPU tests: weight upload, the oracle side of a run
and the acceptance comparisons (per-token cosine and max-abs)."""
import sys

import numpy as np
import torch

import synth
from oracle import ref

COS_MIN = 0.999
ABS_MAX = 3e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upload(W: synth.Weights, device="cuda"):
    """Device tensors of every weight: bf16 patterns as int16 (fp32 values of
    the same bf16 draws for a shape of the fp32 debug build), vectors fp32."""
    out = {}
    f32 = getattr(W.shape, "precision", "bf16") == "fp32"
    for name in W.names():
        r = W.raw(name)
        if r.dtype == np.uint16 and not f32:
            out[name] = torch.from_numpy(r.view(np.int16)).to(device)
        elif r.dtype == np.uint16:
            out[name] = torch.from_numpy(W.f64(name).astype(np.float32)).to(device)
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(r, dtype=np.float32)).to(device)
    return out


def per_token_check(gpu, ora, what, cos_min=COS_MIN, abs_max=ABS_MAX):
    """gpu, ora: [..., n] arrays; cosine per row and max-abs over all."""
    g = np.asarray(gpu, dtype=np.float64).reshape(-1, gpu.shape[-1])
    o = np.asarray(ora, dtype=np.float64).reshape(-1, ora.shape[-1])
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    cos = np.sum(g * o, axis=1) / (np.linalg.norm(g, axis=1) * np.linalg.norm(o, axis=1))
    mad = np.max(np.abs(g - o))
    assert cos.min() >= cos_min, f"{what}: min cosine {cos.min():.6f} (row {int(cos.argmin())})"
    assert mad <= abs_max, f"{what}: max-abs {mad:.3e}"
    return float(cos.min()), float(mad)


def oracle_model(shape, W):
    return ref.OracleModel(shape, W.f64)


def cuda_available():
    return torch.cuda.is_available()
