"""Helpers shared by the GPU tests: device transfer of stored inputs and the
numerical bars the HIP path must meet against the fp64 oracle.

Bars (fixed for this operator):
  * fp32 storage: max |gpu - oracle| <= 1e-5 * max |oracle|;
  * bf16 storage: ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2 and
    max |gpu - oracle| <= 3e-2.
"""
import numpy as np
import torch

import oracle


def to_dev(a: np.ndarray) -> torch.Tensor:
    """Stored input (float32 or bf16 bits) -> device tensor of the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).cuda()
    raise TypeError(a.dtype)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> stored representation (float32, or bf16 bits as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_host64(t: torch.Tensor) -> np.ndarray:
    return oracle.widen(to_host_bits(t))


def errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = gpu - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    ref_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    l2 = float(np.linalg.norm(diff))
    rl2 = l2 / max(float(np.linalg.norm(ref)), 1e-300)
    return {"max_abs": max_abs, "ref_max": ref_max, "rel_l2": rl2, "rel_max": max_abs / max(ref_max, 1e-300),
            "finite": bool(np.isfinite(gpu).all())}


def assert_parity(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    e = errors(gpu, ref)
    assert e["finite"], f"{what}: non-finite GPU output"
    if dtype == "f32":
        assert e["rel_max"] <= 1e-5, f"{what}: fp32 max-abs {e['max_abs']:.3e} > 1e-5 * {e['ref_max']:.3e}"
    else:
        assert e["rel_l2"] <= 1e-2, f"{what}: bf16 rel-L2 {e['rel_l2']:.3e} > 1e-2"
        assert e["max_abs"] <= 3e-2, f"{what}: bf16 max-abs {e['max_abs']:.3e} > 3e-2"
    return e


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Tokens to check one by one: head and tail of the sequence plus random ones."""
    if N <= count:
        return np.arange(N, dtype=np.int64)
    edge = min(64, count // 4)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(edge, N - edge), size=count - 2 * edge, replace=False)
    return np.sort(np.concatenate([np.arange(edge), mid, np.arange(N - edge, N)])).astype(np.int64)
