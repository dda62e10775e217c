"""Helpers shared by the GPU tests (comparison and conversions only)."""
import numpy as np
import pytest
import torch

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    g, r = as_f64(got), as_f64(ref)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g - r))


def tol_for(act: str) -> float:
    """Output tolerance (relative L2 over the whole output, in fp64)."""
    return 1e-5 if act == "f32" else 2e-3


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def banner(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
