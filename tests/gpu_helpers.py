"""Helpers for the GPU parity tests: moving seeded inputs between numpy (the
oracle's side) and torch GPU tensors (the library's side)."""
import numpy as np


def torch_mod():
    import torch
    return torch


def require_gpu():
    torch = torch_mod()
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on a CPU host)"
    import paged_kv_cache_attn_amd as pa
    return pa


def to_gpu(a: np.ndarray):
    """fp32 -> torch.float32, uint16 bf16 bits -> torch.bfloat16, ints unchanged."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t) -> np.ndarray:
    """torch tensor -> numpy (bf16 as uint16 bit patterns)."""
    torch = torch_mod()
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_to_f64(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (RNE via fp32) and widen back, for bf16 outputs."""
    torch = torch_mod()
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.bfloat16).double().numpy()


def max_err(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


TOL = {"f32": 1e-5, "bf16": 2e-3}
