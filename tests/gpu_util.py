"""Helpers for the GPU parity tests: host<->device copies and comparisons."""
import numpy as np
import torch

from fp8_fp4_tensor_amd import fq


def dev(x: np.ndarray) -> torch.Tensor:
    """numpy fp32, or uint16 bf16 bits, -> a CUDA tensor of that dtype."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return torch.from_numpy(x).cuda()
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    raise TypeError(x.dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def in_dtype(x: np.ndarray) -> int:
    return fq.FQ_IN_BF16 if x.dtype == np.uint16 else fq.FQ_IN_F32


def shape2(x: np.ndarray):
    return (1, x.shape[0]) if x.ndim == 1 else x.shape


def same_bytes(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.astype(np.float32).view(np.uint32)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} differ; first at {bad[0]}: "
                           f"gpu {got[bad[0]]:#x} oracle {want[bad[0]]:#x}")


def f32(v) -> np.ndarray:
    return np.array([v], np.float32)
