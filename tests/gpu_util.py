"""Host<->device conversions for the GPU parity tests (bf16 bit patterns <-> torch tensors)."""
import numpy as np
import pytest
import torch

from synth_inputs import bf16_bits_to_f32

DEV = "cuda:0"


def have_gpu() -> bool:
    return torch.cuda.is_available()


def require_gpu():
    if not have_gpu():
        pytest.skip("no GPU")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 bf16 bits or float32 numpy -> device tensor of the matching torch dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> exact float64 numpy copy."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def tol(dtype: str) -> float:
    """Normwise max relative error bounds: 1e-4 for the fp32 path, 2e-2 for bf16."""
    return 1e-4 if dtype == "f32" else 2e-2
