"""Helpers shared by the GPU tests: move stored numpy arrays to the device and
compare device results with the oracle."""
import numpy as np
import torch

import oracle

DT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def dev():
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored array (float32 values or uint16 bit patterns) -> device tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(DT_TORCH[dtype]).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (exact for every dtype used here)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a 16-bit tensor as uint16 (or float32 values)."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def assert_close(y: torch.Tensor, ref: np.ndarray, out_dtype: str, what: str = ""):
    m = oracle.metrics(to_np(y), ref, out_dtype)
    assert oracle.within(m, out_dtype), f"{what}: {m}"
    return m
