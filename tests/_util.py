"""Test helpers: moving seeded inputs to the GPU and back (no method arithmetic)."""
import numpy as np
import torch


def to_dev(arr: np.ndarray, device) -> torch.Tensor:
    """uint16 arrays are bfloat16 bit patterns; float32 stays float32."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def symmetric_f32(F: np.ndarray) -> np.ndarray:
    """float32 copy made exactly symmetric from the upper triangle."""
    F32 = np.asarray(F, dtype=np.float32)
    out = np.empty_like(F32)
    for g in range(F32.shape[0]):
        u = np.triu(F32[g])
        out[g] = u + np.triu(F32[g], 1).T
    return np.ascontiguousarray(out)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
