"""Helpers shared by the GPU parity tests (device transfer, error metrics)."""
import numpy as np
import torch

from _libutil import ensure_built


def setup():
    ensure_built()
    import bit_block_quantized_nvfp4_amd as moe

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    moe.moe_init()
    return moe


def x_dev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> float64 numpy (exact)."""
    b = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    return (b << 16).view(np.float32).astype(np.float64)


def normwise(a: np.ndarray, ref: np.ndarray) -> float:
    """max |a - ref| / max |ref| over the whole array."""
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(a - ref)) / den) if den > 0 else float(np.max(np.abs(a)))


def flush(msg: str):
    print(msg, flush=True)
