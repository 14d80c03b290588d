"""Shared helpers of the GPU parity tests (layout conversions and metrics)."""
import sys

import numpy as np
import torch


def say(*a):
    """Names the case before a GPU step (flushed, so a fault still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def canon(t: torch.Tensor) -> np.ndarray:
    """Logical [B, L, H, D] tensor -> float32 numpy [B, H, L, D] (exact upcast)."""
    return t.detach().float().permute(0, 2, 1, 3).contiguous().cpu().numpy()


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.uint8).numpy()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from quantized_attention_block_amd import sage
    sage.lib()
    return torch.device("cuda", 0)
