"""Shared test helpers: host <-> device marshalling only (no method arithmetic)."""
import numpy as np


def to_dev(x: np.ndarray):
    """numpy float32 or bf16 bit patterns (uint16) -> device tensor of that dtype."""
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t) -> np.ndarray:
    """Device tensor -> numpy (bf16 comes back as uint16 bit patterns)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def lib_built() -> bool:
    import os
    here = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    return os.path.exists(os.path.join(here, "binary_ternary_matmul_amd", "libbwta.so"))
