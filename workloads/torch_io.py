"""Move storage arrays from the generators onto a torch device (input plumbing only)."""
import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_torch(a: np.ndarray, dtype: str, device=None) -> torch.Tensor:
    """Storage array (float32 / bf16 bits as uint16 / float16) -> torch tensor."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device) if device is not None else t


def from_torch(t: torch.Tensor, dtype: str) -> np.ndarray:
    """torch tensor in the storage dtype -> storage array on the host."""
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
