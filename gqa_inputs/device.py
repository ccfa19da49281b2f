"""Host -> device copies of the seeded inputs (torch owns device memory).

bf16 tensors travel as their raw uint16 bit patterns and are viewed as
torch.bfloat16 on the device; everything else is copied as is.
"""
import numpy as np
import torch


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).cuda().view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()
