"""Host -> device upload of synthetic inputs (plumbing only)."""
from __future__ import annotations

import numpy as np
import torch

from . import synth


def to_device(x) -> torch.Tensor:
    """synth.Tensor or NumPy array -> contiguous CUDA tensor.  bf16 inputs are
    uploaded as their exact bits."""
    if isinstance(x, synth.Tensor):
        if x.dt == "bf16":
            bits = np.ascontiguousarray(x.bits).view(np.int16)
            return torch.from_numpy(bits).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x.f32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()
