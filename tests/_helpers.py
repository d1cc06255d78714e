"""Small shared helpers for the tests: tensor <-> stored-numpy conversion, toy workloads."""
from __future__ import annotations

import numpy as np
import torch


def to_storage(t: torch.Tensor) -> np.ndarray:
    """A host numpy array holding the tensor's stored elements (bf16 as raw uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of ``to_storage`` (host tensor)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def random_storage(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values rounded to the dtype (torch's nearest-even casts), as stored numpy."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return to_storage(x.to(tdt))


NAN_BITS = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}
