"""Device-resident layer weights and workspace (torch used for memory only)."""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import _lib


class DeviceLayer:
    """Uploads one layer's host arrays (router_w, gate, up, down, sh_*) to HBM
    and keeps the C descriptor that points at them."""

    def __init__(self, arrays: Dict[str, np.ndarray], H: int, E: int, k: int, I: int, Is: int,
                 shared_weight: float = 1.0, device: str = "cuda", weight_format: int = 0):
        import torch
        # the matrix-core router (more than 32 rows) splits 2^10 * router_w
        # into two fp16 parts: it needs |router_w| < 64 (include/moe.h,
        # router_topk); the host copy is checked once here, at upload
        wr = arrays["router_w"]
        if not np.all(np.abs(wr) < 64.0):
            raise ValueError("router_w must be finite with |router_w| < 64")
        self.H, self.E, self.k, self.I, self.Is = H, E, k, I, Is
        self.weight_format = weight_format
        self.shared_weight = shared_weight
        self.device = device
        self.t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(device) for n, a in arrays.items()}
        self.desc = self._make_desc(self.t)

    @classmethod
    def from_shape(cls, arrays, shape, device="cuda"):
        return cls(arrays, shape.H, shape.E, shape.k, shape.I, shape.Is, shape.shared_weight, device,
                   getattr(shape, "fmt", 0))

    def _make_desc(self, t):
        return _lib.make_desc(self.H, self.E, self.k, self.I, self.Is, self.shared_weight,
                              t["router_w"], t["gate"], t["up"], t["down"], t.get("sh_gate"),
                              t.get("sh_up"), t.get("sh_down"), self.weight_format)

    def clone_weights(self):
        """Another copy of the weights at different addresses (for cache-cold timing)."""
        import torch
        other = object.__new__(DeviceLayer)
        other.__dict__.update(self.__dict__)
        other.t = {n: v.clone() for n, v in self.t.items()}
        torch.cuda.synchronize()
        other.desc = other._make_desc(other.t)
        return other

    def workspace(self, T: int, num_shards: int = 1):
        """A workspace for T rows.  The library needs no particular contents; it
        is filled with 0xFF bytes (NaN as fp16 and fp32) so that a kernel that
        read workspace it had not written would show in its results."""
        import torch
        nbytes = _lib.moe_workspace_bytes(self.desc, T, num_shards)
        if nbytes == 0 and T > 0:
            raise ValueError("invalid layer description")
        return torch.full((max(nbytes, 256),), 255, dtype=torch.uint8, device=self.device)
