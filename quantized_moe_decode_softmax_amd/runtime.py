"""Device-memory helper around the C ABI: PyTorch allocates, libmoe computes.

``DeviceStack`` owns one HBM buffer per layer (filled by the library's seeded
generator, or by the caller with packed weights), a workspace, and calls
``moe_decode_layer``, ``moe_stack_init`` / ``moe_stack_decode`` (the whole
stack) and ``moe_decode_stack`` (any list of its layers) on the current torch
stream. No step of the method runs here.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from . import _lib as L
from .workloads import Workload


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class DeviceStack:
    def __init__(self, shape_kwargs: dict, n_layers: int, t_max: int = 1, seed: Optional[int] = 0,
                 device: str = "cuda:0"):
        if not torch.cuda.is_available():
            raise RuntimeError("DeviceStack needs a GPU (no CPU fallback exists)")
        self.kw = dict(shape_kwargs)
        self.shape = L.make_shape(**self.kw)
        L.moe_validate_shape(self.shape)
        self.layout = L.moe_layer_layout(self.shape)
        self.n_layers, self.t_max, self.device = n_layers, t_max, device
        self.H, self.k = self.kw["hidden"], self.kw["top_k"]
        self.layers: List[torch.Tensor] = [
            torch.empty(self.layout["total_bytes"], dtype=torch.uint8, device=device) for _ in range(n_layers)
        ]
        self.ws_bytes = L.moe_workspace_bytes(self.shape, n_layers, t_max)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        # read the stack kernel's status word after every stack call (waits for the stream)
        self.check_status = False
        if seed is not None:
            for i, buf in enumerate(self.layers):
                L.moe_generate_layer(self.shape, seed, i, buf.data_ptr(), _stream())
        self._states: Dict[int, L.moe_stack_t] = {}

    def state(self, flags: int = L.MOE_PATH_DEFAULT) -> "L.moe_stack_t":
        """The initialised stack (all layers, descriptor table in the workspace) for a path choice."""
        if flags not in self._states:
            self._states[flags] = L.moe_stack_init(self.shape, [b.data_ptr() for b in self.layers], self.t_max,
                                                   flags, self.ws.data_ptr(), self.ws_bytes, _stream())
        return self._states[flags]

    @classmethod
    def from_workload(cls, w: Workload, n_layers: Optional[int] = None, t_max: Optional[int] = None, seed: int = 0):
        return cls(w.shape_kwargs(), n_layers or w.n_layers, t_max or w.T, seed)

    def rows(self, seed_x: int, T: int) -> torch.Tensor:
        x = torch.empty((T, self.H), dtype=torch.bfloat16, device=self.device)
        L.moe_generate_rows(seed_x, T, self.H, x.data_ptr(), _stream())
        return x

    def layer(self, h: torch.Tensor, l: int = 0, out: Optional[torch.Tensor] = None):
        T = h.shape[0]
        out = torch.empty_like(h) if out is None else out
        ids = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        L.moe_decode_layer(self.shape, self.layers[l].data_ptr(), T, h.data_ptr(), out.data_ptr(), ids.data_ptr(),
                           w.data_ptr(), self.ws.data_ptr(), self.ws_bytes, _stream())
        return out, ids, w

    def stack(self, h: torch.Tensor, n_layers: Optional[int] = None, trace: bool = False, routing: bool = True,
              out: Optional[torch.Tensor] = None, layer_ids: Optional[Sequence[int]] = None,
              flags: Optional[int] = None):
        """Runs the whole stack through moe_stack_decode (the initialised stack for ``flags``), or
        layers[0:n_layers] / the listed layer indices as one moe_decode_stack call."""
        T = h.shape[0]
        sel = list(layer_ids) if layer_ids is not None else list(range(n_layers or self.n_layers))
        n = len(sel)
        out = torch.empty_like(h) if out is None else out
        ids = torch.empty((n, T, self.k), dtype=torch.int32, device=self.device) if routing else None
        w = torch.empty((n, T, self.k), dtype=torch.float32, device=self.device) if routing else None
        tr = torch.empty((n + 1, T, self.H), dtype=torch.bfloat16, device=self.device) if trace else None
        pi = None if ids is None else ids.data_ptr()
        pw = None if w is None else w.data_ptr()
        pt = None if tr is None else tr.data_ptr()
        if sel == list(range(self.n_layers)) or flags is not None:
            if sel != list(range(self.n_layers)):
                raise ValueError("path flags apply to the whole initialised stack")
            L.moe_stack_decode(self.state(flags or 0), T, h.data_ptr(), out.data_ptr(), pi, pw, pt, _stream())
        else:
            L.moe_decode_stack(self.shape, [self.layers[i].data_ptr() for i in sel], T, h.data_ptr(), out.data_ptr(),
                               pi, pw, pt, self.ws.data_ptr(), self.ws_bytes, _stream())
        if self.check_status:
            st = self.status(T)
            if st != 0:
                raise RuntimeError(f"moe_decode_stack: a cross-workgroup wait timed out (status {st})")
        return out, ids, w, tr

    def status(self, T: int) -> int:
        """Status word of the last stack call with T rows (0 = every wait was met)."""
        return L.moe_stack_status(self.shape, T, self.ws.data_ptr(), _stream())


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def bf16_from_bits(bits, device: str = "cuda:0") -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 device tensor."""
    import numpy as np

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
