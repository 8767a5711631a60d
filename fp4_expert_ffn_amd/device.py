"""Device-memory plumbing around the C ABI: uploading and packing expert weights, and a
small layer object that owns the packed weights and the workspaces. Torch is used only to
allocate device memory and to name streams; every step of the computation is a call into
the HIP library."""

from __future__ import annotations

from typing import Callable, Optional, Tuple

import numpy as np
import torch

from . import moe_fp4 as C

ExpertSource = Callable[[int], Tuple[np.ndarray, np.ndarray]]


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_bf16(bits: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device tensor of dtype bfloat16."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Device bfloat16 tensor -> host uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def upload_experts(source: ExpertSource, n_experts: int, hidden: int, inter: int, device,
                   chunk: int = 16, stream=None) -> torch.Tensor:
    """Generate (on the host) and pack every expert into one device buffer of
    moe_fp4_packed_bytes bytes, `chunk` experts at a time through a device staging area."""
    stride = C.moe_fp4_packed_expert_stride(hidden, inter)
    packed = torch.empty(stride * n_experts, dtype=torch.uint8, device=device)
    for e0 in range(0, n_experts, chunk):
        e1 = min(n_experts, e0 + chunk)
        blobs = [source(e) for e in range(e0, e1)]
        codes = _dev(np.stack([b[0] for b in blobs]), device)
        scales = _dev(np.stack([b[1] for b in blobs]), device)
        C.moe_fp4_pack(codes, scales, e1 - e0, hidden, inter, packed.data_ptr() + e0 * stride,
                       (e1 - e0) * stride, stream=stream)
        torch.cuda.current_stream(device).synchronize() if stream is None else stream.synchronize()
        del codes, scales
    return packed


class MoeFp4Layer:
    """One MoE layer's routed experts (packed FP4) and router, resident in device memory."""

    def __init__(self, packed: torch.Tensor, n_experts: int, hidden: int, inter: int, k: int,
                 w_router: Optional[torch.Tensor] = None):
        self.packed = packed
        self.n_experts, self.hidden, self.inter, self.k = n_experts, hidden, inter, k
        self.w_router = w_router
        self.device = packed.device
        self._ws = None
        self._rws = None
        self._fws = None

    def _workspace(self, T: int, k: Optional[int] = None) -> torch.Tensor:
        need = C.moe_fp4_workspace_bytes(T, self.k if k is None else k, self.n_experts,
                                         self.hidden, self.inter)
        if self._ws is None or self._ws.numel() < max(need, 256):
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def _route_workspace(self, T: int) -> torch.Tensor:
        need = C.moe_fp4_route_workspace_bytes(T, self.n_experts)
        if self._rws is None or self._rws.numel() < max(need, 256):
            self._rws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._rws

    def route(self, x: torch.Tensor, ids: Optional[torch.Tensor] = None,
              w: Optional[torch.Tensor] = None, stream=None):
        T = x.shape[0]
        if ids is None:
            ids = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        if w is None:
            w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        ws = self._route_workspace(T)
        C.moe_fp4_route(x, self.w_router, T, self.hidden, self.n_experts, self.k, ids, w, ws,
                        stream=stream)
        return ids, w

    def route_residual(self, r_in: torch.Tensor, y_prev: torch.Tensor, r_out: torch.Tensor,
                       x_out: torch.Tensor, eps: float = 1e-6, ids: Optional[torch.Tensor] = None,
                       w: Optional[torch.Tensor] = None, stream=None):
        """moe_fp4_route_residual: r_out = r_in + y_prev, x_out = RMSNorm(r_out), then route
        x_out (one launch at batch 1)."""
        T = r_in.shape[0]
        if ids is None:
            ids = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        if w is None:
            w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        ws = self._route_workspace(T)
        C.moe_fp4_route_residual(r_in, y_prev, r_out, x_out, eps, self.w_router, T, self.hidden,
                                 self.n_experts, self.k, ids, w, ws, stream=stream)
        return ids, w

    def route_logits(self, logits: torch.Tensor, stream=None):
        T = logits.shape[0]
        ids = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        C.moe_fp4_route_logits(logits, T, self.n_experts, self.k, ids, w, stream=stream)
        return ids, w

    def ffn(self, x: torch.Tensor, ids: torch.Tensor, w: torch.Tensor,
            y: Optional[torch.Tensor] = None, stream=None, path: Optional[int] = None) -> torch.Tensor:
        """moe_fp4_expert_ffn (path None: automatic choice) or moe_fp4_expert_ffn_ex."""
        T = x.shape[0]
        k = ids.shape[1] if ids.dim() == 2 else self.k
        if y is None:
            y = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=self.device)
        ws = self._workspace(T, k)
        if path is None:
            C.moe_fp4_expert_ffn(x, ids, w, T, k, self.packed, self.n_experts, self.hidden,
                                 self.inter, y, ws, stream=stream)
        else:
            C.moe_fp4_expert_ffn_ex(x, ids, w, T, k, self.packed, self.n_experts, self.hidden,
                                    self.inter, y, ws, path, stream=stream)
        return y

    def forward(self, x: torch.Tensor, stream=None):
        """moe_fp4_route then moe_fp4_expert_ffn."""
        ids, w = self.route(x, stream=stream)
        return self.ffn(x, ids, w, stream=stream), ids, w

    def _forward_workspace(self, T: int) -> torch.Tensor:
        need = C.moe_fp4_moe_forward_workspace_bytes(T, self.k, self.n_experts, self.hidden,
                                                     self.inter)
        if self._fws is None or self._fws.numel() < max(need, 256):
            self._fws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._fws

    def forward_fused(self, x: torch.Tensor, ids: Optional[torch.Tensor] = None,
                      w: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      stream=None):
        """moe_fp4_moe_forward: the same layer in one call (three kernel launches)."""
        T = x.shape[0]
        if ids is None:
            ids = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        if w is None:
            w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        if y is None:
            y = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=self.device)
        ws = self._forward_workspace(T)
        C.moe_fp4_moe_forward(x, self.w_router, T, self.hidden, self.n_experts, self.k, self.packed,
                              self.inter, ids, w, y, ws, stream=stream)
        return y, ids, w
