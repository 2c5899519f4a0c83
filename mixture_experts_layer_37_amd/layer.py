"""Device-side plumbing around the C ABI: moving seeded inputs into torch tensors, owning a
workspace and exposing its intermediates as tensor views. No layer arithmetic here."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L
from .configs import BF16, SWIGLU, MoEConfig

_VIEW_DTYPES = {
    L.MOE_WS_LOGITS: torch.float32, L.MOE_WS_TOPK_IDX: torch.int32, L.MOE_WS_TOPK_W: torch.float32,
    L.MOE_WS_COUNTS: torch.int32, L.MOE_WS_OFFSETS: torch.int32, L.MOE_WS_SLOT_ROW: torch.int32,
    L.MOE_WS_ROW_TOKEN: torch.int32, L.MOE_WS_AUX_LOSS: torch.float64,
}


def elem_dtype(cfg: MoEConfig) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == BF16 else torch.float32


def to_device(cfg: MoEConfig, a, device="cuda") -> torch.Tensor | None:
    """numpy input (bf16 bits as uint16, or float32) -> device tensor of the layer dtype."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_device(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy (bf16 as uint16 bits, others as is)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def pack_weights(c, w_gate, w_up, w_down, w_router=None, stream=None):
    """Packed copies of the expert weights and, if given, of the router weight
    (moe_pack_expert_weight; w_gate may be None)."""
    out = []
    for which, w in ((L.MOE_WEIGHT_GATE, w_gate), (L.MOE_WEIGHT_UP, w_up),
                     (L.MOE_WEIGHT_DOWN, w_down), (L.MOE_WEIGHT_ROUTER, w_router)):
        if w is None:
            out.append(None)
            continue
        p = torch.empty(L.moe_packed_weight_bytes(c, which) // 2, dtype=w.dtype,
                        device=w.device)
        L.moe_pack_expert_weight(c, which, w, p, stream)
        out.append(p)
    return tuple(out)


class MoELayer:
    """Holds device weights and one workspace; ``forward`` calls moe_forward.

    With ``cfg.weights == "packed"`` the expert and router weights are also repacked once
    (moe_pack_expert_weight) and the forward runs on the packed copies (``fw_*``); the
    training forward and the backward use the plain ones (``w_*``)."""

    def __init__(self, cfg: MoEConfig, inputs: dict, device="cuda", tokens: int | None = None):
        self.cfg = cfg
        self.tokens = cfg.tokens if tokens is None else tokens
        self.c = L.cconfig(cfg, self.tokens)
        self.c_plain = L.cconfig(cfg.with_(weights="plain"), self.tokens)
        self.device = device
        self.w_router = to_device(cfg, inputs["w_router"], device)
        self.bias = to_device(cfg, inputs.get("bias"), device)
        self.w_gate = to_device(cfg, inputs.get("w_gate"), device) if cfg.activation == SWIGLU else None
        self.w_up = to_device(cfg, inputs["w_up"], device)
        self.w_down = to_device(cfg, inputs["w_down"], device)
        self.fw_gate, self.fw_up, self.fw_down = self.w_gate, self.w_up, self.w_down
        self.fw_router = self.w_router
        if cfg.weights == "packed":
            self.fw_gate, self.fw_up, self.fw_down, self.fw_router = pack_weights(
                self.c, self.w_gate, self.w_up, self.w_down, self.w_router)
        self.ws = torch.empty(L.moe_workspace_size(self.c), dtype=torch.uint8, device=device)

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        self._saved = False
        if out is None:
            out = torch.empty_like(x)
        L.moe_forward(self.c, x, self.fw_router, self.bias, self.fw_gate, self.fw_up,
                      self.fw_down, out, self.ws, stream)
        return out

    def _bws(self):
        if not hasattr(self, "bws"):
            self.bws = torch.empty(L.moe_backward_workspace_size(self.c_plain), dtype=torch.uint8,
                                   device=self.device)
        return self.bws

    def forward_train(self, x: torch.Tensor, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
        """moe_forward_train: the forward, keeping GEMM 1's pre-activations for ``backward``."""
        if out is None:
            out = torch.empty_like(x)
        L.moe_forward_train(self.c_plain, x, self.w_router, self.bias, self.w_gate, self.w_up,
                            self.w_down, out, self.ws, self._bws(), stream)
        self._saved = True
        return out

    def backward(self, x: torch.Tensor, dout: torch.Tensor, stream=None) -> dict:
        """moe_backward after the last ``forward`` / ``forward_train`` on ``x``: a dict of
        gradient tensors."""
        cfg, dev = self.cfg, self.device
        self._bws()
        g = dict(dx=torch.empty_like(x),
                 dw_router=torch.empty((cfg.hidden, cfg.experts), dtype=torch.float32, device=dev),
                 dbias=torch.empty(cfg.experts, dtype=torch.float32, device=dev),
                 dw_gate=torch.empty_like(self.w_gate) if self.w_gate is not None else None,
                 dw_up=torch.empty_like(self.w_up), dw_down=torch.empty_like(self.w_down))
        L.moe_backward(self.c_plain, x, self.w_router, self.w_gate, self.w_up, self.w_down, dout,
                       g["dx"], g["dw_router"], g["dbias"], g["dw_gate"], g["dw_up"],
                       g["dw_down"], self.ws, self.bws, getattr(self, "_saved", False), stream)
        self._saved = False
        if cfg.aux_loss_coeff > 0:   # the auxiliary load-balancing loss, float64 [1]
            g["aux_loss"] = self.view(L.MOE_WS_AUX_LOSS)
        return g

    def view(self, which: int) -> torch.Tensor:
        """Tensor aliasing one intermediate of the last forward inside the workspace."""
        ptr, nbytes = L.moe_workspace_view(self.c, self.ws, which)
        off = ptr - self.ws.data_ptr()
        raw = self.ws[off:off + nbytes]
        cfg, T, k = self.cfg, self.tokens, self.cfg.top_k
        if which in _VIEW_DTYPES:
            t = raw.view(_VIEW_DTYPES[which])
            if which in (L.MOE_WS_LOGITS,):
                return t.view(T, cfg.experts)
            if which in (L.MOE_WS_TOPK_IDX, L.MOE_WS_TOPK_W, L.MOE_WS_SLOT_ROW):
                return t.view(T, k)
            return t
        t = raw.view(elem_dtype(cfg))
        width = cfg.inter if which == L.MOE_WS_H else cfg.hidden
        return t.view(T * k, width)

    def device_status(self, which: int = 3) -> int:
        return L.moe_read_device_status(self.c, self.ws, which)
