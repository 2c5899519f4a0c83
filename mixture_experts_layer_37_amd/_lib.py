"""ctypes binding of libmoe.so (include/moe.h). Argument marshalling only: every step of the
layer runs in the library's HIP kernels. torch supplies device memory and the stream.

The binding loads torch first so that the library binds to the HIP runtime torch already
has in the process (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int32, c_size_t, c_void_p

import torch  # noqa: F401  (loads the process's HIP runtime before libmoe.so)

from .configs import BF16, GELU, MoEConfig

LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_DTYPE_BF16, MOE_DTYPE_F32 = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_GELU = 0, 1
MOE_FLAG_BAD_INDEX, MOE_FLAG_NONFINITE_LOGIT, MOE_FLAG_STALE_SAVED = 1, 2, 4
MOE_ROUTE_TOPK, MOE_ROUTE_THRESHOLD = 0, 1
MOE_WEIGHTS_PLAIN, MOE_WEIGHTS_PACKED, MOE_ROUTER_PACKED = 0, 1, 2
MOE_WEIGHT_GATE, MOE_WEIGHT_UP, MOE_WEIGHT_DOWN, MOE_WEIGHT_ROUTER = 0, 1, 2, 3
(MOE_WS_LOGITS, MOE_WS_TOPK_IDX, MOE_WS_TOPK_W, MOE_WS_COUNTS, MOE_WS_OFFSETS, MOE_WS_SLOT_ROW,
 MOE_WS_ROW_TOKEN, MOE_WS_X_PERM, MOE_WS_H, MOE_WS_Y_PERM, MOE_WS_AUX_LOSS) = range(11)

EXPORTS = ("moe_workspace_size", "moe_capacity", "moe_route", "moe_permute",
           "moe_route_permute", "moe_permute_noalloc", "moe_expert_up",
           "moe_expert_up_rows", "moe_expert_down", "moe_grouped_ffn",
           "moe_pack_expert_weight", "moe_packed_weight_bytes", "moe_combine",
           "moe_forward", "moe_forward_train", "moe_backward_workspace_size", "moe_backward",
           "moe_workspace_view", "moe_read_device_status", "moe_status_string",
           "moe_last_hip_error")


class CConfig(ctypes.Structure):
    _fields_ = [("tokens", c_int32), ("hidden", c_int32), ("inter", c_int32),
                ("experts", c_int32), ("top_k", c_int32), ("activation", c_int32),
                ("dtype", c_int32), ("renormalize", c_int32), ("capacity_factor", c_double),
                ("routing", c_int32), ("weight_layout", c_int32), ("threshold", c_double),
                ("aux_loss_coeff", c_double)]


class MoEError(RuntimeError):
    def __init__(self, fn, status, lib):
        msg = lib.moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" (hipError {lib.moe_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_37_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        cfgp = POINTER(CConfig)
        vp = c_void_p
        sig = {
            "moe_workspace_size": [cfgp, POINTER(c_size_t)],
            "moe_capacity": [cfgp, POINTER(c_int32)],
            "moe_route": [cfgp, vp, vp, vp, vp, vp, vp, vp, c_size_t, vp],
            "moe_permute": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, c_size_t, vp],
            "moe_route_permute": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_size_t, vp],
            "moe_permute_noalloc": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "moe_expert_up": [cfgp, vp, vp, vp, vp, vp, vp],
            "moe_expert_up_rows": [cfgp, vp, vp, vp, vp, vp, vp, vp],
            "moe_expert_down": [cfgp, vp, vp, vp, vp, vp, c_size_t, vp],
            "moe_grouped_ffn": [cfgp, vp, vp, vp, vp, vp, vp, vp, c_size_t, vp],
            "moe_pack_expert_weight": [cfgp, c_int32, vp, vp, vp],
            "moe_combine": [cfgp, vp, vp, vp, vp, vp],
            "moe_forward": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, c_size_t, vp],
            "moe_backward_workspace_size": [cfgp, POINTER(c_size_t)],
            "moe_backward": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_size_t,
                             vp, c_size_t, c_int32, vp],
            "moe_forward_train": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, c_size_t, vp, c_size_t,
                                  vp],
            "moe_workspace_view": [cfgp, vp, c_int32, POINTER(c_void_p), POINTER(c_size_t)],
            "moe_read_device_status": [cfgp, vp, c_int32, vp, POINTER(c_int32)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = c_int32
        L.moe_packed_weight_bytes.argtypes = [cfgp, c_int32]
        L.moe_packed_weight_bytes.restype = c_size_t
        L.moe_status_string.argtypes = [c_int32]
        L.moe_status_string.restype = c_char_p
        L.moe_last_hip_error.argtypes = []
        L.moe_last_hip_error.restype = c_int32
        _lib = L
    return _lib


def cconfig(cfg: MoEConfig, tokens: int | None = None) -> CConfig:
    return CConfig(tokens=cfg.tokens if tokens is None else tokens, hidden=cfg.hidden,
                   inter=cfg.inter, experts=cfg.experts, top_k=cfg.top_k,
                   activation=MOE_ACT_GELU if cfg.activation == GELU else MOE_ACT_SWIGLU,
                   dtype=MOE_DTYPE_BF16 if cfg.dtype == BF16 else MOE_DTYPE_F32,
                   renormalize=1 if cfg.renormalize else 0,
                   capacity_factor=float(cfg.capacity_factor),
                   routing=MOE_ROUTE_THRESHOLD if cfg.routing == "threshold" else MOE_ROUTE_TOPK,
                   weight_layout=(MOE_WEIGHTS_PACKED | MOE_ROUTER_PACKED
                                  if cfg.weights == "packed" else MOE_WEIGHTS_PLAIN),
                   threshold=float(cfg.threshold),
                   aux_loss_coeff=float(cfg.aux_loss_coeff))


def _as_cfg(cfg):
    return cfg if isinstance(cfg, CConfig) else cconfig(cfg)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != MOE_OK:
        raise MoEError(fn, status, lib())


def _nbytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


# ------------------------------------------------------------------ host-only queries
def moe_workspace_size(cfg) -> int:
    n = c_size_t()
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(_as_cfg(cfg)), ctypes.byref(n)))
    return n.value


def moe_capacity(cfg) -> int:
    c = c_int32()
    _check("moe_capacity", lib().moe_capacity(ctypes.byref(_as_cfg(cfg)), ctypes.byref(c)))
    return c.value


# ------------------------------------------------------------------ the entry points
def moe_route(cfg, x, w_router, gate_bias, logits, topk_idx, topk_w, ws, stream=None):
    _check("moe_route", lib().moe_route(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(w_router), _ptr(gate_bias), _ptr(logits),
        _ptr(topk_idx), _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute(cfg, x, topk_idx, x_perm, expert_counts, expert_offsets, row_token, slot_row,
                ws, stream=None):
    _check("moe_permute", lib().moe_permute(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(topk_idx), _ptr(x_perm), _ptr(expert_counts),
        _ptr(expert_offsets), _ptr(row_token), _ptr(slot_row), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def moe_route_permute(cfg, x, w_router, gate_bias, logits, topk_idx, topk_w, expert_counts,
                      expert_offsets, row_token, slot_row, ws, stream=None):
    _check("moe_route_permute", lib().moe_route_permute(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(w_router), _ptr(gate_bias), _ptr(logits),
        _ptr(topk_idx), _ptr(topk_w), _ptr(expert_counts), _ptr(expert_offsets), _ptr(row_token),
        _ptr(slot_row), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute_noalloc(cfg, x, topk_idx, x_perm, expert_counts, expert_offsets, row_token,
                        slot_row, flags=None, stream=None):
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(topk_idx), _ptr(x_perm), _ptr(expert_counts),
        _ptr(expert_offsets), _ptr(row_token), _ptr(slot_row), _ptr(flags), _stream(stream)))


def moe_expert_up(cfg, x_perm, expert_offsets, w_gate, w_up, h, stream=None):
    _check("moe_expert_up", lib().moe_expert_up(
        ctypes.byref(_as_cfg(cfg)), _ptr(x_perm), _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up),
        _ptr(h), _stream(stream)))


def moe_expert_up_rows(cfg, x, row_token, expert_offsets, w_gate, w_up, h, stream=None):
    _check("moe_expert_up_rows", lib().moe_expert_up_rows(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(row_token), _ptr(expert_offsets), _ptr(w_gate),
        _ptr(w_up), _ptr(h), _stream(stream)))


def moe_expert_down(cfg, h, expert_offsets, w_down, y_perm, ws=None, stream=None):
    """ws: the layer's workspace (enables the split-K tail on bf16 layers) or None."""
    _check("moe_expert_down", lib().moe_expert_down(
        ctypes.byref(_as_cfg(cfg)), _ptr(h), _ptr(expert_offsets), _ptr(w_down), _ptr(y_perm),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_grouped_ffn(cfg, x_perm, expert_offsets, w_gate, w_up, w_down, y_perm, ws, stream=None):
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        ctypes.byref(_as_cfg(cfg)), _ptr(x_perm), _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(y_perm), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_pack_expert_weight(cfg, which: int, w, packed, stream=None):
    _check("moe_pack_expert_weight", lib().moe_pack_expert_weight(
        ctypes.byref(_as_cfg(cfg)), which, _ptr(w), _ptr(packed), _stream(stream)))


def moe_packed_weight_bytes(cfg, which: int) -> int:
    return int(lib().moe_packed_weight_bytes(ctypes.byref(_as_cfg(cfg)), which))


def moe_combine(cfg, y_perm, slot_row, topk_w, out, stream=None):
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(_as_cfg(cfg)), _ptr(y_perm), _ptr(slot_row), _ptr(topk_w), _ptr(out),
        _stream(stream)))


def moe_forward(cfg, x, w_router, gate_bias, w_gate, w_up, w_down, out, ws, stream=None):
    _check("moe_forward", lib().moe_forward(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(w_router), _ptr(gate_bias), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_backward_workspace_size(cfg) -> int:
    n = c_size_t()
    _check("moe_backward_workspace_size",
           lib().moe_backward_workspace_size(ctypes.byref(_as_cfg(cfg)), ctypes.byref(n)))
    return n.value


def moe_backward(cfg, x, w_router, w_gate, w_up, w_down, dout, dx, dw_router, dgate_bias,
                 dw_gate, dw_up, dw_down, ws, bws, saved=False, stream=None):
    """Gradients of the layer; ``ws`` is the workspace of the moe_forward call it follows
    (``saved``: that call was moe_forward_train with this ``bws``)."""
    _check("moe_backward", lib().moe_backward(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(dout), _ptr(dx), _ptr(dw_router), _ptr(dgate_bias), _ptr(dw_gate),
        _ptr(dw_up), _ptr(dw_down), _ptr(ws), _nbytes(ws), _ptr(bws), _nbytes(bws),
        1 if saved else 0, _stream(stream)))


def moe_forward_train(cfg, x, w_router, gate_bias, w_gate, w_up, w_down, out, ws, bws,
                      stream=None):
    _check("moe_forward_train", lib().moe_forward_train(
        ctypes.byref(_as_cfg(cfg)), _ptr(x), _ptr(w_router), _ptr(gate_bias), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(out), _ptr(ws), _nbytes(ws), _ptr(bws), _nbytes(bws),
        _stream(stream)))


def moe_workspace_view(cfg, ws, which: int):
    """(device address, bytes) of one intermediate inside a moe_forward workspace."""
    p, n = c_void_p(), c_size_t()
    _check("moe_workspace_view", lib().moe_workspace_view(
        ctypes.byref(_as_cfg(cfg)), _ptr(ws), which, ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value


def moe_read_device_status(cfg, ws, which: int = 3, stream=None) -> int:
    f = c_int32()
    _check("moe_read_device_status", lib().moe_read_device_status(
        ctypes.byref(_as_cfg(cfg)), _ptr(ws), which, _stream(stream), ctypes.byref(f)))
    return f.value
