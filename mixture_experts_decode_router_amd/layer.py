"""Device-side holder of one MoE layer: weights, workspace and config, with
methods that call the C entry points.  torch provides device memory and
streams; every step of the block runs in the HIP library."""
from __future__ import annotations

import copy
import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib as L


def _dev(a: np.ndarray, device) -> torch.Tensor:
    """Host array -> device tensor with the same bytes (uint16 -> int16 view)."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class MoELayer:
    """One sparse-MoE layer on the GPU.

    `inp` is any object with the fields H, E, k, I, wfmt, w_router, bias and
    either (w_gate_up, w_down) bf16 bit arrays or (q_gate_up, s_gate_up,
    q_down, s_down, codebook) 4-bit arrays (see synthetic.MoEInputs).
    """

    def __init__(self, inp, t_max: int, device: str = "cuda", tiled: bool = True,
                 out_bf16: bool = False, renorm: bool = True, lora: Optional[dict] = None, train: bool = False,
                 poison: Optional[bool] = None):
        """out_bf16: bf16 output (else fp32); renorm: top-k weights renormalised
        over the k chosen (else the full softmax at the chosen); lora: fp32
        adapters (a_gate_up, b_gate_up, a_down, b_down arrays and scale, as
        synthetic.lora_adapters makes them) fused into the expert GEMMs;
        train: the forward keeps what backward() needs; poison: fill the
        workspace with 0xFF bytes on the call's stream before every eager
        route, permute and forward, so that a kernel reading workspace it did
        not write first gives wrong results (default: the environment
        variable MOE_POISON_WORKSPACE=1)."""
        self.poison = os.environ.get("MOE_POISON_WORKSPACE") == "1" if poison is None else bool(poison)
        self.device = torch.device(device)
        self.H, self.E, self.k, self.I = inp.H, inp.E, inp.k, inp.I
        rowmajor = L.MOE_W_BF16 if inp.wfmt == "bf16" else L.MOE_W_NF4_B64
        self.wfmt = rowmajor + 2 if tiled else rowmajor
        self.out_dtype = torch.bfloat16 if out_bf16 else torch.float32
        self.cfg = L.moe_config(inp.H, inp.I, inp.E, inp.k, t_max, self.wfmt,
                                L.MOE_OUT_BF16 if out_bf16 else L.MOE_OUT_F32,
                                L.MOE_TOPK_RENORM if renorm else L.MOE_TOPK_SOFTMAX, int(train))
        st = L.moe_config_check(self.cfg)
        if st != L.MOE_OK:
            raise L.MoEError(st, L.moe_last_error())
        self.t_max = t_max
        self.tensors = {}
        t = self.tensors
        t["w_router"] = _dev(inp.w_router, self.device)
        if inp.bias is not None:
            t["router_bias"] = _dev(np.asarray(inp.bias, np.float32), self.device)
        if inp.wfmt == "bf16":
            t["w_gate_up"] = _dev(inp.w_gate_up, self.device)
            t["w_down"] = _dev(inp.w_down, self.device)
        else:
            for name in ("q_gate_up", "s_gate_up", "q_down", "s_down", "codebook"):
                t[name] = _dev(getattr(inp, name), self.device)
        self.w = L.moe_weights(*[t[f].data_ptr() if f in t else None
                                 for f, _ in L.moe_weights._fields_])
        if tiled:
            # convert once into the tiled layout on the device; the
            # row-major copies are released afterwards
            src_cfg = L.moe_config(inp.H, inp.I, inp.E, inp.k, t_max, rowmajor)
            names = ("w_gate_up", "w_down") if inp.wfmt == "bf16" else \
                ("q_gate_up", "s_gate_up", "q_down", "s_down")
            packed = {n: torch.empty_like(t[n]) for n in names}
            dst = L.moe_weights(*[(packed[f] if f in packed else t[f]).data_ptr() if (f in packed or f in t)
                                  else None for f, _ in L.moe_weights._fields_])
            L.moe_pack_weights(src_cfg, self.w, dst)
            torch.cuda.synchronize(self.device)
            t.update(packed)
            self.w = dst
        self.lora = None
        if lora is not None:
            for name in ("a_gate_up", "b_gate_up", "a_down", "b_down"):
                t["lora_" + name] = _dev(np.ascontiguousarray(lora[name], dtype=np.float32), self.device)
            self.lora = L.moe_lora(*[t["lora_" + n].data_ptr() for n in ("a_gate_up", "b_gate_up", "a_down",
                                                                            "b_down")],
                                   float(lora["scale"]), int(lora["a_gate_up"].shape[1]))
            self.w.lora = ctypes.addressof(self.lora)
        self.ws_bytes = L.moe_workspace_size(self.cfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.graph = None

    def with_options(self, out_bf16: bool = False, renorm: bool = True, train: bool = False) -> "MoELayer":
        """The same device weights under another output dtype / top-k weight
        mode / training flag, with a workspace of its own."""
        other = copy.copy(self)
        c = self.cfg
        other.cfg = L.moe_config(c.hidden, c.inter, c.n_experts, c.top_k, c.t_max, c.wfmt,
                                 L.MOE_OUT_BF16 if out_bf16 else L.MOE_OUT_F32,
                                 L.MOE_TOPK_RENORM if renorm else L.MOE_TOPK_SOFTMAX, int(train))
        other.out_dtype = torch.bfloat16 if out_bf16 else torch.float32
        other.ws_bytes = L.moe_workspace_size(other.cfg)
        other.workspace = torch.empty(other.ws_bytes, dtype=torch.uint8, device=self.device)
        other.graph = None
        return other

    def with_lora(self, lora: dict) -> "MoELayer":
        """The same device weights with fp32 LoRA adapters attached (see
        __init__), with a workspace of its own."""
        other = copy.copy(self)
        other.tensors = dict(self.tensors)
        for name in ("a_gate_up", "b_gate_up", "a_down", "b_down"):
            other.tensors["lora_" + name] = _dev(np.ascontiguousarray(lora[name], dtype=np.float32), self.device)
        other.lora = L.moe_lora(*[other.tensors["lora_" + n].data_ptr() for n in ("a_gate_up", "b_gate_up",
                                                                                  "a_down", "b_down")],
                                float(lora["scale"]), int(lora["a_gate_up"].shape[1]))
        other.w = L.moe_weights(*[getattr(self.w, f) for f, _ in L.moe_weights._fields_])
        other.w.lora = ctypes.addressof(other.lora)
        other.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        other.graph = None
        return other

    # ------------------------------------------------------------ helpers
    def upload_x(self, x_bits: np.ndarray) -> torch.Tensor:
        return _dev(x_bits, self.device)

    def _poison(self, stream) -> None:
        if not self.poison:
            return
        if isinstance(stream, int):
            raise ValueError("workspace poisoning needs a torch stream (or None)")
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            self.workspace.fill_(0xFF)

    def _view(self, addr: int, n: int, dtype) -> torch.Tensor:
        off = addr - self.workspace.data_ptr()
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype)

    # ------------------------------------------------------------ entry points
    def route(self, x: torch.Tensor, T: Optional[int] = None, with_logits: bool = False, stream=None):
        T = T or x.shape[0]
        ids = torch.empty(T, self.k, dtype=torch.int32, device=self.device)
        wts = torch.empty(T, self.k, dtype=torch.float32, device=self.device)
        logits = torch.empty(T, self.E, dtype=torch.float32, device=self.device) if with_logits else None
        self._poison(stream)
        L.moe_route(self.cfg, self.w, x, T, ids, wts, logits, self.workspace, self.ws_bytes, stream)
        return ids, wts, logits

    def permute(self, ids: torch.Tensor, T: Optional[int] = None, with_pos: bool = True, stream=None):
        T = T or ids.shape[0]
        n = T * self.k
        counts = torch.empty(self.E, dtype=torch.int32, device=self.device)
        offsets = torch.empty(self.E + 1, dtype=torch.int32, device=self.device)
        perm = torch.empty(n, dtype=torch.int32, device=self.device)
        pos = torch.empty(n, dtype=torch.int32, device=self.device) if with_pos else None
        self._poison(stream)
        L.moe_permute(self.cfg, ids, T, counts, offsets, perm, pos, self.workspace, self.ws_bytes, stream)
        return counts, offsets, perm, pos

    def forward(self, x: torch.Tensor, T: Optional[int] = None, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
        T = T or x.shape[0]
        if out is None:
            out = torch.empty(T, self.H, dtype=self.out_dtype, device=self.device)
        self._poison(stream)
        L.moe_forward(self.cfg, self.w, x, T, out, self.workspace, self.ws_bytes, stream)
        return out

    def forward_prenorm(self, residual: torch.Tensor, delta: Optional[torch.Tensor], gamma: torch.Tensor,
                        eps: float, T: Optional[int] = None, out: Optional[torch.Tensor] = None,
                        x_out: Optional[torch.Tensor] = None, residual_out: Optional[torch.Tensor] = None,
                        write_residual: bool = True, stream=None):
        """The block with the pre-block step fused into its router pass (bf16
        tensors as int16 bit patterns).  Returns (out, x_out, residual_out)."""
        T = T or residual.shape[0]
        if out is None:
            out = torch.empty(T, self.H, dtype=self.out_dtype, device=self.device)
        if x_out is None:
            x_out = torch.empty(T, self.H, dtype=torch.int16, device=self.device)
        if residual_out is None and write_residual:
            residual_out = torch.empty(T, self.H, dtype=torch.int16, device=self.device)
        pn = L.make_prenorm(residual, delta, gamma, eps, residual_out, x_out)
        self._poison(stream)
        L.moe_forward_prenorm(self.cfg, self.w, pn, T, out, self.workspace, self.ws_bytes, stream)
        return out, x_out, residual_out

    def backward(self, x: torch.Tensor, d_out: torch.Tensor, T: Optional[int] = None, stream=None,
                 weight_grads=None):
        """Gradients for the routing of the last forward on this layer's
        workspace (a train layer; that forward must have been of the same x):
        returns (d_x fp32 [T][H], d_topk_w fp32 [T][k]), and with adapters
        attached a third item, the adapter gradients {a_gate_up, b_gate_up,
        a_down, b_down} (fp32, the adapters' shapes).  weight_grads: a pair of
        fp32 device tensors ([E][2I][H], [E][H][I]) that receive the expert-
        weight gradients, or None."""
        T = T or x.shape[0]
        d_x = torch.empty(T, self.H, dtype=torch.float32, device=self.device)
        d_w = torch.empty(T, self.k, dtype=torch.float32, device=self.device)
        grads, d_lora = None, None
        if self.lora is not None:
            grads = {n: torch.empty_like(self.tensors["lora_" + n])
                     for n in ("a_gate_up", "b_gate_up", "a_down", "b_down")}
            d_lora = L.make_lora_grads(grads["a_gate_up"], grads["b_gate_up"], grads["a_down"], grads["b_down"])
        d_weights = None
        if weight_grads is not None:
            gu, dn = weight_grads
            if tuple(gu.shape) != (self.E, 2 * self.I, self.H) or tuple(dn.shape) != (self.E, self.H, self.I) \
                    or gu.dtype != torch.float32 or dn.dtype != torch.float32:
                raise ValueError("weight_grads must be fp32 [E][2I][H] and [E][H][I]")
            d_weights = L.moe_weight_grads(gu.data_ptr(), dn.data_ptr())
        L.moe_backward(self.cfg, self.w, x, T, d_out, d_x, d_w, self.workspace, self.ws_bytes, stream, d_lora,
                       d_weights)
        return (d_x, d_w) if grads is None else (d_x, d_w, grads)

    def forward_timed(self, x: torch.Tensor, out: torch.Tensor, events, T: Optional[int] = None,
                      stream=None) -> None:
        L.moe_forward_timed(self.cfg, self.w, x, T or x.shape[0], out, self.workspace, self.ws_bytes,
                            stream, events)

    def views(self, T: int) -> dict:
        """Routing arrays a forward / replay wrote into the workspace (device tensors)."""
        v = L.moe_workspace_views(self.cfg, self.workspace, self.ws_bytes)
        n = T * self.k
        return dict(
            ids=self._view(v.topk_ids, n, torch.int32).view(T, self.k),
            w=self._view(v.topk_w, n, torch.float32).view(T, self.k),
            counts=self._view(v.counts, self.E, torch.int32),
            offsets=self._view(v.offsets, self.E + 1, torch.int32),
            perm=self._view(v.perm, n, torch.int32),
            pos=self._view(v.pos, n, torch.int32),
        )

    def read_counts(self, stream=None) -> np.ndarray:
        return L.moe_read_counts(self.cfg, self.workspace, self.ws_bytes, stream)

    # ------------------------------------------------------------ graphs
    def capture(self, buckets: Sequence[int], x_static: torch.Tensor, out_static: torch.Tensor,
                stream) -> int:
        self.release_graph()
        self.graph = L.moe_graph_capture(self.cfg, self.w, list(buckets), x_static, out_static,
                                         self.workspace, self.ws_bytes, stream)
        return self.graph

    def capture_prenorm(self, buckets: Sequence[int], residual: torch.Tensor, delta: Optional[torch.Tensor],
                        gamma: torch.Tensor, eps: float, residual_out: Optional[torch.Tensor],
                        x_out: torch.Tensor, out_static: torch.Tensor, stream) -> int:
        self.release_graph()
        pn = L.make_prenorm(residual, delta, gamma, eps, residual_out, x_out)
        self.graph = L.moe_graph_capture_prenorm(self.cfg, self.w, list(buckets), pn, out_static,
                                                 self.workspace, self.ws_bytes, stream)
        return self.graph

    def replay(self, T: int, stream=None) -> None:
        L.moe_graph_replay(self.graph, T, stream)

    def release_graph(self) -> None:
        if self.graph is not None:
            L.moe_graph_destroy(self.graph)
            self.graph = None

    def __del__(self):
        try:
            self.release_graph()
        except Exception:
            pass
