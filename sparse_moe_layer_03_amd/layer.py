"""Device-resident MoE layer: weights and workspace in HBM, calls into libmoe355.

PyTorch is used for device memory and streams only; every step of the layer
runs in the HIP kernels behind ``moe.py``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from . import moe

BF16_KEYS = ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down", "w_sg")
FP8_KEYS = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")


def to_device_bf16(a: Optional[np.ndarray], device):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on ``device`` (bits unchanged)."""
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bf16_to_numpy_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class Shapes:
    H: int
    E: int
    k: int
    I: int
    I_s: int


class DeviceLayer:
    """The layer's weights on one GPU plus a reusable workspace.

    ``fp8``: also upload the FP8 expert weights (``<key>_fp8`` codes and
    ``<key>_scale`` row scales of ``weights``); ``forward`` then calls
    ``moe_forward_fp8``.  ``q4``: likewise the 4-bit weights (``<key>_q4``
    codes and ``<key>_q4scale`` fp16 group scales) and ``moe_forward_q4``.
    """

    def __init__(self, weights: Dict[str, np.ndarray], k: int, device="cuda:0", fp8: bool = False,
                 q4: bool = False):
        import torch
        self.device = torch.device(device)
        self.fp8 = fp8
        self.q4 = q4
        self.w = {key: to_device_bf16(weights.get(key), self.device) for key in BF16_KEYS}
        self.q = {}
        if fp8:
            for key in FP8_KEYS:
                c, sc = weights.get(key + "_fp8"), weights.get(key + "_scale")
                self.q[key] = None if c is None else torch.from_numpy(np.ascontiguousarray(c, np.uint8)).to(self.device)
                self.q[key + "_scale"] = (None if sc is None else
                                          torch.from_numpy(np.ascontiguousarray(sc, np.float32)).to(self.device))
        if q4:
            for key in FP8_KEYS:
                c, sc = weights.get(key + "_q4"), weights.get(key + "_q4scale")
                self.q[key + "_q4"] = (None if c is None else
                                       torch.from_numpy(np.ascontiguousarray(c, np.uint8)).to(self.device))
                self.q[key + "_q4scale"] = (None if sc is None else torch.from_numpy(
                    np.ascontiguousarray(sc, np.uint16).view(np.int16)).to(self.device))
        b = weights.get("bias")
        self.bias = None if b is None else torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(self.device)
        E, I, H = weights["w_gate"].shape
        I_s = 0 if weights.get("ws_gate") is None else weights["ws_gate"].shape[0]
        self.shapes = Shapes(H=H, E=E, k=k, I=I, I_s=I_s)
        self._ws = None
        self._ws_bytes = 0
        self._ws_streams = []  # streams the current workspace has been used on since it was allocated

    @classmethod
    def from_inputs(cls, inp, device="cuda:0", fp8: bool = False, q4: bool = False):
        return cls(inp, inp["wl"].k, device, fp8=fp8, q4=q4)

    def workspace(self, T: int):
        import torch
        s = self.shapes
        need = moe.moe_workspace_size(T, s.H, s.E, s.k, s.I, s.I_s)
        if need == 0 and T > 0:
            raise moe.MoEError(moe.MOE_ERR_SHAPE, "unsupported shapes")
        if self._ws is None or self._ws_bytes < need:
            if self._ws is not None:
                # the caching allocator tracks only the allocating stream: keep the old buffer from being
                # handed out again before work already enqueued on the other streams that used it is done
                for st in self._ws_streams:
                    self._ws.record_stream(st)
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            self._ws_bytes = max(need, 256)
            self._ws_streams = []
        return self._ws, self._ws_bytes

    def _note_stream(self, stream):
        """Remember a stream (None, a torch stream or a raw handle) the workspace is used on."""
        import torch
        if stream is None:
            st = torch.cuda.current_stream(self.device)
        elif isinstance(stream, int):
            st = torch.cuda.ExternalStream(stream, device=self.device)
        else:
            st = stream
        if all(st != u for u in self._ws_streams):
            self._ws_streams.append(st)

    def forward(self, x, y=None, stream=None):
        """y = layer(x); x is a [T, H] bfloat16 device tensor."""
        import torch
        s = self.shapes
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, s.H), dtype=torch.bfloat16, device=self.device)
        ws, nbytes = self.workspace(T)
        self._note_stream(stream)
        W = self.w
        if self.q4:
            q = self.q
            moe.moe_forward_q4(x, W["w_router"], self.bias, q["w_gate_q4"], q["w_gate_q4scale"], q["w_up_q4"],
                               q["w_up_q4scale"], q["w_down_q4"], q["w_down_q4scale"], q["ws_gate_q4"],
                               q["ws_gate_q4scale"], q["ws_up_q4"], q["ws_up_q4scale"], q["ws_down_q4"],
                               q["ws_down_q4scale"], W["w_sg"], T, s.H, s.E, s.k, s.I, s.I_s, y, ws, nbytes, stream)
            return y
        if self.fp8:
            q = self.q
            moe.moe_forward_fp8(x, W["w_router"], self.bias, q["w_gate"], q["w_gate_scale"], q["w_up"],
                                q["w_up_scale"], q["w_down"], q["w_down_scale"], q["ws_gate"], q["ws_gate_scale"],
                                q["ws_up"], q["ws_up_scale"], q["ws_down"], q["ws_down_scale"], W["w_sg"],
                                T, s.H, s.E, s.k, s.I, s.I_s, y, ws, nbytes, stream)
            return y
        moe.moe_forward(x, W["w_router"], self.bias, W["w_gate"], W["w_up"], W["w_down"], W["ws_gate"], W["ws_up"],
                        W["ws_down"], W["w_sg"], T, s.H, s.E, s.k, s.I, s.I_s, y, ws, nbytes, stream)
        return y

    def forward_ids(self, T: int):
        """The expert ids [T, k] (int32, rank order) the last forward of T tokens selected, read back
        from the workspace."""
        import torch
        s = self.shapes
        off = moe.moe_forward_ids_offset(T, s.H, s.E, s.k, s.I, s.I_s)
        return self._ws[off:off + T * s.k * 4].view(torch.int32).view(T, s.k)

    # ---------------------------------------------------------------- stages
    def alloc_stage_buffers(self, T: int):
        import torch
        s = self.shapes
        dev = self.device
        max_rows = moe.moe_align_max_rows(T, s.E, s.k)
        max_tiles = moe.moe_align_max_tiles(T, s.E, s.k)
        i32 = dict(dtype=torch.int32, device=dev)
        return {
            "ids": torch.empty((T, s.k), **i32),
            "w": torch.empty((T, s.k), dtype=torch.float32, device=dev),
            "s": torch.empty(max(T, 1), dtype=torch.float32, device=dev),
            "logits": torch.empty((T, s.E), dtype=torch.float32, device=dev),
            "counts": torch.empty(s.E, **i32),
            "pad_off": torch.empty(s.E + 1, **i32),
            "sorted": torch.empty(max_rows, **i32),
            "inv": torch.empty(T * s.k, **i32),
            "tiles": torch.empty(2 * max_tiles, **i32),
            "n_tiles": torch.empty(2, **i32),
            "scratch": torch.empty(moe.moe_align_scratch_size(T, s.E, s.k), dtype=torch.uint8, device=dev),
            "route_scratch": torch.empty(moe.moe_route_scratch_size(T, s.H, s.E), dtype=torch.uint8, device=dev),
            "h": torch.empty((max_rows, s.I), dtype=torch.bfloat16, device=dev),
            "h_s": torch.empty((T, s.I_s), dtype=torch.bfloat16, device=dev) if s.I_s else None,
            "o": torch.empty((T * s.k, s.H), dtype=torch.bfloat16, device=dev),
            "y": torch.empty((T, s.H), dtype=torch.bfloat16, device=dev),
        }

    def run_route(self, x, b, stream=None, streamed=True):
        """streamed: the form moe_forward runs (W_router copied in operand order into scratch, then
        the streamed router); else the one-launch router with W_router staged through LDS."""
        s = self.shapes
        T = x.shape[0]
        moe.moe_route(x, self.w["w_router"], self.bias, self.w["w_sg"], T, s.H, s.E, s.k, b["ids"], b["w"],
                      b["s"] if s.I_s else None, b["logits"], stream, scratch=b["route_scratch"] if streamed else None)

    def run_align(self, T, b, stream=None):
        s = self.shapes
        moe.moe_align(b["ids"], T, s.E, s.k, b["counts"], b["pad_off"], b["sorted"], b["inv"],
                      b["tiles"], b["n_tiles"], b["scratch"], b["scratch"].numel(), stream)

    def run_gate_up(self, x, b, stream=None):
        s = self.shapes
        T = x.shape[0]
        W = self.w
        moe.moe_grouped_gate_up(x, W["w_gate"], W["w_up"], W["ws_gate"], W["ws_up"], b["sorted"], b["tiles"],
                                b["n_tiles"], T, s.H, s.E, s.k, s.I, s.I_s, b["h"], b["h_s"], stream)

    def run_down(self, T, b, stream=None):
        s = self.shapes
        moe.moe_grouped_down(b["h"], self.w["w_down"], b["sorted"], b["tiles"], b["n_tiles"], T, s.H, s.E, s.k,
                             s.I, b["o"], stream)

    def run_combine(self, T, b, stream=None):
        s = self.shapes
        moe.moe_combine(b["o"], b["w"], b["h_s"], self.w["ws_down"], b["s"] if s.I_s else None, T,
                        s.H, s.k, s.I_s, b["y"], stream)

    def run_stages(self, x, b=None, stream=None, ids=None, w=None, s=None):
        """All prefill stages one by one (same kernels as ``forward``); returns the buffers.

        ``ids`` ([T, k] int32), ``w`` ([T, k] fp32) and ``s`` ([T] fp32) device
        tensors, when given, replace the router's outputs before the align
        stage, so align, the grouped GEMMs and the combine can be driven with
        crafted expert loads.
        """
        T = x.shape[0]
        if b is None:
            b = self.alloc_stage_buffers(T)
        self.run_route(x, b, stream)
        if ids is not None:
            b["ids"].copy_(ids)
        if w is not None:
            b["w"].copy_(w)
        if s is not None:
            b["s"][:T].copy_(s)
        self.run_align(T, b, stream)
        self.run_gate_up(x, b, stream)
        self.run_down(T, b, stream)
        self.run_combine(T, b, stream)
        return b


class PrefillRunner:
    """Prefill of any length through per-bucket HIP graphs (moe_prefill_runner_*) for a DeviceLayer's
    weights: its FP8 codes when the layer was built with ``fp8``, else its BF16 weights.  The layer
    must outlive the runner."""

    PAGE_BUCKETS = (1024, 2048, 4096, 8192)

    def __init__(self, layer: DeviceLayer, buckets=PAGE_BUCKETS):
        s = layer.shapes
        W = layer.w
        self.layer = layer
        self.buckets = tuple(buckets)
        self.handle = None
        if layer.q4:
            raise ValueError("the prefill runner takes BF16 or FP8 weights (4-bit weights serve T <= %d)"
                             % moe.Q4_MAX_T)
        if layer.fp8:
            q = layer.q
            self.handle = moe.moe_prefill_runner_create_fp8(
                W["w_router"], layer.bias, q["w_gate"], q["w_gate_scale"], q["w_up"], q["w_up_scale"], q["w_down"],
                q["w_down_scale"], q["ws_gate"], q["ws_gate_scale"], q["ws_up"], q["ws_up_scale"], q["ws_down"],
                q["ws_down_scale"], W["w_sg"], s.H, s.E, s.k, s.I, s.I_s, list(self.buckets))
        else:
            self.handle = moe.moe_prefill_runner_create(W["w_router"], layer.bias, W["w_gate"], W["w_up"],
                                                        W["w_down"], W["ws_gate"], W["ws_up"], W["ws_down"],
                                                        W["w_sg"], s.H, s.E, s.k, s.I, s.I_s, list(self.buckets))

    def plan(self, T: int):
        return moe.moe_bucket_plan(T, list(self.buckets))

    def run(self, x, y=None, stream=None):
        """y = layer(x) for a [T, H] bfloat16 device tensor, segment by segment."""
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.layer.shapes.H), dtype=torch.bfloat16, device=self.layer.device)
        moe.moe_prefill_runner_run(self.handle, x, T, y, stream)
        return y

    def close(self):
        """Free the runner's buffers and graphs (after its last run has completed)."""
        if self.handle:
            import torch
            torch.cuda.synchronize(self.layer.device)
            moe.moe_prefill_runner_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
