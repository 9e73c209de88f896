"""CPU oracle of the sparse MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It loads ``liboracle.so`` built from ``moe_oracle.c`` (plain
C, OpenMP, no shared code with the HIP library) and marshals NumPy arrays.
It never imports the product package.

The arithmetic, and the passages it follows, are described at the top of
``moe_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", LIB_PATH, "-lm"]


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build(out: str = LIB_PATH, sanitize: bool = False) -> str:
    """Compile the oracle library (gcc) at ``out`` (``sanitize``: with ASan and UBSan; a process loading
    it must preload gcc's libasan); returns its path."""
    tmp = out + ".tmp"
    cmd = GCC_CMD[:-3] + (SANITIZE_FLAGS if sanitize else []) + ["-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, lib_path: str = LIB_PATH):
        if lib_path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(lib_path)
        p = C.c_void_p
        i = C.c_int
        L.oracle_route.argtypes = [p, p, p, p, i, i, i, i, p, p, p, p]
        L.oracle_route_from_logits.argtypes = [p, i, i, i, p, p]
        L.oracle_align.argtypes = [p, i, i, i, p, p, p]
        L.oracle_forward.argtypes = [p] * 10 + [i] * 6 + [p] * 10
        L.oracle_forward_fp8.argtypes = [p] * 16 + [i] * 6 + [p] * 10
        L.oracle_e4m3_decode.argtypes = [p, C.c_long, p]
        L.oracle_forward_q4.argtypes = [p] * 16 + [i] * 6 + [p] * 10
        L.oracle_f16_decode.argtypes = [p, C.c_long, p]
        L.oracle_q4_dequant.argtypes = [p, p, C.c_long, i, p]
        for f in (L.oracle_route, L.oracle_route_from_logits, L.oracle_align, L.oracle_forward,
                  L.oracle_forward_fp8, L.oracle_e4m3_decode, L.oracle_forward_q4, L.oracle_f16_decode,
                  L.oracle_q4_dequant):
            f.restype = C.c_int
        self.lib = L
        self.path = lib_path

    def route(self, x, w_router, bias, w_sg, k: int) -> Dict[str, np.ndarray]:
        """Router logits (fp32), top-k ids, renormalised weights (double), shared gate s."""
        x = _c(x, np.uint16)
        w_router = _c(w_router, np.uint16)
        bias = _c(bias, np.float32)
        w_sg = _c(w_sg, np.uint16)
        T, H = x.shape
        E = w_router.shape[0]
        logits = np.empty((T, E), np.float32)
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        s = np.empty(T, np.float64) if w_sg is not None else None
        _check(self.lib.oracle_route(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_sg), T, H, E, k,
                                     _ptr(logits), _ptr(ids), _ptr(w), _ptr(s)), "oracle_route")
        return {"logits": logits, "ids": ids, "w": w, "s": s}

    def route_from_logits(self, logits, k: int):
        logits = _c(logits, np.float32)
        T, E = logits.shape
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        _check(self.lib.oracle_route_from_logits(_ptr(logits), T, E, k, _ptr(ids), _ptr(w)),
               "oracle_route_from_logits")
        return ids, w

    def align(self, ids, E: int):
        """Stable expert grouping: counts[E], offsets[E+1], perm[T*k] (unpadded)."""
        ids = _c(ids, np.int32)
        T, k = ids.shape
        counts = np.empty(E, np.int32)
        offsets = np.empty(E + 1, np.int32)
        perm = np.empty(T * k, np.int32)
        _check(self.lib.oracle_align(_ptr(ids), T, E, k, _ptr(counts), _ptr(offsets), _ptr(perm)),
               "oracle_align")
        return counts, offsets, perm

    def e4m3_decode(self, codes) -> np.ndarray:
        """Values (float64) of OCP FP8 E4M3 codes; NaN for the NaN codes."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape, np.float64)
        _check(self.lib.oracle_e4m3_decode(_ptr(codes), codes.size, _ptr(out)), "oracle_e4m3_decode")
        return out

    def f16_decode(self, bits) -> np.ndarray:
        """Values (float64) of IEEE fp16 bit patterns."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float64)
        _check(self.lib.oracle_f16_decode(_ptr(bits), bits.size, _ptr(out)), "oracle_f16_decode")
        return out

    def q4_dequant(self, codes, scales) -> np.ndarray:
        """Dequantised 4-bit matrix: codes [..., n/2] uint8, fp16 scale bits [..., n/32] -> [..., n] float64."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        n = codes.shape[-1] * 2
        rows = codes.size * 2 // n
        out = np.empty(codes.shape[:-1] + (n,), np.float64)
        _check(self.lib.oracle_q4_dequant(_ptr(codes), _ptr(scales), rows, n, _ptr(out)), "oracle_q4_dequant")
        return out

    def forward(self, inp: Dict[str, np.ndarray], k: Optional[int] = None, ids_in=None,
                want=(), fp8: bool = False, q4: bool = False) -> Dict[str, np.ndarray]:
        """Whole layer on the arrays of ``inp`` (keys as produced by the seeded generator).

        ``want`` may name any of "h", "o", "hs", "os" for per-stage outputs.
        ``fp8``: take the expert weights from the ``*_fp8`` codes and
        ``*_scale`` row scales of ``inp`` instead of the BF16 arrays.
        ``q4``: take them from the ``*_q4`` codes and ``*_q4scale`` fp16
        group scales.
        """
        x = _c(inp["x"], np.uint16)
        wr = _c(inp["w_router"], np.uint16)
        bias = _c(inp.get("bias"), np.float32)
        sfx = "_fp8" if fp8 else ("_q4" if q4 else "")
        dt = np.uint8 if (fp8 or q4) else np.uint16
        wg = _c(inp["w_gate" + sfx], dt)
        wu = _c(inp["w_up" + sfx], dt)
        wd = _c(inp["w_down" + sfx], dt)
        sg = _c(inp.get("ws_gate" + sfx), dt)
        su = _c(inp.get("ws_up" + sfx), dt)
        sd = _c(inp.get("ws_down" + sfx), dt)
        wsg = _c(inp.get("w_sg"), np.uint16)
        T, H = x.shape
        E, I, _ = wg.shape
        I_s = 0 if sg is None else sg.shape[0]
        if k is None:
            k = inp["wl"].k
        ids_in = _c(ids_in, np.int32)
        y = np.empty((T, H), np.float64)
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        s = np.empty(T, np.float64)
        logits = np.empty((T, E), np.float32)
        h = np.empty((T * k, I), np.float64) if "h" in want else None
        o = np.empty((T * k, H), np.float64) if "o" in want else None
        hs = np.empty((T, I_s), np.float64) if ("hs" in want and I_s) else None
        os_ = np.empty((T, H), np.float64) if ("os" in want and I_s) else None
        tail = (_ptr(ids_in), _ptr(y), _ptr(ids), _ptr(w), _ptr(s), _ptr(logits),
                _ptr(h), _ptr(o), _ptr(hs), _ptr(os_))
        if q4:
            codes = (wg, wu, wd, sg, su, sd)
            scales = [_c(inp.get(key + "_q4scale"), np.uint16)
                      for key in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]
            mats = [a for pair in zip(codes, scales) for a in pair]
            _check(self.lib.oracle_forward_q4(_ptr(x), _ptr(wr), _ptr(bias), *[_ptr(a) for a in mats], _ptr(wsg),
                                              T, H, E, k, I, I_s, *tail), "oracle_forward_q4")
        elif fp8:
            codes = (wg, wu, wd, sg, su, sd)
            scales = [_c(inp.get(key + "_scale"), np.float32)
                      for key in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]
            mats = [a for pair in zip(codes, scales) for a in pair]
            _check(self.lib.oracle_forward_fp8(_ptr(x), _ptr(wr), _ptr(bias), *[_ptr(a) for a in mats], _ptr(wsg),
                                               T, H, E, k, I, I_s, *tail), "oracle_forward_fp8")
        else:
            _check(self.lib.oracle_forward(_ptr(x), _ptr(wr), _ptr(bias), _ptr(wg), _ptr(wu), _ptr(wd),
                                           _ptr(sg), _ptr(su), _ptr(sd), _ptr(wsg), T, H, E, k, I, I_s, *tail),
                   "oracle_forward")
        out = {"y": y, "ids": ids, "w": w, "s": s if I_s else None, "logits": logits}
        if h is not None:
            out["h"] = h
        if o is not None:
            out["o"] = o
        if hs is not None:
            out["hs"] = hs
        if os_ is not None:
            out["os"] = os_
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def route(*a, **kw):
    return default().route(*a, **kw)


def route_from_logits(*a, **kw):
    return default().route_from_logits(*a, **kw)


def align(*a, **kw):
    return default().align(*a, **kw)


def forward(*a, **kw):
    return default().forward(*a, **kw)


def e4m3_decode(*a, **kw):
    return default().e4m3_decode(*a, **kw)


def f16_decode(*a, **kw):
    return default().f16_decode(*a, **kw)


def q4_dequant(*a, **kw):
    return default().q4_dequant(*a, **kw)


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between consecutive sorted logits over ranks 0..k (per token).

    A token whose margin is below a threshold is a near-tie: a different
    fp32 summation order may legitimately change its selection or order.
    """
    lg = np.asarray(logits, np.float64)
    srt = -np.sort(-lg, axis=1)
    kk = min(k + 1, lg.shape[1])
    d = srt[:, : kk - 1] - srt[:, 1:kk]
    return d.min(axis=1) if d.shape[1] else np.full(lg.shape[0], np.inf)
