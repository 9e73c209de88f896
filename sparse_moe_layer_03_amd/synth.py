"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module only draws numbers.  It holds none of the layer's arithmetic
(no router, no top-k, no FFN, no combine), so both the oracle's tests and
the HIP path's tests, the benchmark and the smoke check may take their
inputs from it without sharing any of the method.

Workloads are named by what they are.  The shapes follow the Qwen3-class
MoE block that the engine pages run as a selected-expert MoE path
(guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B", section on the data path;
kongchang.com "GFX1151 engine", section on the MoE kernel, which defines
MoE as many expert sub-networks of which only a few are active per step).

Every array that the layer reads in BF16 is returned as ``uint16`` bit
patterns (round-to-nearest-even from float32 draws); the router bias is
float32.

Draws: every tensor has a fixed id (x 0, W_router 1, bias 2, W_gate 3,
W_up 4, W_down 5, Ws_gate 6, Ws_up 7, Ws_down 8, w_sg 9, tie rows 10,
Zipf rank permutation 11).  A tensor is flattened row-major and cut into
blocks of 2**20 values; block b is ``standard_normal(dtype=float32)`` from
``numpy.random.default_rng([seed, tensor_id, b])`` (PCG64 seeded by a
SeedSequence over that triple), scaled by the tensor's sigma and rounded to
bf16.  Blocks are independent, so they are drawn on several threads, and a
tensor's values do not depend on the shapes of the other tensors (the
weights of a workload are the same for every token count T).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

WEIGHT_SIGMA = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    I_s: int
    bias: Optional[str] = None  # None | "normal" | "zipf"
    bias_sigma: float = 1.0
    zipf_s: float = 1.1
    tie_frac: float = 0.0  # fraction of tokens given x_t = 0 (exact ties)
    note: str = field(default="", compare=False)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", T=16, H=256, E=8, k=2, I=128, I_s=0,
                     note="T=16, hidden 256, 8 experts, top-2, FFN 128, no shared expert"),
    "decode": Workload("decode", T=1, H=2048, E=256, k=8, I=512, I_s=512,
                       note="T=1 decode step, hidden 2048, 256 experts, top-8, FFN 512, shared expert 512"),
    "prefill1k": Workload("prefill1k", T=1024, H=2048, E=256, k=8, I=512, I_s=512,
                          note="T=1024 short prefill, no router bias (near-uniform load)"),
    "prefill8k": Workload("prefill8k", T=8192, H=2048, E=256, k=8, I=512, I_s=512,
                          bias="normal", bias_sigma=1.0,
                          note="T=8192 long prefill, router bias ~ N(0,1) (uneven load)"),
    "skew32k": Workload("skew32k", T=32768, H=2048, E=256, k=8, I=512, I_s=512,
                        bias="zipf", zipf_s=1.1, tie_frac=0.01,
                        note="T=32768 skewed chunk, Zipf(1.1) expert popularity, 1% exact-tie tokens"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BLOCK = 1 << 20
TENSOR_IDS = {"x": 0, "w_router": 1, "bias": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
              "ws_gate": 6, "ws_up": 7, "ws_down": 8, "w_sg": 9, "tie_rows": 10, "zipf_perm": 11}
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _rng(seed: int, name: str, block: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, TENSOR_IDS[name], block])


def _draw_bf16(seed: int, name: str, shape, sigma: float) -> np.ndarray:
    """Blockwise seeded normal draws scaled by sigma, rounded to bf16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def fill(b):
        s0 = b * BLOCK
        m = min(BLOCK, n - s0)
        v = _rng(seed, name, b).standard_normal(m, dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        out[s0:s0 + m] = f32_to_bf16_bits(v)

    nb = (n + BLOCK - 1) // BLOCK
    if nb <= 2:
        for b in range(nb):
            fill(b)
    else:
        list(_pool().map(fill, range(nb)))
    return out.reshape(shape)


def zipf_log_pmf_bias(rng: np.random.Generator, E: int, s: float) -> np.ndarray:
    """Per-expert bias b_e = ln p(r_e), p(r) = r^-s / sum_r' r'^-s, r_e a seeded permutation of 1..E."""
    ranks = rng.permutation(E).astype(np.float64) + 1.0
    norm = np.sum(np.arange(1, E + 1, dtype=np.float64) ** (-s))
    return (np.log(ranks ** (-s) / norm)).astype(np.float32)


def make_inputs(wl, seed: int = 0, reuse: Optional[Dict[str, object]] = None, **overrides) -> Dict[str, np.ndarray]:
    """Seeded inputs of workload ``wl`` (a name or a Workload).

    Returns a dict with keys x, w_router, bias, w_gate, w_up, w_down,
    ws_gate, ws_up, ws_down, w_sg (absent tensors are None) and the
    workload itself under "wl".  ``reuse``: the result of an earlier call
    with the same seed and layer shapes (H, E, I, I_s); its weight arrays are
    taken as they are instead of being drawn again (they would be identical).
    """
    if isinstance(wl, str):
        wl = workload(wl, **overrides)
    elif overrides:
        wl = replace(wl, **overrides)
    T, H, E, k, I, I_s = wl.T, wl.H, wl.E, wl.k, wl.I, wl.I_s
    out: Dict[str, object] = {"wl": wl}
    out["x"] = _draw_bf16(seed, "x", (T, H), 1.0)
    out["w_router"] = _draw_bf16(seed, "w_router", (E, H), WEIGHT_SIGMA)
    if wl.bias == "normal":
        out["bias"] = (_rng(seed, "bias").standard_normal(E, dtype=np.float32)
                       * np.float32(wl.bias_sigma)).astype(np.float32)
    elif wl.bias == "zipf":
        out["bias"] = zipf_log_pmf_bias(_rng(seed, "zipf_perm"), E, wl.zipf_s)
    else:
        out["bias"] = None
    if reuse is not None:
        rw = reuse["wl"]
        if (reuse.get("seed", seed), rw.H, rw.E, rw.I, rw.I_s) != (seed, H, E, I, I_s):
            raise ValueError("reuse: weights were drawn for another seed or layer shape")
        for key in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down", "w_sg"):
            out[key] = reuse[key]
    else:
        out["w_gate"] = _draw_bf16(seed, "w_gate", (E, I, H), WEIGHT_SIGMA)
        out["w_up"] = _draw_bf16(seed, "w_up", (E, I, H), WEIGHT_SIGMA)
        out["w_down"] = _draw_bf16(seed, "w_down", (E, H, I), WEIGHT_SIGMA)
        if I_s > 0:
            out["ws_gate"] = _draw_bf16(seed, "ws_gate", (I_s, H), WEIGHT_SIGMA)
            out["ws_up"] = _draw_bf16(seed, "ws_up", (I_s, H), WEIGHT_SIGMA)
            out["ws_down"] = _draw_bf16(seed, "ws_down", (H, I_s), WEIGHT_SIGMA)
            out["w_sg"] = _draw_bf16(seed, "w_sg", (H,), WEIGHT_SIGMA)
        else:
            out["ws_gate"] = out["ws_up"] = out["ws_down"] = out["w_sg"] = None
    out["seed"] = seed
    if wl.tie_frac > 0.0:
        n_tie = int(round(wl.tie_frac * T))
        rows = (np.sort(_rng(seed, "tie_rows").choice(T, size=n_tie, replace=False)) if n_tie
                else np.zeros(0, np.int64))
        out["x"][rows] = 0
        out["tie_rows"] = rows.astype(np.int64)
        b = out["bias"]
        if b is None:
            b = np.zeros(E, dtype=np.float32)
            out["bias"] = b
        # Equal values at the k-th/(k+1)-th boundary and inside the top-k, so
        # the tokens with x_t = 0 (whose logits are exactly b) need the
        # lowest-index rule to decide both the set and the order.
        order = np.lexsort((np.arange(E), -b.astype(np.float64)))
        if E > k:
            b[order[k]] = b[order[k - 1]]
        if k >= 3:
            b[order[2]] = b[order[1]]
    else:
        out["tie_rows"] = np.zeros(0, dtype=np.int64)
    return out


def make_logits(T: int, E: int, seed: int = 0, sigma: float = 0.905, tie_frac: float = 0.01,
                k: int = 8) -> np.ndarray:
    """Random fp32 router logits with a share of rows carrying exact ties.

    In a tie row the values at several positions are copied from other
    positions of the same row (so some of them land on the k/k+1 boundary
    and inside the top-k), and one position gets -0.0 paired with a +0.0.
    """
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((T, E), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    n_tie = int(round(tie_frac * T))
    rows = rng.choice(T, size=n_tie, replace=False) if n_tie else []
    for r in rows:
        order = np.lexsort((np.arange(E), -lg[r].astype(np.float64)))
        kk = min(k, E - 1)
        if E > kk:
            lg[r, order[kk]] = lg[r, order[kk - 1]]
        if kk >= 3:
            lg[r, order[2]] = lg[r, order[1]]
        if E >= 4:
            a, c = rng.choice(E, size=2, replace=False)
            lg[r, a] = np.float32(-0.0)
            lg[r, c] = np.float32(0.0)
    return lg


FP8_KEYS = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
E4M3_MAX = 448.0


def add_fp8_weights(inp: Dict[str, object]) -> Dict[str, object]:
    """Add FP8 copies of the expert weights of ``inp`` (a make_inputs result).

    For every expert matrix key K in FP8_KEYS that is present, adds
    ``K + "_fp8"`` (uint8 E4M3 codes, same shape) and ``K + "_scale"``
    (float32, one per output row, shape = the matrix shape without its last
    axis).  The scale of a row is its largest magnitude / 448 (1 for an
    all-zero row); the codes are torch's float32 -> float8_e4m3fn cast of
    the bf16 values divided by the row's scale, clamped to +-448 first.
    Returns a new dict; the BF16 arrays stay as they are.
    """
    import torch

    out = dict(inp)
    for key in FP8_KEYS:
        w = inp.get(key)
        if w is None:
            out[key + "_fp8"] = out[key + "_scale"] = None
            continue
        v = torch.from_numpy(bf16_bits_to_f32(w))
        amax = v.abs().amax(dim=-1)
        scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
        q = (v / scale.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        out[key + "_fp8"] = q.view(torch.uint8).numpy().copy()
        out[key + "_scale"] = scale.numpy().copy()
    return out


Q4_GROUP = 32


def add_q4_weights(inp: Dict[str, object]) -> Dict[str, object]:
    """Add 4-bit copies of the expert weights of ``inp`` (a make_inputs result).

    For every expert matrix key K in FP8_KEYS that is present, adds
    ``K + "_q4"`` (uint8, last axis halved: two signed 4-bit weights per
    byte, the even index in the low nibble) and ``K + "_q4scale"`` (uint16
    fp16 bit patterns, last axis / 32: one scale per group of 32 weights).
    The scale of a group is its largest magnitude / 7 rounded to fp16 by
    NumPy (1 for an all-zero group); the weights are the bf16 values divided
    by the group's scale, rounded to the nearest integer (NumPy's rint) and
    clamped to [-8, 7].  Returns a new dict; the BF16 arrays stay as they are.
    """
    out = dict(inp)
    for key in FP8_KEYS:
        w = inp.get(key)
        if w is None:
            out[key + "_q4"] = out[key + "_q4scale"] = None
            continue
        v = bf16_bits_to_f32(w).astype(np.float32)
        shape = v.shape
        g = v.reshape(shape[:-1] + (shape[-1] // Q4_GROUP, Q4_GROUP))
        amax = np.abs(g).max(axis=-1)
        scale = np.where(amax > 0, amax / np.float32(7.0), np.float32(1.0)).astype(np.float16)
        s32 = scale.astype(np.float32)
        s32 = np.where(s32 > 0, s32, np.float32(1.0))
        q = np.clip(np.rint(g / s32[..., None]), -8, 7).astype(np.int8).reshape(shape)
        u = (q.astype(np.int16) & 15).astype(np.uint8)
        out[key + "_q4"] = (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
        out[key + "_q4scale"] = scale.view(np.uint16).copy()
    return out


def content_hash(inputs: Dict[str, object]) -> str:
    h = hashlib.sha256()
    for key in ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down", "w_sg"):
        v = inputs.get(key)
        h.update(key.encode())
        if v is not None:
            h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()[:16]
