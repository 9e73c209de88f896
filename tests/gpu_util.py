"""Helpers for the GPU parity tests: device setup, inputs, comparison rules.

Comparison rules
  * routing ids / counts / permutation: bit-exact.  On generated inputs a
    token is excluded from the exact-id comparison when its top-k margin
    (smallest gap between consecutive sorted oracle logits over ranks 0..k)
    is below 1e-4, unless it is an engineered exact-tie token (x_t = 0,
    whose logits are the bias on both sides); exclusions are counted.  Ids
    fed from the oracle's own logits are compared for every token.
  * outputs y: max |dy| <= 2e-2 and ||dy||_2 / ||y_ref||_2 <= 1e-2 over all
    tokens; a token whose GPU selection differs (a near-tie) is compared
    with the oracle re-evaluated on the GPU's selection.
"""
from __future__ import annotations

import functools
import os
import sys

import numpy as np
import pytest

import oracle
from sparse_moe_layer_03_amd import synth

MARGIN = 1e-4
Y_MAX_ABS = 2e-2
Y_REL_L2 = 1e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@functools.lru_cache(maxsize=None)
def full_weights(seed: int = 0):
    """Full-shape weights (hidden 2048, 256 experts, FFN 512, shared 512), drawn once."""
    return synth.make_inputs(synth.workload("decode"), seed=seed)


@functools.lru_cache(maxsize=None)
def full_fp8_weights(seed: int = 0):
    """FP8 (E4M3, per-row scale) copies of the full-shape expert weights, made once."""
    return synth.add_fp8_weights(full_weights(seed))


def with_fp8(inp, seed: int = 0):
    """``inp`` plus FP8 expert weights (the cached full-shape ones when the shapes match)."""
    wl = inp["wl"]
    if (wl.H, wl.E, wl.I, wl.I_s) == (2048, 256, 512, 512):
        out = dict(inp)
        src = full_fp8_weights(seed)
        for key in synth.FP8_KEYS:
            out[key + "_fp8"], out[key + "_scale"] = src[key + "_fp8"], src[key + "_scale"]
        return out
    return synth.add_fp8_weights(inp)


@functools.lru_cache(maxsize=None)
def full_q4_weights(seed: int = 0):
    """4-bit (fp16 group scale) copies of the full-shape expert weights, made once."""
    return synth.add_q4_weights(full_weights(seed))


def with_q4(inp, seed: int = 0):
    """``inp`` plus 4-bit expert weights (the cached full-shape ones when the shapes match)."""
    wl = inp["wl"]
    if (wl.H, wl.E, wl.I, wl.I_s) == (2048, 256, 512, 512):
        out = dict(inp)
        src = full_q4_weights(seed)
        for key in synth.FP8_KEYS:
            out[key + "_q4"], out[key + "_q4scale"] = src[key + "_q4"], src[key + "_q4scale"]
        return out
    return synth.add_q4_weights(inp)


def inputs(name: str, T=None, seed: int = 0, **over):
    wl = synth.workload(name, **({"T": T} if T is not None else {}), **over)
    if (wl.H, wl.E, wl.I, wl.I_s) == (2048, 256, 512, 512):
        return synth.make_inputs(wl, seed=seed, reuse=full_weights(seed))
    return synth.make_inputs(wl, seed=seed)


def to_dev_x(inp, device="cuda:0"):
    from sparse_moe_layer_03_amd.layer import to_device_bf16
    return to_device_bf16(inp["x"], device)


def y_to_f64(t) -> np.ndarray:
    from sparse_moe_layer_03_amd.layer import bf16_to_numpy_bits
    return synth.bf16_bits_to_f32(bf16_to_numpy_bits(t)).astype(np.float64)


def excluded_tokens(logits: np.ndarray, k: int, tie_rows=()) -> np.ndarray:
    m = oracle.topk_margin(logits, k)
    ex = m < MARGIN
    if len(tie_rows):
        ex[np.asarray(tie_rows)] = False
    return ex


def check_ids(gpu_ids: np.ndarray, orc_ids: np.ndarray, excluded: np.ndarray, label: str):
    keep = ~excluded
    bad = np.nonzero(np.any(gpu_ids[keep] != orc_ids[keep], axis=1))[0]
    say(f"[{label}] ids: {keep.sum()} compared, {excluded.sum()} near-tie tokens excluded, {len(bad)} mismatches")
    assert len(bad) == 0, f"{label}: ids differ on tokens {np.nonzero(keep)[0][bad][:10]}"


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, label: str):
    d = y_gpu - y_ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(y_ref), 1e-30)) if d.size else 0.0
    say(f"[{label}] y: max|dy| {max_abs:.3e} (<= {Y_MAX_ABS}), rel-L2 {rel:.3e} (<= {Y_REL_L2})")
    assert max_abs <= Y_MAX_ABS and rel <= Y_REL_L2, label
    return max_abs, rel


def oracle_y_with_gpu_ids(inp, rows, gpu_ids, ref, fp8=False, q4=False):
    """Oracle y for ``rows`` of ``inp`` evaluated under ``gpu_ids`` (near-tie tokens)."""
    sub = dict(inp)
    sub["x"] = inp["x"][rows]
    r = oracle.forward(sub, ids_in=gpu_ids, fp8=fp8, q4=q4)
    return r["y"]


def reference_y(inp, gpu_ids: np.ndarray, label: str, fp8: bool = False, q4: bool = False):
    """Oracle y for every token, with near-tie tokens re-evaluated on the GPU's selection.

    ``fp8`` / ``q4``: the oracle takes the FP8 / 4-bit expert weights of ``inp``."""
    r = oracle.forward(inp, fp8=fp8, q4=q4)
    wl = inp["wl"]
    ex = excluded_tokens(r["logits"], wl.k, inp.get("tie_rows", ()))
    check_ids(gpu_ids, r["ids"], ex, label)
    y = r["y"].copy()
    diff = np.nonzero(np.any(gpu_ids != r["ids"], axis=1))[0]
    if len(diff):
        y[diff] = oracle_y_with_gpu_ids(inp, diff, gpu_ids[diff], r, fp8=fp8, q4=q4)
    return y, r


def gpu_env_note():
    return os.environ.get("HIP_VISIBLE_DEVICES", "")
