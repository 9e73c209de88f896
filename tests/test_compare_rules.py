"""The GPU tests' comparison rules, checked on the CPU with oracle outputs and planted mistakes.

check_admissible must accept the oracle's own selection and a swap of two logits closer than the
summation bound, and reject a selection that skips a clearly larger logit, lists its experts out of
rank order, repeats an expert or names one outside [0, E).  check_stage must accept bf16 rounding of
the reference and reject a wrong column.
"""
import numpy as np
import pytest

import oracle
from sparse_moe_layer_03_amd import synth
from tests import gpu_util as G


@pytest.fixture(scope="module")
def routed():
    wl = synth.Workload("rules", T=64, H=256, E=16, k=4, I=128, I_s=0, bias="normal")
    inp = synth.make_inputs(wl, seed=31)
    r = oracle.route(inp["x"], inp["w_router"], inp["bias"], None, wl.k)
    return inp, r


def test_own_selection_is_admissible(routed):
    inp, r = routed
    G.check_admissible(r["ids"], inp, r["logits"], np.arange(64), "own")


def test_swap_within_bound_is_admissible(routed):
    inp, r = routed
    lg = r["logits"].astype(np.float64).copy()
    t = 3
    order = np.argsort(-lg[t], kind="stable")
    a, b = order[3], order[4]  # rank k-1 and the best unselected expert
    lg[t, b] = lg[t, a] - 1e-9  # a near-tie, well inside the summation bound
    ids = r["ids"].copy()
    ids[t, 3] = b
    G.check_admissible(ids, inp, lg.astype(np.float32), [t], "near-tie swap")


def test_clear_misselection_rejected(routed):
    inp, r = routed
    lg = r["logits"]
    t = int(np.argmax(oracle.topk_margin(lg, 4)))  # the clearest token
    order = np.argsort(-lg[t].astype(np.float64), kind="stable")
    ids = r["ids"].copy()
    ids[t, 0] = order[-1]  # the smallest logit instead of the largest
    with pytest.raises(AssertionError):
        G.check_admissible(ids, inp, lg, [t], "wrong expert")
    ids = r["ids"].copy()
    ids[t, [0, 3]] = ids[t, [3, 0]]  # out of rank order
    with pytest.raises(AssertionError):
        G.check_admissible(ids, inp, lg, [t], "wrong order")
    ids = r["ids"].copy()
    ids[t, 1] = ids[t, 0]
    with pytest.raises(AssertionError):
        G.check_admissible(ids, inp, lg, [t], "repeat")
    ids = r["ids"].copy()
    ids[t, 2] = 16
    with pytest.raises(AssertionError):
        G.check_admissible(ids, inp, lg, [t], "out of range")


def test_stage_bound():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((200, 96))
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    G.check_stage(got, ref, "bf16 rounding")
    bad = got.copy()
    bad[:, 7] = got[:, 8]  # a wrong column
    with pytest.raises(AssertionError):
        G.check_stage(bad, ref, "wrong column")


def test_down_rounding_bound():
    """o computed from bf16-rounded h (as the GPU does) is inside the bound; a wrong column is not."""
    rng = np.random.default_rng(6)
    T, k, E, H, I = 40, 2, 3, 64, 32
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    h = rng.standard_normal((T * k, I)) * 0.5
    wd = synth.f32_to_bf16_bits((rng.standard_normal((E, H, I)) * 0.02).astype(np.float32))
    wf = synth.bf16_bits_to_f32(wd).astype(np.float64)
    e_of = ids.reshape(-1)
    o_ref = np.einsum("ai,aci->ac", h, wf[e_of])
    h_bf = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(h.astype(np.float32))).astype(np.float64)
    o_gpu = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        np.einsum("ai,aci->ac", h_bf, wf[e_of]).astype(np.float32))).astype(np.float64)
    extra = G.down_rounding_bound(h, ids, wd)
    G.check_stage(o_gpu, o_ref, "o from rounded h", extra=extra)
    bad = o_gpu.copy()
    bad[:, 3] = o_gpu[:, 4]
    with pytest.raises(AssertionError):
        G.check_stage(bad, o_ref, "o wrong column", extra=extra)
