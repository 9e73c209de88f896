"""GPU parity of the 4-bit-weight path (moe_forward_q4) against the oracle.

Expert weights are signed 4-bit integers with an fp16 scale per group of 32
weights of a row (kongchang.com "GFX1151 engine", section on the two weight
formats, names 4-bit GGUF weights; the group layout is this library's own
reading).  The single-token and small-batch kernels are checked against the
oracle's 4-bit layer under the BF16 tolerance, and against the BF16 kernels
bitwise where the dequantised weights are exact in BF16.
"""
import numpy as np
import pytest

from sparse_moe_layer_03_amd import moe, synth
from sparse_moe_layer_03_amd.layer import DeviceLayer
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return G.torch_cuda()


@pytest.fixture(scope="module")
def q4_layer(torch):
    """Full-shape layer (hidden 2048, 256 experts, top-8, FFN 512, shared 512) with 4-bit expert weights."""
    G.say("[setup] quantising the full-shape weights to 4 bits and uploading them")
    return DeviceLayer(G.full_q4_weights(0), k=8, q4=True)


def _q4_layer_for(inp, q4_layer):
    wl = inp["wl"]
    if (wl.H, wl.E, wl.I, wl.I_s, wl.k) == (2048, 256, 512, 512, 8):
        import torch
        q4_layer.bias = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to("cuda:0")
        return q4_layer
    return DeviceLayer.from_inputs(inp, q4=True)


Q4_CASES = [
    ("full-T1", dict(wl="decode", T=1)),
    ("full-T1-bias", dict(wl="prefill8k", T=1)),
    ("full-T2", dict(wl="prefill1k", T=2)),
    ("full-T8", dict(wl="prefill1k", T=8)),
    ("full-T32-bias", dict(wl="prefill8k", T=32)),
    ("k16-T1", dict(wl=synth.Workload("q16", T=1, H=512, E=32, k=16, I=256, I_s=128))),
    ("k16-T20", dict(wl=synth.Workload("q16b", T=20, H=512, E=32, k=16, I=256, I_s=128))),
    ("noshared-T1", dict(wl=synth.Workload("q9", T=1, H=256, E=12, k=9, I=384, I_s=0))),
    ("noshared-T7", dict(wl=synth.Workload("q9b", T=7, H=256, E=12, k=9, I=384, I_s=0))),
    ("wide-T1", dict(wl=synth.Workload("qw", T=1, H=4096, E=64, k=4, I=640, I_s=256, bias="normal"))),
    ("wide-T10", dict(wl=synth.Workload("qwb", T=10, H=4096, E=64, k=4, I=640, I_s=256, bias="normal"))),
    ("k1-T5", dict(wl=synth.Workload("q1", T=5, H=256, E=8, k=1, I=128, I_s=128))),
]


def _case_inputs(case, seed=4):
    wl = case["wl"]
    if isinstance(wl, str):
        return G.with_q4(G.inputs(wl, case.get("T")))
    return synth.add_q4_weights(synth.make_inputs(wl, seed=seed))


@pytest.mark.parametrize("label,case", Q4_CASES, ids=[c[0] for c in Q4_CASES])
def test_q4_parity(torch, q4_layer, label, case):
    """moe_forward_q4 at 1..32 tokens vs the oracle's 4-bit layer; ids exact outside near-ties."""
    inp = _case_inputs(case)
    wl = inp["wl"]
    T = inp["x"].shape[0]
    G.say(f"[q4] {label}: T={T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} I_s={wl.I_s}")
    lay = _q4_layer_for(inp, q4_layer)
    y = lay.forward(G.to_dev_x(inp))
    ids = lay.forward_ids(T).cpu().numpy()
    torch.cuda.synchronize()
    y_ref, _ = G.reference_y(inp, ids, f"q4 {label}", q4=True)
    G.check_y(G.y_to_f64(y), y_ref, f"q4 {label}")


def _exact_q4(inp, seed):
    """Random 4-bit weights and power-of-two fp16 group scales, and the BF16 matrices they dequantise to."""
    rng = np.random.default_rng(seed)
    out = dict(inp)
    for key in synth.FP8_KEYS:
        if inp.get(key) is None:
            out[key + "_q4"] = out[key + "_q4scale"] = None
            continue
        shape = inp[key].shape
        q = rng.integers(-8, 8, size=shape)
        sc = np.ldexp(1.0, rng.integers(-9, -5, size=shape[:-1] + (shape[-1] // 32,))).astype(np.float16)
        u = (q.astype(np.int16) & 15).astype(np.uint8)
        out[key + "_q4"] = (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
        out[key + "_q4scale"] = sc.view(np.uint16)
        vals = q.astype(np.float32) * np.repeat(sc.astype(np.float32), 32, axis=-1)
        out[key] = synth.f32_to_bf16_bits(vals)
        assert np.array_equal(synth.bf16_bits_to_f32(out[key]), vals)
    return out


@pytest.mark.parametrize("T", [1, 2, 13, 32])
def test_q4_equals_bf16_kernels_on_exact_weights(torch, T):
    """Power-of-two group scales make every dequantised weight exact in BF16 and every product the same
    number, so the 4-bit kernels give bitwise the BF16 kernels' output on those BF16 weights."""
    wl = synth.Workload("qx", T=T, H=1024, E=32, k=6, I=384, I_s=256, bias="normal")
    inp = _exact_q4(synth.make_inputs(wl, seed=8), seed=T)
    G.say(f"[q4-vs-bf16] T={T}")
    x = G.to_dev_x(inp)
    y4 = DeviceLayer.from_inputs(inp, q4=True).forward(x)
    y16 = DeviceLayer.from_inputs(inp).forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y4.view(torch.int16), y16.view(torch.int16))


def test_q4_graph_replay_and_determinism(torch, q4_layer):
    """4-bit decode and small-batch calls: eager repeats and HIP-graph replays are bitwise identical."""
    for T in (1, 16):
        inp = G.with_q4(G.inputs("prefill1k", T))
        lay = _q4_layer_for(inp, q4_layer)
        x = G.to_dev_x(inp)
        y1 = lay.forward(x).clone()
        y2 = lay.forward(x).clone()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        yg = torch.empty_like(y1)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            lay.forward(x, y=yg)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lay.forward(x, y=yg)
        for i in range(3):
            yg.zero_()
            g.replay()
            torch.cuda.synchronize()
            _ = (x.float() * 2).sum().item()
            assert torch.equal(yg.view(torch.int16), y1.view(torch.int16)), f"T={T} replay {i}"


def test_q4_rejects_large_T(torch, q4_layer):
    inp = G.with_q4(G.inputs("prefill1k", moe.Q4_MAX_T + 1))
    with pytest.raises(moe.MoEError):
        _q4_layer_for(inp, q4_layer).forward(G.to_dev_x(inp))
