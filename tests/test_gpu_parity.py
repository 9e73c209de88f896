"""GPU parity: every stage of the HIP path, through the C ABI, against the CPU oracle.

Run on an MI355X:  python -u -m pytest tests -m gpu -x -v --timeout 300
"""
import os
import sys

import numpy as np
import pytest

import oracle
from sparse_moe_layer_03_amd import moe, synth
from sparse_moe_layer_03_amd.layer import DeviceLayer
from tests import gpu_util as G
from tests.boundary_case import BOUNDARY_CASES, check_align, run_boundary_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return G.torch_cuda()


@pytest.fixture(scope="module")
def full_layer(torch):
    """Full-shape layer (hidden 2048, 256 experts, top-8, FFN 512, shared 512) on cuda:0."""
    G.say("[setup] drawing full-shape weights and uploading them")
    return DeviceLayer(G.full_weights(0), k=8)


def _layer_for(inp, full_layer):
    wl = inp["wl"]
    if (wl.H, wl.E, wl.I, wl.I_s, wl.k) == (2048, 256, 512, 512, 8) and full_layer is not None:
        import torch
        full_layer.bias = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to("cuda:0")
        return full_layer
    return DeviceLayer.from_inputs(inp)


# ----------------------------------------------------------------- routing
@pytest.mark.parametrize("T,E,k", [(4096, 256, 8), (333, 8, 2), (1000, 64, 16), (77, 256, 1), (5, 3, 3)])
def test_route_from_logits_bit_exact(torch, T, E, k):
    """Top-k on the oracle-supplied logits: ids bit-exact for every token, ties included."""
    G.say(f"[route_from_logits] T={T} E={E} k={k}")
    lg = synth.make_logits(T, E, seed=T + E, tie_frac=0.05, k=k)
    ids_ref, w_ref = oracle.route_from_logits(lg, k)
    d_lg = torch.from_numpy(lg).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route_from_logits(d_lg, T, E, k, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=0, atol=1e-6)


ROUTE_CASES = [("tiny", None), ("prefill1k", 300), ("prefill8k", 1000), ("skew32k", 2048)]


@pytest.mark.parametrize("streamed", [True, False], ids=["streamed", "staged"])
@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_generated(torch, full_layer, name, T, streamed):
    """Router GEMM + top-k on generated inputs, both forms (W_router copied in operand order and
    streamed into registers, as moe_forward runs it; W_router staged through LDS): ids exact outside
    near-ties; logits, w, s close."""
    G.say(f"[route] {name} T={T} streamed={streamed}")
    inp = G.inputs(name, T)
    _check_route(torch, inp, _layer_for(inp, full_layer), streamed, name)


ROUTE_SHAPES = [
    # (label, workload): streamed form with 1 to 8 groups of 32 experts (a group's K split over
    # 4, 2 or 1 waves, idle waves when E <= 224), 4 to 32 sub-steps per block, H in segments
    # of 2048 (x tile streamed in the first), expert counts that leave columns past E in a
    # group, k = 1 and k = E, no bias, no shared gate, ragged token counts
    ("E3-H256-T33", synth.Workload("r3", T=33, H=256, E=3, k=2, I=128, I_s=128, bias="normal")),
    ("E5-kE-noshared", synth.Workload("r5", T=100, H=512, E=5, k=5, I=128, I_s=0)),
    ("E13-k1-T257", synth.Workload("r13", T=257, H=1024, E=13, k=1, I=128, I_s=128, bias="normal")),
    ("E64-k16-H4096", synth.Workload("r64", T=70, H=4096, E=64, k=16, I=256, I_s=256)),
    ("E200-H768-T1500", synth.Workload("r200", T=1500, H=768, E=200, k=6, I=128, I_s=0, bias="normal")),
    ("E256-T33", synth.Workload("r256", T=33, H=2048, E=256, k=8, I=512, I_s=512, bias="normal")),
    ("E100-H1536-T65", synth.Workload("r100", T=65, H=1536, E=100, k=4, I=128, I_s=128, bias="normal")),
    ("E256-H2560-T40", synth.Workload("r256w", T=40, H=2560, E=256, k=8, I=128, I_s=128, bias="normal")),
]


@pytest.mark.parametrize("streamed", [True, False], ids=["streamed", "staged"])
@pytest.mark.parametrize("name,wl", ROUTE_SHAPES)
def test_route_shapes(torch, name, wl, streamed):
    """Both router forms at shapes that exercise the streamed router's wave layouts, block depths
    and K segments, and the selection's edge cases, against the oracle."""
    G.say(f"[route-shape] {name} streamed={streamed}")
    inp = synth.make_inputs(wl, seed=5)
    _check_route(torch, inp, DeviceLayer.from_inputs(inp), streamed, name)


def _check_route(torch, inp, lay, streamed, name):
    x = G.to_dev_x(inp)
    Tn = x.shape[0]
    b = lay.alloc_stage_buffers(Tn)
    lay.run_route(x, b, streamed=streamed)
    torch.cuda.synchronize()
    wl = inp["wl"]
    r = oracle.route(inp["x"], inp["w_router"], inp["bias"], inp["w_sg"], wl.k)
    lg = b["logits"].cpu().numpy()
    # fp32 sums of the same products in another order: within the summation bound
    xf = synth.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    wf = synth.bf16_bits_to_f32(inp["w_router"]).astype(np.float64)
    bound = 2 * wl.H * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T) + 1e-6
    assert np.all(np.abs(lg.astype(np.float64) - r["logits"]) <= bound)
    ex = G.excluded_tokens(r["logits"], wl.k, inp.get("tie_rows", ()))
    ids = b["ids"].cpu().numpy()
    G.check_ids(ids, r["ids"], ex, f"route {name}", inp=inp, logits=r["logits"])
    same = np.all(ids == r["ids"], axis=1)
    # w_j = exp(l_j - l_0) / sum: a logit error d moves w_j by at most about 2 w_j max|d|
    dl = np.abs(lg.astype(np.float64) - r["logits"]).max(axis=1, keepdims=True)
    dw = np.abs(b["w"].cpu().numpy().astype(np.float64) - r["w"])
    assert np.all((dw <= 1e-6 + 2.0 * dl)[same])
    if wl.I_s:
        np.testing.assert_allclose(b["s"].cpu().numpy()[:Tn], r["s"], rtol=0, atol=1e-6)
    if len(inp.get("tie_rows", ())):
        rows = inp["tie_rows"]
        assert np.array_equal(lg[rows], np.broadcast_to(inp["bias"], lg[rows].shape))


# ------------------------------------------------------------------- align
@pytest.mark.parametrize("name,T", [("tiny", None), ("prefill1k", 1024), ("prefill8k", 8192), ("skew32k", 32768)])
def test_align_exact(torch, full_layer, name, T):
    """Align on the GPU's own ids equals the oracle's stable grouping, bit for bit."""
    G.say(f"[align] {name} T={T}")
    inp = G.inputs(name, T)
    lay = _layer_for(inp, full_layer)
    x = G.to_dev_x(inp)
    b = lay.alloc_stage_buffers(x.shape[0])
    lay.run_route(x, b)
    lay.run_align(x.shape[0], b)
    torch.cuda.synchronize()
    wl = inp["wl"]
    check_align(b, b["ids"].cpu().numpy(), x.shape[0], wl.E, wl.k)


# -------------------------------------------------------------- whole layer
SMALL = synth.Workload("small", T=200, H=512, E=16, k=4, I=256, I_s=128, bias="normal", bias_sigma=0.5)
SMALL_BM128 = synth.Workload("small128", T=700, H=256, E=16, k=6, I=128, I_s=128)
SMALL_BM32 = synth.Workload("small32", T=45, H=256, E=12, k=3, I=384, I_s=0)

WIDE = synth.Workload("wide", T=96, H=4096, E=32, k=4, I=256, I_s=256, bias="normal", bias_sigma=0.5)
K16 = synth.Workload("k16", T=70, H=512, E=32, k=16, I=256, I_s=128)

LAYER_CASES = [
    ("tiny", dict(wl="tiny")),
    ("wide-H4096", dict(wl=WIDE)),
    ("k16", dict(wl=K16)),
    ("small-bm64", dict(wl=SMALL)),
    ("small-bm128", dict(wl=SMALL_BM128)),
    ("small-bm32", dict(wl=SMALL_BM32)),
    ("full-T300", dict(wl="prefill1k", T=300)),
    ("full-T2", dict(wl="prefill1k", T=2)),
    ("full-bias-T257", dict(wl="prefill8k", T=257)),
    # 64-row combine tiles (2049 <= T < 8192), 256-row routed tiles (mean 156 rows per expert)
    ("full-T5000", dict(wl="prefill1k", T=5000)),
    # the persistent 256-row kernel at the lowest mean that takes it (64 rows per expert: most tiles
    # hold about a quarter data rows), and 64-row tiles just below it
    ("full-T2048", dict(wl="prefill1k", T=2048)),
    ("full-T2047", dict(wl="prefill1k", T=2047)),
]


def _inputs_for(case):
    wl = case["wl"]
    if isinstance(wl, str):
        return G.inputs(wl, case.get("T"))
    return synth.make_inputs(wl, seed=3)


@pytest.mark.parametrize("label,case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_parity(torch, full_layer, label, case):
    """moe_forward vs the oracle within the BF16 tolerance; stage outputs checked too."""
    inp = _inputs_for(case)
    wl = inp["wl"]
    G.say(f"[layer] {label}: T={inp['x'].shape[0]} H={wl.H} E={wl.E} k={wl.k} I={wl.I} I_s={wl.I_s} "
          f"BIG={moe.moe_align_tile_rows(inp['x'].shape[0], wl.E, wl.k)}")
    lay = _layer_for(inp, full_layer)
    x = G.to_dev_x(inp)
    T = x.shape[0]
    y = lay.forward(x)
    fwd_ids = lay.forward_ids(T).cpu().numpy()
    b = lay.run_stages(x)
    torch.cuda.synchronize()
    ids = b["ids"].cpu().numpy()
    y_ref, r = G.reference_y(inp, ids, label)
    if 2 <= T <= moe.SMALL_BATCH_MAX_T:
        # moe_forward runs the small-batch kernels, the stage entry points the
        # tiled ones: each against the oracle under its own selection
        G.check_y(G.y_to_f64(b["y"]), y_ref, label + " (stages)")
        y_ref_f, _ = G.reference_y(inp, fwd_ids, label + " (forward)")
        G.check_y(G.y_to_f64(y), y_ref_f, label + " (forward)")
    else:
        G.check_y(G.y_to_f64(y), y_ref, label)
        # the staged path runs the same kernels: bitwise identical to moe_forward
        assert torch.equal(b["y"].view(torch.int16), y.view(torch.int16))
        assert np.array_equal(fwd_ids, ids)
    # stages h (padded rows, reached through inv) and o (one row per
    # assignment t*k + j): every element against the oracle's, for tokens
    # with the same selection
    same = np.all(ids == r["ids"], axis=1)
    if same.sum() > 0:
        ro = oracle.forward(inp, want=("h", "o"))
        inv = b["inv"].cpu().numpy()
        sel = np.repeat(same, wl.k)
        h_got = G.y_to_f64(b["h"][torch.from_numpy(inv).long().cuda()])
        G.check_stage(h_got[sel], ro["h"][sel], f"{label} h")
        G.check_stage(G.y_to_f64(b["o"])[sel], ro["o"][sel], f"{label} o",
                      extra=G.down_rounding_bound(ro["h"][sel], ids[same], inp["w_down"]))


# ------------------------------------------------------------ small batches
SMALL_BATCH_CASES = [
    ("full-T2", dict(wl="prefill1k", T=2)),
    ("full-T3-bias", dict(wl="prefill8k", T=3)),
    ("full-T8", dict(wl="prefill1k", T=8)),
    ("full-T16-bias", dict(wl="prefill8k", T=16)),
    ("full-T24", dict(wl="prefill1k", T=24)),
    ("full-T32-bias", dict(wl="prefill8k", T=32)),
    ("k16-T20", dict(wl=synth.Workload("sb16", T=20, H=512, E=32, k=16, I=256, I_s=128))),
    ("noshared-T7", dict(wl=synth.Workload("sb9", T=7, H=256, E=12, k=9, I=384, I_s=0))),
    ("wide-T10", dict(wl=synth.Workload("sbw", T=10, H=4096, E=64, k=4, I=640, I_s=256, bias="normal"))),
    ("k1-T5", dict(wl=synth.Workload("sb1", T=5, H=256, E=8, k=1, I=128, I_s=128))),
    ("kE-T4", dict(wl=synth.Workload("sbE", T=4, H=256, E=8, k=8, I=128, I_s=128))),
]


@pytest.mark.parametrize("label,case", SMALL_BATCH_CASES, ids=[c[0] for c in SMALL_BATCH_CASES])
def test_small_batch_parity(torch, full_layer, label, case):
    """moe_forward at 2..32 tokens (the small-batch kernels) vs the oracle, under the GPU's own selection
    for near-tie tokens; ids exact elsewhere."""
    inp = _inputs_for(case)
    wl = inp["wl"]
    T = inp["x"].shape[0]
    assert 2 <= T <= moe.SMALL_BATCH_MAX_T
    G.say(f"[small-batch] {label}: T={T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} I_s={wl.I_s}")
    lay = _layer_for(inp, full_layer)
    y = lay.forward(G.to_dev_x(inp))
    ids = lay.forward_ids(T).cpu().numpy()
    torch.cuda.synchronize()
    y_ref, _ = G.reference_y(inp, ids, label)
    G.check_y(G.y_to_f64(y), y_ref, label)


def test_small_batch_graph_and_determinism(torch, full_layer):
    """Small-batch calls: repeated eager calls and HIP-graph replays are bitwise identical."""
    inp = G.inputs("prefill8k", 24)
    lay = _layer_for(inp, full_layer)
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
        assert torch.equal(yg.view(torch.int16), y1.view(torch.int16)), f"replay {i}"


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_decode_parity(torch, full_layer, seed):
    """T = 1 decode path (GEMVs over the selected experts) vs the oracle."""
    G.say(f"[decode] seed={seed}")
    inp = G.inputs("decode", 1, seed=0)
    inp["x"] = synth._draw_bf16(100 + seed, "x", (1, 2048), 1.0)
    lay = _layer_for(inp, full_layer)
    x = G.to_dev_x(inp)
    y = lay.forward(x)
    ids = lay.forward_ids(1).cpu().numpy()
    torch.cuda.synchronize()
    # a near-tie token is compared under the GPU's (admissible) selection
    y_ref, _ = G.reference_y(inp, ids, f"decode seed {seed}")
    G.check_y(G.y_to_f64(y), y_ref, f"decode seed {seed}")


DECODE_SHAPES = [
    ("k16-shared", synth.Workload("d16", T=1, H=512, E=32, k=16, I=256, I_s=128)),
    ("k9-noshared", synth.Workload("d9", T=1, H=256, E=12, k=9, I=384, I_s=0)),
    ("wide-H4096", synth.Workload("dwide", T=1, H=4096, E=64, k=4, I=640, I_s=256, bias="normal")),
    ("k1", synth.Workload("d1", T=1, H=256, E=8, k=1, I=128, I_s=128)),
]


@pytest.mark.parametrize("label,wl", DECODE_SHAPES, ids=[c[0] for c in DECODE_SHAPES])
def test_decode_shapes(torch, label, wl):
    """Decode kernels at other shapes: k above 8 (the wide top-k template), no shared expert, H above
    2048 (several chunk groups per row), I not a multiple of 512, k = 1."""
    G.say(f"[decode-shape] {label}")
    inp = synth.make_inputs(wl, seed=4)  # seed 4: the token's top-k margin is >= 4e-3 for every shape here
    lay = DeviceLayer.from_inputs(inp)
    y = lay.forward(G.to_dev_x(inp))
    torch.cuda.synchronize()
    r = oracle.forward(inp)
    assert not G.excluded_tokens(r["logits"], wl.k)[0]
    G.check_y(G.y_to_f64(y), r["y"], f"decode {label}")


def test_decode_with_bias_and_zero_token(torch, full_layer):
    """Decode with a router bias; a zero token gives exactly zero output."""
    inp = G.inputs("prefill8k", 1)
    lay = _layer_for(inp, full_layer)
    x = G.to_dev_x(inp)
    y = lay.forward(x)
    torch.cuda.synchronize()
    r = oracle.forward(inp)
    G.check_y(G.y_to_f64(y), r["y"], "decode biased")
    x.zero_()
    y0 = lay.forward(x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y0.view(torch.int16)).item() == 0


def test_decode_repeated_calls(torch, full_layer):
    """Many single-token calls on one workspace, each with its own token: every call matches the oracle."""
    inp = G.inputs("decode", 1, seed=0)
    lay = _layer_for(inp, full_layer)
    n = 24
    xs = synth._draw_bf16(300, "x", (n, 2048), 1.0)
    ys, ids = [], []
    for i in range(n):
        sub = dict(inp)
        sub["x"] = xs[i:i + 1]
        ys.append(lay.forward(G.to_dev_x(sub)))
        ids.append(lay.forward_ids(1).clone())  # stream-ordered: this call's selection
    torch.cuda.synchronize()
    for i in range(n):
        sub = dict(inp)
        sub["x"] = xs[i:i + 1]
        y_ref, _ = G.reference_y(sub, ids[i].cpu().numpy(), f"decode call {i}")
        G.check_y(G.y_to_f64(ys[i]), y_ref, f"decode call {i}")


def test_decode_graph_replay(torch, full_layer):
    """Single-token calls captured in a HIP graph: every replay equals the eager results bit for bit."""
    inp = G.inputs("decode", 1, seed=0)
    lay = _layer_for(inp, full_layer)
    n = 8
    xs = G.to_dev_x({"x": synth._draw_bf16(400, "x", (n, 2048), 1.0)})
    eager = torch.stack([lay.forward(xs[i:i + 1])[0] for i in range(n)])
    ys = torch.empty((n, 2048), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):
            lay.forward(xs[i:i + 1], y=ys[i:i + 1])
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            lay.forward(xs[i:i + 1], y=ys[i:i + 1])
    for rep in range(3):
        ys.zero_()
        g.replay()
        torch.cuda.synchronize()
        _ = (xs.float() * 2).sum().item()  # eager work between replays
        assert torch.equal(ys.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


# ------------------------------------------------------- padded boundaries
@pytest.mark.parametrize("E,k,T", BOUNDARY_CASES)
def test_padded_tile_boundaries(torch, E, k, T):
    """Crafted loads at the tile edges, one tile class (the default tiling)."""
    run_boundary_case(E, k, T)


@pytest.mark.parametrize("big,small", [(64, 32), (128, 64), (256, 256), (256, 64)])
def test_padded_tile_boundaries_other_tilings(torch, big, small):
    """The same cases under another tiling, in a child process (the tiling is read once per process):
    BIG and SMALL tile lists, and the persistent 256-row kernel alone and beside 64-row remainder tiles."""
    import subprocess
    env = dict(os.environ, MOE_TILE_ROWS=str(big), MOE_SMALL_ROWS=str(small))
    G.say(f"[boundaries] child process with MOE_TILE_ROWS={big} MOE_SMALL_ROWS={small}")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-m", "tests.boundary_case"], cwd=root, env=env, capture_output=True,
                       text=True, timeout=240)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0
    assert r.stdout.count("ok ") == len(BOUNDARY_CASES) and f"BIG={big} SMALL={small}" in r.stdout


# ------------------------------------------------------------ determinism
def test_determinism_and_graph_replay(torch, full_layer):
    """Two eager runs and HIP-graph replays give bitwise-identical y (no atomics in the path)."""
    inp = G.inputs("prefill8k", 2048)
    lay = _layer_for(inp, full_layer)
    x = G.to_dev_x(inp)
    y1 = lay.forward(x).clone()
    y2 = lay.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    yg = torch.empty_like(y1)
    lay.workspace(x.shape[0])
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
        _ = (x.float() * 2).sum().item()  # eager work between replays
        assert torch.equal(yg.view(torch.int16), y1.view(torch.int16)), f"replay {i}"


def test_zero_tokens_is_noop(torch):
    inp = synth.make_inputs("tiny", seed=0)
    lay = DeviceLayer.from_inputs(inp)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    y = lay.forward(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)
