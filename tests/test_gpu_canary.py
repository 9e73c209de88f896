"""Guard bytes around every workspace section and around y (out-of-bounds writes).

The workspace is carved into sections, each followed by at least 256 bytes that no kernel writes
(moe_workspace_sections lists them).  The workspace and y are placed inside larger buffers filled with
a pattern; after the call, every gap between sections, the bytes before and after the workspace and
the rows before and after y must still hold it.  Single-token, small-batch and tiled paths (64- and
256-row tiles), BF16 and FP8 weights, and the bucketed prefill runner (its output rows and its
input).
"""
import numpy as np
import pytest

from sparse_moe_layer_03_amd import moe
from sparse_moe_layer_03_amd.layer import DeviceLayer, PrefillRunner
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

PAT = 0xA5
GUARD = 4096  # bytes before and after the workspace (a multiple of 256: the workspace stays aligned)
YG = 2        # guard rows before and after y


@pytest.fixture(scope="module")
def torch():
    return G.torch_cuda()


@pytest.fixture(scope="module")
def layers(torch):
    return {"bf16": DeviceLayer(G.full_weights(0), k=8), "fp8": DeviceLayer(G.full_fp8_weights(0), k=8, fp8=True)}


def _check_gaps(buf, need, sections, label):
    b = buf.cpu().numpy()
    assert np.all(b[:GUARD] == PAT), f"{label}: bytes before the workspace were written"
    assert np.all(b[GUARD + need:] == PAT), f"{label}: bytes after the workspace were written"
    ws = b[GUARD:GUARD + need]
    ends = [o for o, _ in sections[1:]] + [need]
    for i, ((off, nb), end) in enumerate(zip(sections, ends)):
        assert end - (off + nb) >= 256, f"{label}: section {i} has no guard gap"
        gap = ws[off + nb:end]
        assert np.all(gap == PAT), f"{label}: guard after section {i} (offset {off}, {nb} bytes) was written"


CASES = [(1, "bf16"), (16, "bf16"), (2048, "bf16"), (8192, "bf16"), (8192, "fp8"), (1, "fp8")]


@pytest.mark.parametrize("T,fmt", CASES, ids=[f"T{t}-{f}" for t, f in CASES])
def test_guards(torch, layers, T, fmt):
    lay = layers[fmt]
    inp = G.inputs("prefill8k", T)
    lay.bias = torch.from_numpy(inp["bias"]).to("cuda:0")
    s = lay.shapes
    need = moe.moe_workspace_size(T, s.H, s.E, s.k, s.I, s.I_s)
    sections = moe.moe_workspace_sections(T, s.H, s.E, s.k, s.I, s.I_s)
    G.say(f"[canary] T={T} {fmt}: {len(sections)} sections, {need} bytes")
    buf = torch.full((GUARD + need + GUARD,), PAT, dtype=torch.uint8, device="cuda")
    ws = buf[GUARD:GUARD + need]
    ybuf = torch.empty((T + 2 * YG, s.H), dtype=torch.bfloat16, device="cuda")
    ybuf.view(torch.uint8).fill_(PAT)
    y = ybuf[YG:YG + T]
    x = G.to_dev_x(inp)
    lay._ws, lay._ws_bytes = ws, need
    try:
        lay.forward(x, y)
        torch.cuda.synchronize()
    finally:
        lay._ws, lay._ws_bytes = None, 0
    _check_gaps(buf, need, sections, f"T={T} {fmt}")
    yb = ybuf.view(torch.uint8).cpu().numpy()
    assert np.all(yb[:YG] == PAT) and np.all(yb[YG + T:] == PAT), "rows around y were written"
    # and the result is the layer's: the same call on a fresh workspace gives the same bits
    y2 = lay.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_runner_guards(torch, layers):
    """The bucketed runner writes only its output rows and leaves its input untouched."""
    lay = layers["bf16"]
    T = 5000  # 4096 + a padded 1024-token segment
    inp = G.inputs("prefill8k", T)
    lay.bias = torch.from_numpy(inp["bias"]).to("cuda:0")
    run = PrefillRunner(lay)
    try:
        x = G.to_dev_x(inp)
        x0 = x.clone()
        ybuf = torch.empty((T + 2 * YG, lay.shapes.H), dtype=torch.bfloat16, device="cuda")
        ybuf.view(torch.uint8).fill_(PAT)
        run.run(x, y=ybuf[YG:YG + T])
        torch.cuda.synchronize()
        yb = ybuf.view(torch.uint8).cpu().numpy()
        assert np.all(yb[:YG] == PAT) and np.all(yb[YG + T:] == PAT), "rows around the runner's output were written"
        assert torch.equal(x.view(torch.int16), x0.view(torch.int16)), "the runner changed its input"
    finally:
        run.close()
