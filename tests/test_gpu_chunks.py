"""GPU parity of prefill through fixed-size buckets (moe_prefill_runner_*).

guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B" (data-path and runtime
sections): any prompt is covered by resident buckets, only the final segment
padded.  Every token's output must be the layer's output on that token, so
the oracle is the layer oracle on the whole prompt; lengths just off a
bucket multiple exercise the padded last segment.
"""
import numpy as np
import pytest

import oracle
from sparse_moe_layer_03_amd import moe, synth
from sparse_moe_layer_03_amd.layer import DeviceLayer, PrefillRunner
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return G.torch_cuda()


SMALL_WL = synth.Workload("chunks", T=0, H=512, E=16, k=4, I=256, I_s=128, bias="normal")
SMALL_BUCKETS = (40, 64, 128)  # 40 runs the tiled path, every bucket > the small-batch limit
SMALL_T = [1, 5, 39, 40, 41, 63, 64, 65, 104, 127, 128, 129, 300, 1000]


@pytest.fixture(scope="module")
def small(torch):
    inp = synth.make_inputs(SMALL_WL, seed=5, T=1000)
    lay = DeviceLayer.from_inputs(inp)
    run = PrefillRunner(lay, SMALL_BUCKETS)
    r = oracle.forward(inp)
    yield inp, lay, run, r
    run.close()


@pytest.mark.parametrize("T", SMALL_T)
def test_runner_small_buckets(torch, small, T):
    """Runner output for the first T tokens == oracle (the layer on each token); ids from moe_forward."""
    inp, lay, run, r = small
    segs = run.plan(T)
    G.say(f"[chunks] T={T} segments={segs[0]} lens={segs[1]}")
    x = G.to_dev_x(inp)[:T].contiguous()
    y = run.run(x)
    y_full = lay.forward(x)  # one call over all T tokens
    ids = lay.forward_ids(T).cpu().numpy()
    torch.cuda.synchronize()
    sub = dict(inp)
    sub["x"] = inp["x"][:T]
    y_ref, _ = G.reference_y(sub, ids, f"chunks T={T}")
    G.check_y(G.y_to_f64(y), y_ref, f"runner T={T}")
    G.check_y(G.y_to_f64(y_full), y_ref, f"moe_forward T={T}")


def test_runner_repeat_and_other_stream(torch, small):
    """Repeated runs, and a run on a side stream, are bitwise identical; the output buffer is fully written."""
    inp, lay, run, r = small
    x = G.to_dev_x(inp)[:300].contiguous()
    y1 = run.run(x).clone()
    y2 = torch.full_like(y1, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.run(x, y=y2)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("T", [10000, 16380])
def test_runner_page_buckets_full_shape(torch, T):
    """Full shapes with the 1024/2048/4096/8192 buckets at lengths off a bucket multiple: sampled tokens
    (every segment, both ends of the padded last one) against the oracle; the whole output against one
    moe_forward call over all T tokens."""
    inp = G.inputs("prefill8k", T)
    lay = DeviceLayer.from_inputs(inp)
    run = PrefillRunner(lay)
    segs, lens = run.plan(T)
    G.say(f"[chunks-full] T={T} segments={segs} lens={lens}")
    x = G.to_dev_x(inp)
    y = run.run(x)
    y_full = lay.forward(x)
    ids = lay.forward_ids(T).cpu().numpy()
    torch.cuda.synchronize()
    starts = np.cumsum([0] + lens[:-1])
    rows = sorted(set(int(v) for s0, l in zip(starts, lens) for v in (s0, s0 + 1, s0 + l // 2, s0 + l - 2, s0 + l - 1)))
    sub = dict(inp)
    sub["x"] = inp["x"][rows]
    y_ref, _ = G.reference_y(sub, ids[rows], f"chunks full T={T}")
    G.check_y(G.y_to_f64(y)[rows], y_ref, f"runner full T={T} (sampled)")
    G.check_y(G.y_to_f64(y), G.y_to_f64(y_full), f"runner vs moe_forward T={T}")
    run.close()


@pytest.mark.parametrize("T", [1, 7, 8, 9, 31, 57])
def test_runner_small_batch_buckets(torch, T):
    """Buckets of 8, 16 and 32 tokens: the captured graphs run the small-batch kernels."""
    wl = synth.Workload("chunks-sb", T=64, H=512, E=16, k=4, I=256, I_s=128, bias="normal")
    inp = synth.make_inputs(wl, seed=6)
    lay = DeviceLayer.from_inputs(inp)
    run = PrefillRunner(lay, (8, 16, 32))
    segs, lens = run.plan(T)
    G.say(f"[chunks-sb] T={T} segments={segs} lens={lens}")
    x = G.to_dev_x(inp)[:T].contiguous()
    y = run.run(x)
    torch.cuda.synchronize()
    # every token, under the selection the runner's segment call made (near-ties admissible)
    y_seg = G.runner_reference(lay, run, x, inp, T, f"runner small buckets T={T}")
    assert torch.equal(y.view(torch.int16), y_seg.view(torch.int16)), "runner differs from its segment calls"
    run.close()


@pytest.mark.parametrize("T", [1, 39, 41, 129, 300])
def test_runner_fp8_small_buckets(torch, T):
    """A runner over FP8 expert weights (graphs of moe_forward_fp8) against the oracle on the same codes."""
    inp = G.with_fp8(synth.make_inputs(SMALL_WL, seed=7, T=300))
    lay = DeviceLayer.from_inputs(inp, fp8=True)
    run = PrefillRunner(lay, SMALL_BUCKETS)
    segs, lens = run.plan(T)
    G.say(f"[chunks-fp8] T={T} segments={segs} lens={lens}")
    x = G.to_dev_x(inp)[:T].contiguous()
    y = run.run(x)
    y_full = lay.forward(x)
    ids = lay.forward_ids(T).cpu().numpy()
    torch.cuda.synchronize()
    sub = dict(inp)
    sub["x"] = inp["x"][:T]
    y_ref, _ = G.reference_y(sub, ids, f"chunks fp8 T={T}", fp8=True)
    G.check_y(G.y_to_f64(y), y_ref, f"fp8 runner T={T}")
    G.check_y(G.y_to_f64(y_full), y_ref, f"moe_forward_fp8 T={T}")
    run.close()


def test_runner_fp8_page_buckets_full_shape(torch):
    """FP8 weights at full shape, 10000 tokens (8192 + a padded 2048): sampled tokens against the oracle,
    the whole output against one moe_forward_fp8 call."""
    T = 10000
    inp = G.with_fp8(G.inputs("prefill8k", T))
    lay = DeviceLayer.from_inputs(inp, fp8=True)
    run = PrefillRunner(lay)
    segs, lens = run.plan(T)
    G.say(f"[chunks-fp8-full] T={T} segments={segs} lens={lens}")
    x = G.to_dev_x(inp)
    y = run.run(x)
    y_full = lay.forward(x)
    ids = lay.forward_ids(T).cpu().numpy()
    torch.cuda.synchronize()
    starts = np.cumsum([0] + lens[:-1])
    rows = sorted(set(int(v) for s0, l in zip(starts, lens) for v in (s0, s0 + l // 2, s0 + l - 1)))
    sub = dict(inp)
    sub["x"] = inp["x"][rows]
    y_ref, _ = G.reference_y(sub, ids[rows], f"chunks fp8 full T={T}", fp8=True)
    G.check_y(G.y_to_f64(y)[rows], y_ref, f"fp8 runner full T={T} (sampled)")
    G.check_y(G.y_to_f64(y), G.y_to_f64(y_full), f"fp8 runner vs moe_forward_fp8 T={T}")
    run.close()


@pytest.mark.parametrize("T", [7, 57])
def test_runner_fp8_small_batch_buckets(torch, T):
    """FP8 weights with 8/16/32-token buckets: the graphs run the FP8 small-batch kernels."""
    wl = synth.Workload("chunks-sb", T=64, H=512, E=16, k=4, I=256, I_s=128, bias="normal")
    inp = G.with_fp8(synth.make_inputs(wl, seed=8))
    lay = DeviceLayer.from_inputs(inp, fp8=True)
    run = PrefillRunner(lay, (8, 16, 32))
    segs, lens = run.plan(T)
    G.say(f"[chunks-sb-fp8] T={T} segments={segs} lens={lens}")
    x = G.to_dev_x(inp)[:T].contiguous()
    y = run.run(x)
    torch.cuda.synchronize()
    y_seg = G.runner_reference(lay, run, x, inp, T, f"fp8 runner small buckets T={T}", fp8=True)
    assert torch.equal(y.view(torch.int16), y_seg.view(torch.int16)), "runner differs from its segment calls"
    run.close()


def test_runner_rejects_4bit_layer(torch):
    """4-bit weights serve T <= 32 only: the runner refuses such a layer instead of using other weights."""
    inp = synth.add_q4_weights(synth.make_inputs(SMALL_WL, seed=9, T=8))
    lay = DeviceLayer.from_inputs(inp, q4=True)
    with pytest.raises(ValueError):
        PrefillRunner(lay, SMALL_BUCKETS)
