"""The seeded input generator: determinism, bf16 rounding, workload structure."""
import numpy as np

from sparse_moe_layer_03_amd import synth


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 3.140625], np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(vals))
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6); 1+2^-9 rounds down
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0, 3.140625]


def test_blockwise_draws():
    n = synth.BLOCK * 2 + 37
    a = synth._draw_bf16(5, "w_up", (n,), 0.02)
    for b in range(3):
        m = min(synth.BLOCK, n - b * synth.BLOCK)
        ref = synth.f32_to_bf16_bits(np.random.default_rng([5, synth.TENSOR_IDS["w_up"], b])
                                     .standard_normal(m, dtype=np.float32) * np.float32(0.02))
        assert np.array_equal(a[b * synth.BLOCK:b * synth.BLOCK + m], ref)


def test_weights_do_not_depend_on_T():
    a = synth.make_inputs(synth.workload("prefill1k", T=3, E=4), seed=0)
    b = synth.make_inputs(synth.workload("prefill1k", T=9, E=4), seed=0)
    assert np.array_equal(a["w_down"], b["w_down"]) and np.array_equal(a["x"], b["x"][:3])


def test_deterministic_and_seeded():
    a = synth.make_inputs("tiny", seed=0)
    b = synth.make_inputs("tiny", seed=0)
    c = synth.make_inputs("tiny", seed=1)
    assert synth.content_hash(a) == synth.content_hash(b) != synth.content_hash(c)
    assert a["x"].dtype == np.uint16 and a["x"].shape == (16, 256)
    assert a["w_down"].shape == (8, 256, 128) and a["ws_gate"] is None


def test_weight_scale():
    a = synth.make_inputs(synth.workload("prefill1k", T=4, E=8), seed=0)
    sd = synth.bf16_bits_to_f32(a["w_gate"]).std()
    assert abs(sd - 0.02) < 0.0005
    assert abs(synth.bf16_bits_to_f32(a["x"]).std() - 1.0) < 0.05


def test_zipf_bias_and_ties():
    wl = synth.workload("skew32k", T=500, E=64)
    inp = synth.make_inputs(wl, seed=0)
    rows = inp["tie_rows"]
    assert len(rows) == 5 and np.all(inp["x"][rows] == 0)
    b = inp["bias"].astype(np.float64)
    order = np.lexsort((np.arange(64), -b))
    assert b[order[wl.k]] == b[order[wl.k - 1]] and b[order[2]] == b[order[1]]
    # log-pmf: exp(b) sums to ~1 apart from the two edited entries
    assert 0.9 < np.exp(b).sum() < 1.2


def test_logit_ties():
    lg = synth.make_logits(200, 256, seed=0, tie_frac=0.05)
    assert lg.dtype == np.float32 and lg.shape == (200, 256)
    assert np.any(np.signbit(lg) & (lg == 0))
