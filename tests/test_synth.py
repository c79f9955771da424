"""Synthetic input generation: determinism, rounding and shapes."""
import numpy as np

from gated_linear_attention_fwd_amd import synth


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1).
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -8 + 2.0 ** -20],
                 np.float32)
    back = synth.bf16_value(synth.bf16_bits(x))
    assert back[0] == 1.0
    assert back[1] == 1.0
    assert back[2] == np.float32(1.0 + 2 * 2.0 ** -7)
    assert back[3] == -2.5
    assert back[4] == np.float32(1.0 + 2.0 ** -7)


def test_bf16_round_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    mine = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_chunked_draws_equal_single_draw():
    a = synth._draw(np.random.default_rng(5), (3, 1000), 0.5, "bf16", chunk=333)
    b = synth._draw(np.random.default_rng(5), (3, 1000), 0.5, "bf16", chunk=1 << 24)
    assert np.array_equal(a, b)


def test_workload_shapes_and_determinism():
    w = synth.WORKLOADS[2]
    x = synth.workload_inputs(w)
    y = synth.workload_inputs(w)
    for n in "qkvg":
        assert x[n].shape == (w.B, w.H, w.N, w.d) and x[n].dtype == np.uint16
        assert np.array_equal(x[n], y[n])
    assert x["gamma"].shape == (w.B, w.H, w.F) and x["gamma"].dtype == np.float32
    assert np.all((x["gamma"] > 0) & (x["gamma"] < 1))


def test_latent_shapes():
    assert synth.WORKLOADS[4].N == 221720 and synth.WORKLOADS[3].N == 19320
    w5 = synth.WORKLOADS[5]
    assert sum(w5.blocks) == w5.F == 241 and len(w5.blocks) == 8
    assert synth.WORKLOADS[4].io_bytes() == 4_540_825_600


def test_stream_blocks_cover_gamma():
    w = synth.WORKLOADS[5]
    ga = synth.stream_gamma(w)
    bounds = synth.stream_block_bounds(w)
    assert bounds[-1] == (210, 31)
    small = synth.Workload("t", 1, 1, 16, 5, 3, "bf16", 9, 2.0, 1.0, True, ("framecausal",),
                           blocks=(2, 3))
    g = synth.stream_gamma(small)
    b1 = synth.stream_block_inputs(small, 1, g)
    assert b1["q"].shape == (1, 1, 9, 16) and np.array_equal(b1["gamma"], g[:, :, 2:5])
    assert ga.shape == (2, 40, 241)
