"""Seeded input generator: determinism, bf16 rounding, realized sparsity (no GPU)."""
import numpy as np
import pytest

import oracle
from activation_sparse_feed_gate_amd import synth


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9,
                  -2.5, 0.0, -0.0, 2.0 ** 100, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(f))
    # bf16 keeps 8 significant bits: 1 + 2^-8 is a tie -> even (1.0);
    # 1 + 3*2^-8 is a tie -> even (1 + 2^-6); just above a tie rounds up
    want = np.array([1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5, 0.0, -0.0,
                     2.0 ** 100, 1.0 + 2.0 ** -7], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_deterministic_and_bias_column():
    w = synth.WORKLOADS["tiny"]
    a, b = synth.make_inputs(w), synth.make_inputs(w)
    for k in ("x", "wg_t", "wu_t", "wd"):
        assert np.array_equal(a[k], b[k])
    assert np.all(synth.bf16_bits_to_f32(a["x"][:, -1]) == 1.0)
    assert np.all(synth.bf16_bits_to_f32(a["wg_t"][:, -1]) == -a["bias"])
    assert a["x"].shape == (w.M, w.K) and a["wd"].shape == (w.N, w.K)
    c = synth.make_inputs(w.with_(seed=1))
    assert not np.array_equal(a["x"], c["x"])


@pytest.mark.parametrize("name", ["tiny", "ffn-0.5b", "ffn-1b", "ffn-2b", "ffn-ovf", "ffn-paper"])
def test_realized_density(name):
    """Mean active fraction within 5% of the target over all rows (float32
    products are enough for a count); heavy-tailed workloads have rows more
    than ten times above the mean."""
    w = synth.WORKLOADS[name]
    d = synth.make_inputs(w)
    z = synth.bf16_bits_to_f32(d["x"]) @ synth.bf16_bits_to_f32(d["wg_t"]).T
    per_row = (z > 0).mean(axis=1)
    dens = per_row.mean()
    assert abs(dens - w.density) <= 0.05 * w.density, (dens, w.density)
    if w.sigma_s > 0:
        assert per_row.max() >= 10 * dens


def test_exact_density_extremes():
    w = synth.WORKLOADS["tiny"]
    for dens, want in ((0.0, 0.0), (1.0, 1.0)):
        d = synth.make_inputs(w.with_(density=dens))
        z = oracle.default().gate(d["x"], d["wg_t"])
        assert (z > 0).mean() == want
