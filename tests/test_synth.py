"""The seeded input generator: determinism, rounding and value ranges (CPU only)."""
import numpy as np
import torch

from memory_bounded_chunked_amd import synth


def test_bf16_rounding_is_rne():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(100000).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(synth.f64_to_bf16_bits(v), ref.view(np.uint16))
    # exact ties go to the even significand: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)])
    back = synth.bf16_bits_to_f64(synth.f64_to_bf16_bits(ties))
    assert list(back) == [1.0, 1.0 + 2.0 ** -6, -1.0]
    # a value just above a tie rounds up (fp64 input, not pre-rounded to fp32)
    assert synth.bf16_bits_to_f64(synth.f64_to_bf16_bits(np.array([1 + 2.0 ** -8 + 2.0 ** -40])))[0] \
        == 1 + 2.0 ** -7


def test_deterministic_and_ranges():
    sh = synth.BlockShape("t", 64, 2, 32, 128, 300, "bf16")
    a, b = synth.make_inputs(sh, 0), synth.make_inputs(sh, 0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    c = synth.make_inputs(sh, 1)
    assert not np.array_equal(a["x"], c["x"])
    x = synth.to_f64(a["x"])
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    assert abs(a["mod"].std() - np.sqrt(0.1)) < 0.03
    w = synth.to_f64(a["w_gu"])
    assert abs(w.std() * np.sqrt(64) - 1) < 0.05
    # weights do not depend on whether x is returned
    nox = synth.make_inputs(sh, 0, with_x=False)
    assert "x" not in nox and np.array_equal(nox["w_down"], a["w_down"])


def test_int8_weights():
    sh = synth.BlockShape("t", 64, 2, 32, 128, 20, "w8_bf16")
    a = synth.make_inputs(sh, 0)
    for name, rows in (("qkv", 192), ("o", 64), ("gu", 256), ("down", 64)):
        q, s = a["w_" + name], a["s_" + name]
        assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
        assert s.dtype == np.float32 and s.shape == (rows,)
        assert s.min() >= 1e-4 and s.max() < 1e-3
    assert a["x"].dtype == np.uint16


def test_sample_rows():
    r = synth.sample_rows(32768)
    assert len(r) == 512 and len(set(r.tolist())) == 512 and np.all(np.diff(r) > 0)
    assert np.array_equal(r, synth.sample_rows(32768))
    assert len(synth.sample_rows(100)) == 100


def test_configs_and_flops():
    large = synth.CONFIGS["large"]
    assert (large.d, large.n_heads * large.head_dim, large.ffn, large.n_tokens) == (5120, 5120, 13824, 32768)
    assert abs(large.flops - 4.278e13) / 4.278e13 < 1e-3
    assert abs(synth.CONFIGS["tiny"].flops - 3.22e9) / 3.22e9 < 1e-2
