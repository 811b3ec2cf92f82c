"""The output head (dit_final_layer) on the GPU against the oracle.

Bar: the head computes in fp32 from exactly representable inputs, as the fp32
block does, so max-abs and rel-L2 1e-4 against the fp64 oracle (output values
are O(1)). Row ranges: a row's bits do not depend on the range it is computed
in. Full size: 32 768 tokens x 5120 (the large block's width) to 64 outputs,
512 sampled rows checked against the oracle."""
import numpy as np
import pytest
import torch

from memory_bounded_chunked_amd import block as B
from memory_bounded_chunked_amd import synth
from oracle import dit_block as O

from _helpers import max_abs, rel_l2

pytestmark = pytest.mark.gpu


def _device(inp):
    return {k: B.tensor_from_stored(v, "cuda") for k, v in inp.items()}


def _oracle(inp, rows=None, eps=1e-6):
    x = synth.to_f64(inp["x"] if rows is None else inp["x"][rows])
    return O.final_layer(x, synth.to_f64(inp["shift"]), synth.to_f64(inp["scale"]), synth.to_f64(inp["w_out"]), eps)


CASES = [
    # (n, d, out_dim, act)
    (1, 64, 1, "bf16"),
    (31, 64, 17, "f32"),
    (33, 256, 32, "bf16"),
    (300, 256, 64, "bf16"),
    (300, 256, 64, "f32"),
    (77, 512, 100, "bf16"),
    (129, 1024, 128, "f32"),
    (200, 3072, 64, "bf16"),
    (65, 5120, 64, "bf16"),
    (40, 8192, 48, "bf16"),
]


@pytest.mark.parametrize("n,d,out_dim,act", CASES)
def test_final_layer_matches_oracle(n, d, out_dim, act):
    print(f"final_layer n={n} d={d} out_dim={out_dim} act={act}", flush=True)
    inp = synth.make_final_inputs(n, d, out_dim, act, seed=n + d)
    t = _device(inp)
    out = B.final_layer(t["x"], t["shift"], t["scale"], t["w_out"])
    torch.cuda.synchronize()
    ref = _oracle(inp)
    got = out.cpu().numpy().astype(np.float64)
    assert max_abs(got, ref) <= 1e-4
    assert rel_l2(got, ref) <= 1e-4


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_final_layer_row_ranges_bit_identical(act):
    n, d, out_dim = 300, 512, 64
    inp = synth.make_final_inputs(n, d, out_dim, act, seed=5)
    t = _device(inp)
    full = B.final_layer(t["x"], t["shift"], t["scale"], t["w_out"])
    parts = torch.empty_like(full)
    for r0, r1 in ((0, 1), (1, 37), (37, 100), (100, 257), (257, 300)):
        B.final_layer(t["x"][r0:r1], t["shift"], t["scale"], t["w_out"], out=parts[r0:r1])
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int32), parts.view(torch.int32))


def test_final_layer_strided_rows_and_output():
    n, d, out_dim = 97, 256, 40
    inp = synth.make_final_inputs(n, d, out_dim, "bf16", seed=9)
    t = _device(inp)
    xw = torch.zeros((n, d + 24), dtype=torch.bfloat16, device="cuda")
    xw[:, :d] = t["x"]
    ow = torch.full((n, 56), 7.0, dtype=torch.float32, device="cuda")
    B.final_layer(xw[:, :d], t["shift"], t["scale"], t["w_out"], out=ow[:, :out_dim])
    dense = B.final_layer(t["x"], t["shift"], t["scale"], t["w_out"])
    torch.cuda.synchronize()
    assert torch.equal(ow[:, :out_dim], dense)
    assert torch.all(ow[:, out_dim:] == 7.0)  # padding columns untouched
    ref = _oracle(inp)
    assert max_abs(dense.cpu().numpy().astype(np.float64), ref) <= 1e-4


def test_final_layer_empty_is_noop():
    d, out_dim = 128, 32
    inp = synth.make_final_inputs(4, d, out_dim, "bf16", seed=1)
    t = _device(inp)
    out = torch.full((4, out_dim), 3.0, device="cuda")
    B.final_layer(t["x"][:0], t["shift"], t["scale"], t["w_out"], out=out[:0])
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_final_layer_constant_rows():
    # A constant row has zero variance: LN gives 0, so the output is shift . w_j.
    n, d, out_dim = 40, 256, 64
    inp = synth.make_final_inputs(n, d, out_dim, "f32", seed=3)
    inp["x"][:] = np.float32(2.5)
    t = _device(inp)
    out = B.final_layer(t["x"], t["shift"], t["scale"], t["w_out"]).cpu().numpy().astype(np.float64)
    expect = synth.to_f64(inp["w_out"]) @ synth.to_f64(inp["shift"])
    assert max_abs(out, np.broadcast_to(expect, out.shape)) <= 1e-5


def test_final_layer_rows_far_from_zero_mean():
    # The kernel takes the moments of x - p for a per-row shift p (the mean of
    # the row's first 8 values): rows centred far from zero, some with an
    # outlier among those first values, must still match the oracle.
    n, d, out_dim = 96, 1024, 64
    inp = synth.make_final_inputs(n, d, out_dim, "f32", seed=4)
    x = inp["x"].astype(np.float64)
    x = 1000.0 + x
    x[::3, 0] += 50.0
    x[1::3, :8] -= 20.0
    inp["x"] = x.astype(np.float32)
    t = _device(inp)
    got = B.final_layer(t["x"], t["shift"], t["scale"], t["w_out"]).cpu().numpy().astype(np.float64)
    ref = _oracle(inp)
    assert max_abs(got, ref) <= 1e-4 * max(1.0, float(np.abs(ref).max()))
    assert rel_l2(got, ref) <= 1e-4


def test_final_layer_full_size_sampled_rows():
    n, d, out_dim = 32768, 5120, 64
    print(f"final_layer full n={n} d={d} out_dim={out_dim}", flush=True)
    inp = synth.make_final_inputs(n, d, out_dim, "bf16", seed=0)
    t = _device(inp)
    out = B.final_layer(t["x"], t["shift"], t["scale"], t["w_out"])
    torch.cuda.synchronize()
    rows = synth.sample_rows(n, 512)
    got = out.cpu().numpy()[rows].astype(np.float64)
    ref = _oracle(inp, rows)
    assert max_abs(got, ref) <= 1e-4
    assert rel_l2(got, ref) <= 1e-4
    assert torch.isfinite(out).all()
