"""Where the bars of the GPU parity tests come from (CPU): an emulation of the
GPU path's own rounding points, on the same seeded inputs and rows as the GPU
test that uses the bar.

The GPU path rounds to bf16 (nearest even) at n1, Q, K, V, P (the softmax row
sum is taken from the rounded P), O, n2, h and y; everything else is fp32. The
emulation shows how far from the exact block output (the oracle) those
roundings alone put y and O, before any fp32 accumulation order comes in.

Two forms: ``emulate`` takes fp64 between the rounding points and serves the
small blocks; ``emulate_rows`` takes fp32 between them (as the GPU does; torch
CPU, so the full-size workloads take tens of seconds) and serves the sampled
rows of the full-size tests: norm1, K and V for all N tokens, then every later
step for the sampled rows only (each is per token). int8 weights enter both
exactly, with the per-row scale on the product (the GPU's order).
"""
import time

import numpy as np
import pytest
import torch

import oracle.dit_block as O
from _helpers import (BAR_LADDER, BF16_OVER_FRACTION, INT8_ADAPTER_SHAPES, INT8_BARS, half_ulp_bf16, oracle_inputs,
                      rel_l2)
from memory_bounded_chunked_amd import synth

R = lambda a: synth.bf16_bits_to_f64(synth.f64_to_bf16_bits(a))  # noqa: E731


def _proj(a, w, lora, name):
    y = a @ w.T
    if lora and name in lora:
        a_m, b_m, alpha = lora[name]
        y = y + (alpha * (a @ a_m.T)) @ b_m.T  # t = alpha (A a) is not rounded
    return y


def emulate(x, mod, w, n_heads, lora=None, eps=1e-6):
    d = x.shape[1]
    f = w["down"].shape[1]
    dh = d // n_heads
    n1 = R(O.modulate(O.layer_norm(x, eps), mod[0], mod[1]))
    q = R(_proj(n1, w["qkv"][:d], lora, "q"))
    k = R(_proj(n1, w["qkv"][d:2 * d], lora, "k"))
    v = R(_proj(n1, w["qkv"][2 * d:], lora, "v"))
    o = np.empty_like(q)
    for h in range(n_heads):
        c = slice(h * dh, (h + 1) * dh)
        s = q[:, c] @ k[:, c].T / np.sqrt(dh)
        p = R(np.exp(s - s.max(1, keepdims=True)))
        o[:, c] = (p @ v[:, c]) / p.sum(1, keepdims=True)
    o = R(o)
    x1 = x + mod[2] * _proj(o, w["o"], lora, "o")
    n2 = R(O.modulate(O.layer_norm(x1, eps), mod[3], mod[4]))
    h_ = R(O.silu(_proj(n2, w["gu"][:f], lora, "gate")) * _proj(n2, w["gu"][f:], lora, "up"))
    return R(x1 + mod[5] * _proj(h_, w["down"], lora, "down"))


def test_emulation_reduces_to_the_oracle_without_rounding():
    global R
    shape = synth.BlockShape("emul-check", 64, 2, 32, 128, 20, "bf16")
    inputs = synth.make_inputs(shape, seed=0)
    x, mod, w = oracle_inputs(inputs)
    saved, R = R, (lambda a: a)
    try:
        y = emulate(x, mod, w, shape.n_heads)
    finally:
        R = saved
    assert rel_l2(y, O.block_forward(x, mod, w, shape.n_heads)) < 1e-12


def test_single_gate_adapter_bar():
    # The 64-token bf16 block with one alpha = 2 gate adapter (the GPU test of
    # each single adapter): the rounding points alone put the worst element
    # more than 2e-2 beyond its half-ulp, so that test holds y to 3e-2 beyond it.
    shape = synth.BlockShape("single-bf16", 256, 2, 128, 512, 64, "bf16")
    inputs = synth.make_inputs(shape, seed=0)
    x, mod, w = oracle_inputs(inputs)
    lora = synth.make_lora(shape, 32, seed=1, targets=("gate",), alpha=2.0)
    lf = {k: (synth.to_f64(a), synth.to_f64(b), al) for k, (a, b, al) in lora.items()}
    y_ref = O.block_forward(x, mod, w, shape.n_heads, lora=O.lora_f64(lf))
    y = emulate(x, mod, w, shape.n_heads, lora=lf)
    worst = float((np.abs(y - y_ref) - half_ulp_bf16(y_ref)).max())
    assert 2e-2 < worst < 3e-2, worst
    assert rel_l2(y, y_ref) < 1e-2


# ---------------------------------------------------------------- sampled rows at full size

def _t32(arr: np.ndarray) -> torch.Tensor:
    """A stored array (bf16 bits, fp32, int8) as an fp32 CPU tensor (exact)."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).float()
    return torch.from_numpy(np.ascontiguousarray(arr)).float()


ROUND = True  # False: the same arithmetic without the bf16 rounding points


def _r(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16).float() if ROUND else t


def _modnorm32(x, shift, scale, eps):
    mu = x.mean(1, keepdim=True)
    xc = x - mu
    var = (xc * xc).mean(1, keepdim=True)
    return _r(xc * torch.rsqrt(var + eps) * (1 + scale) + shift)


def emulate_rows(inputs: dict, shape, rows: np.ndarray, eps: float = 1e-6, lora: dict | None = None):
    """(y, O) of the sampled ``rows`` through the GPU path's rounding points, fp32 between them.
    ``lora``: {target: (A, B, alpha)} stored adapters; t = alpha (A a) stays unrounded and
    B t joins the projection's sum (after the per-row scale of int8 weights)."""
    d, f, heads = shape.d, shape.ffn, shape.n_heads
    dh = d // heads
    mod = torch.from_numpy(inputs["mod"])
    lo = {k: (_t32(a), _t32(b), al) for k, (a, b, al) in (lora or {}).items()}

    def weight(name, r0, r1, target=None):
        s = inputs.get("s_" + name)
        return _t32(inputs["w_" + name][r0:r1]), None if s is None else torch.from_numpy(s[r0:r1]), target

    def proj(a, w):
        y = a @ w[0].T
        y = y if w[1] is None else y * w[1]
        if w[2] in lo:
            a_m, b_m, alpha = lo[w[2]]
            y = y + (alpha * (a @ a_m.T)) @ b_m.T
        return y

    n = shape.n_tokens
    wk, wv = weight("qkv", d, 2 * d, "k"), weight("qkv", 2 * d, 3 * d, "v")
    kh = torch.empty(heads, n, dh)
    vh = torch.empty(heads, n, dh)
    for r0 in range(0, n, 8192):
        n1 = _modnorm32(_t32(inputs["x"][r0:r0 + 8192]), mod[0], mod[1], eps)
        kh[:, r0:r0 + 8192] = _r(proj(n1, wk)).view(-1, heads, dh).transpose(0, 1)
        vh[:, r0:r0 + 8192] = _r(proj(n1, wv)).view(-1, heads, dh).transpose(0, 1)
    del wk, wv
    xr = _t32(inputs["x"][rows])
    q = _r(proj(_modnorm32(xr, mod[0], mod[1], eps), weight("qkv", 0, d, "q"))).view(-1, heads, dh).transpose(0, 1)
    o = torch.empty(heads, len(rows), dh)
    for h in range(heads):
        s = (q[h] @ kh[h].T) / float(np.sqrt(dh))
        p = _r(torch.exp(s - s.amax(1, keepdim=True)))
        o[h] = (p @ vh[h]) / p.sum(1, keepdim=True)
    del kh, vh
    o = _r(o.transpose(0, 1).reshape(-1, d))
    x1 = xr + mod[2] * proj(o, weight("o", 0, d, "o"))
    n2 = _modnorm32(x1, mod[3], mod[4], eps)
    hh = _r(torch.nn.functional.silu(proj(n2, weight("gu", 0, f, "gate"))) * proj(n2, weight("gu", f, 2 * f, "up")))
    y = _r(x1 + mod[5] * proj(hh, weight("down", 0, d, "down")))
    return y.double().numpy(), o.double().numpy()


def _oracle_then_emulation(shape, rows):
    inputs = synth.make_inputs(shape, seed=0)
    x, mod, w = oracle_inputs(inputs)
    t0 = time.time()
    y_ref, o_ref = O.block_rows(x, mod, w, shape.n_heads, rows, eps=shape.eps, want=("o",))
    del x, w
    t1 = time.time()
    y, o = emulate_rows(inputs, shape, rows, shape.eps)
    print(f"\n{shape.name}: oracle {t1 - t0:.1f} s, emulation {time.time() - t1:.1f} s")
    return y, o, y_ref, o_ref


def test_row_emulation_reduces_to_the_oracle_without_rounding():
    global ROUND
    for shape in (synth.BlockShape("emul-rows", 256, 2, 128, 512, 300, "bf16"),
                  synth.BlockShape("emul-rows-w8", 256, 2, 128, 512, 300, "w8_bf16")):
        inputs = synth.make_inputs(shape, seed=0)
        x, mod, w = oracle_inputs(inputs)
        rows = synth.sample_rows(shape.n_tokens, 40)
        y_ref, o_ref = O.block_rows(x, mod, w, shape.n_heads, rows, want=("o",))
        ROUND = False
        try:
            y, o = emulate_rows(inputs, shape, rows)
        finally:
            ROUND = True
        assert rel_l2(y - x[rows], y_ref - x[rows]) < 1e-5
        assert rel_l2(o, o_ref) < 1e-5


def _bf16_floor(y, y_ref):
    err = np.abs(y - y_ref)
    return float(err.max()), float((err - half_ulp_bf16(y_ref)).max()), float((err > 2e-2).mean())


SMALL_BF16 = [synth.BlockShape("small-bf16", 256, 2, 128, 512, 777, "bf16"),
              synth.BlockShape("small-dh64", 256, 4, 64, 768, 450, "bf16"),
              synth.BlockShape("smoke", 256, 2, 128, 512, 300, "bf16")]


@pytest.mark.parametrize("shape", SMALL_BF16, ids=lambda s: s.name)
def test_bf16_bar_on_the_small_blocks(shape):
    # the whole-block GPU tests: the per-element excess over the half-ulp stays
    # within 3/4 of 2e-2 and the fraction above 2e-2 ten times under its allowance
    inputs = synth.make_inputs(shape, seed=0)
    x, mod, w = oracle_inputs(inputs)
    y_ref = O.block_forward(x, mod, w, shape.n_heads)
    y = emulate(x, mod, w, shape.n_heads)
    _, excess, frac = _bf16_floor(y, y_ref)
    assert excess <= 0.75 * 2e-2, excess
    assert 10 * frac <= BF16_OVER_FRACTION, frac
    assert rel_l2(y, y_ref) <= 0.25 * 1e-2


@pytest.mark.slow
def test_bf16_bar_at_the_32k_block():
    # 512 sampled rows of the 32768-token block (the GPU full-size test's rows):
    # the literal max-abs 2e-2 is out of reach of the rounding points alone
    # (0.025), while the excess over the bf16 output's half-ulp stays at 0.014
    # and the fraction above 2e-2 at about 3e-6; O within a fifth of 1e-2.
    shape = synth.CONFIGS["large"]
    rows = synth.sample_rows(shape.n_tokens, 512)
    y, o, y_ref, o_ref = _oracle_then_emulation(shape, rows)
    mx, excess, frac = _bf16_floor(y, y_ref)
    print(f"large emulated: max-abs {mx:.4g}, excess {excess:.4g}, over-2e-2 fraction {frac:.3g}, "
          f"rel-L2 y {rel_l2(y, y_ref):.4g}, O {rel_l2(o, o_ref):.4g}")
    assert mx > 2e-2
    assert excess <= 0.75 * 2e-2
    assert 10 * frac <= BF16_OVER_FRACTION
    assert rel_l2(y, y_ref) <= 0.25 * 1e-2
    assert rel_l2(o, o_ref) <= 1e-2 / 5


def _bar_for(floor: float) -> float:
    return min(b for b in BAR_LADDER if b >= 1.5 * floor)


def _int8_floors(y, o, y_ref, o_ref) -> dict:
    return {"y_rel": rel_l2(y, y_ref), "y_max_frac": float(np.abs(y - y_ref).max() / np.abs(y_ref).max()),
            "o_rel": rel_l2(o, o_ref)}


@pytest.mark.slow
def test_int8_bar_at_full_size():
    # 512 sampled rows of the 65536-token int8-weight block (the GPU full-size
    # test's rows). The rounding points alone give rel-L2 0.0195 on y and
    # 0.0149 on O (the GPU measures the same to three digits), above the 1e-2
    # of the bf16 blocks; each int8 bar is derived from its emulated floor.
    shape = synth.CONFIGS["int8"]
    rows = synth.sample_rows(shape.n_tokens, 512)
    y, o, y_ref, o_ref = _oracle_then_emulation(shape, rows)
    floors = _int8_floors(y, o, y_ref, o_ref)
    print("int8 emulated floors:", {k: round(v, 5) for k, v in floors.items()})
    assert 1e-2 < floors["y_rel"] < 2.5e-2
    for key, floor in floors.items():
        assert INT8_BARS[key] == _bar_for(floor), (key, floor)


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(INT8_ADAPTER_SHAPES))
def test_int8_adapter_bars(name):
    # the GPU test of int8 weights with adapters in the 256-wide weight tiles:
    # its bars are derived from the emulated floors at ranks 80 and 256, on
    # its own inputs (adapters from seed 3) and 512 sampled rows
    (d, heads, dh, ffn, n), bars = INT8_ADAPTER_SHAPES[name]
    shape = synth.BlockShape(name, d, heads, dh, ffn, n, "w8_bf16")
    inputs = synth.make_inputs(shape, seed=0)
    rows = synth.sample_rows(n, 512)
    x, mod, w = oracle_inputs(inputs)
    worst = {}
    for rank in (80, 256):
        lora = synth.make_lora(shape, rank, seed=3)
        lf = O.lora_f64({k: (synth.to_f64(a), synth.to_f64(b), al) for k, (a, b, al) in lora.items()})
        y_ref, o_ref = O.block_rows(x, mod, w, heads, rows, want=("o",), lora=lf)
        y, o = emulate_rows(inputs, shape, rows, lora=lora)
        for key, v in _int8_floors(y, o, y_ref, o_ref).items():
            worst[key] = max(worst.get(key, 0.0), v)
    print(f"\n{name} emulated floors:", {k: round(v, 5) for k, v in worst.items()})
    for key, bar in bars.items():
        assert bar == _bar_for(worst[key]), (key, worst[key])
