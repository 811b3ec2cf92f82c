"""Where a bf16 bar comes from (CPU): an fp64 emulation of the GPU path's own
rounding points, on the same seeded inputs as the GPU test that uses the bar.

The GPU path rounds to bf16 (nearest even) at n1, Q, K, V, P (the softmax row
sum is taken from the rounded P), O, n2, h and y; everything else is fp32 and
is emulated here exactly. The emulation shows how far from the exact block
output those roundings alone put y, before any fp32 accumulation order or
rounding decision taken on an fp32 value comes in.
"""
import numpy as np

import oracle.dit_block as O
from _helpers import half_ulp_bf16, oracle_inputs, rel_l2
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
