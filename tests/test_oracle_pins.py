"""Pins of the fp64 oracle to things other than itself (CPU only).

Each ``pin_*`` checks the oracle module passed in against an independent fact:
torch fp64 library routines (layer_norm, linear, silu, scaled_dot_product_
attention), brute-force attention written as plain Python loops on tiny inputs,
closed forms (zero gates, one token, constant rows, zero gate weights,
linearity in the gates), invariants (LayerNorm moments, permutation
equivariance) and the chunked schedule of "How the slicing works"
(LayerStream: H3 Chunking), which must reproduce the unchunked block.

``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle
(unbiased variance, a dropped eps, a transposed operand, a wrong softmax axis
or scale, swapped gates, a dropped residual, an in-place hazard, a per-column
int8 scale, ...) and requires at least one pin to fail for each.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as tF

import oracle.dit_block as O
from memory_bounded_chunked_amd import synth


def _case(d=32, heads=2, ffn=96, n=19, seed=0, dtype="bf16"):
    sh = synth.BlockShape("t", d, heads, d // heads, ffn, n, dtype)
    inp = synth.make_inputs(sh, seed)
    x = synth.to_f64(inp["x"])
    mod = inp["mod"].astype(np.float64)
    w = O.block_weights_f64({k: synth.to_f64(v) for k, v in inp.items() if k[:2] in ("w_", "s_")})
    return x, mod, w, heads


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def _order_stable(a, b):
    # Each output element is one pairwise sum whose order depends only on the
    # contracted length, never on how many rows are in the call.
    return (a[:, :, None] * b[None, :, :]).sum(axis=1)


def torch_block(x, mod, w, heads, eps=1e-6):
    """The block composed from torch fp64 library routines."""
    X = torch.from_numpy(x)
    n, d = X.shape
    ffn = w["down"].shape[1]
    sh1, sc1, g1, sh2, sc2, g2 = torch.from_numpy(np.asarray(mod, np.float64))
    n1 = tF.layer_norm(X, (d,), eps=eps) * (1 + sc1) + sh1
    q, k, v = tF.linear(n1, torch.from_numpy(w["qkv"])).split(d, dim=1)

    def hd(t):
        return t.reshape(n, heads, d // heads).transpose(0, 1).unsqueeze(0)

    o = tF.scaled_dot_product_attention(hd(q), hd(k), hd(v))
    o = o.squeeze(0).transpose(0, 1).reshape(n, d)
    x1 = X + g1 * tF.linear(o, torch.from_numpy(w["o"]))
    n2 = tF.layer_norm(x1, (d,), eps=eps) * (1 + sc2) + sh2
    g, u = tF.linear(n2, torch.from_numpy(w["gu"])).split(ffn, dim=1)
    y = x1 + g2 * tF.linear(tF.silu(g) * u, torch.from_numpy(w["down"]))
    return y.numpy()


def brute_attention(q, k, v, heads):
    """Softmax attention as plain Python loops over heads, queries and keys."""
    n_q, d = q.shape
    dh = d // heads
    out = np.zeros((n_q, d))
    for h in range(heads):
        c0 = h * dh
        for i in range(n_q):
            s = [sum(q[i, c0 + t] * k[j, c0 + t] for t in range(dh)) / math.sqrt(dh)
                 for j in range(k.shape[0])]
            m = max(s)
            e = [math.exp(val - m) for val in s]
            z = sum(e)
            for t in range(dh):
                out[i, c0 + t] = sum(e[j] * v[j, c0 + t] for j in range(k.shape[0])) / z
    return out


# ----------------------------------------------------------------------------
# pins: each takes the oracle module and raises AssertionError on a mismatch

def pin_layer_norm(M):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 33)) * 3.0 + 1.5
    got = M.layer_norm(x, 1e-6)
    ref = tF.layer_norm(torch.from_numpy(x), (33,), eps=1e-6).numpy()
    assert _rel(got, ref) < 1e-12, "layer_norm vs torch"
    var = x.var(axis=1)
    assert np.abs(got.mean(axis=1)).max() < 1e-12, "normalised rows have mean 0"
    assert np.abs(got.var(axis=1) - var / (var + 1e-6)).max() < 1e-12, "normalised variance"


def pin_silu(M):
    z = np.linspace(-30, 30, 1001)
    assert _rel(M.silu(z), tF.silu(torch.from_numpy(z)).numpy()) < 1e-12, "silu vs torch"


def pin_attention_brute(M):
    rng = np.random.default_rng(6)
    for n, dh in ((1, 4), (2, 8), (3, 4), (17, 8)):
        q, k, v = (rng.standard_normal((n, 2 * dh)) for _ in range(3))
        assert _rel(M.attention(q, k, v, 2), brute_attention(q, k, v, 2)) < 1e-12, f"brute n={n}"
    # a subset of query rows against all keys
    q, k, v = (rng.standard_normal((11, 8)) for _ in range(3))
    assert _rel(M.attention(q[3:5], k, v, 2), brute_attention(q[3:5], k, v, 2)) < 1e-12


def pin_attention_sdpa(M):
    rng = np.random.default_rng(7)
    n, heads, dh = 64, 3, 16
    q, k, v = (rng.standard_normal((n, heads * dh)) * 2.0 for _ in range(3))

    def hd(a):
        return torch.from_numpy(a).reshape(n, heads, dh).transpose(0, 1).unsqueeze(0)

    ref = tF.scaled_dot_product_attention(hd(q), hd(k), hd(v))
    ref = ref.squeeze(0).transpose(0, 1).reshape(n, heads * dh).numpy()
    assert _rel(M.attention(q, k, v, heads), ref) < 1e-12, "attention vs sdpa"


def pin_block_torch(M):
    for dtype, args in (("bf16", dict(d=32, heads=2, ffn=96, n=19)),
                        ("f32", dict(d=48, heads=3, ffn=64, n=33)),
                        ("w8_bf16", dict(d=32, heads=2, ffn=64, n=21))):
        x, mod, w, heads = _case(dtype=dtype, **args)
        ref = torch_block(x, mod, w, heads)
        assert _rel(M.block_forward(x, mod, w, heads), ref) < 1e-12, f"block vs torch ({dtype})"
        rows = np.array([0, 4, args["n"] - 1])
        assert _rel(M.block_rows(x, mod, w, heads, rows), ref[rows]) < 1e-12, "rows vs torch"
        assert _rel(M.block_forward_chunked(x, mod, w, heads, 5, 7), ref) < 1e-12, "chunked vs torch"


def pin_chunked_schedule(M):
    x, mod, w, heads = _case(d=32, heads=2, ffn=96, n=37)
    n = x.shape[0]
    saved = M.matmul
    try:
        M.matmul = _order_stable
        y = M.block_forward(x, mod, w, heads)
        for ca, cm in ((0, n), (n, 1), (1, n), (10, 10), (12, 5), (36, 100), (5, 13)):
            yc = M.block_forward_chunked(x, mod, w, heads, ca, cm)
            assert np.array_equal(y, yc), f"chunked ({ca},{cm}) not bitwise equal"
    finally:
        M.matmul = saved
    y = M.block_forward(x, mod, w, heads)
    for ca, cm, fc in ((7, 9, 0), (0, 37, 32), (16, 16, 40), (3, 30, 96)):
        assert _rel(M.block_forward_chunked(x, mod, w, heads, ca, cm, fc), y) < 1e-12, \
            f"chunked ({ca},{cm},{fc})"


def pin_closed_forms(M):
    x, mod, w, heads = _case(d=32, heads=2, ffn=64, n=13)
    # zero gates: the block is the identity on the residual stream
    mz = mod.copy()
    mz[2] = 0.0
    mz[5] = 0.0
    assert np.array_equal(M.block_forward(x, mz, w, heads), x), "gates 0 => y == x"
    # one token: softmax over a single key is exactly 1, so o == v
    _, o, v = M.block_forward(x[:1], mod, w, heads, want=("o", "v"))
    assert np.array_equal(o, v), "N=1 => o == v"
    # scale1 = -1: every normalised row equals shift1, so every query sees identical
    # keys and values and o_i == v for all i
    m1 = mod.copy()
    m1[1] = -1.0
    _, o, v = M.block_forward(x, m1, w, heads, want=("o", "v"))
    assert np.abs(o - v[0]).max() < 1e-12 and np.abs(v - v[0]).max() == 0.0, "scale1=-1"
    # zero gate projection: silu(0) = 0, the MLP branch vanishes and y == x1
    w0 = dict(w)
    w0["gu"] = w["gu"].copy()
    w0["gu"][:64] = 0.0
    y, x1 = M.block_forward(x, mod, w0, heads, want=("x1",))
    assert np.array_equal(y, x1), "W_gate = 0 => y == x1"
    # each branch enters linearly through its gate
    y, x1 = M.block_forward(x, mod, w, heads, want=("x1",))
    m2 = mod.copy()
    m2[5] *= 2.0
    y2, x12 = M.block_forward(x, m2, w, heads, want=("x1",))
    assert np.array_equal(x1, x12) and _rel(y2 - x1, 2.0 * (y - x1)) < 1e-12, "linear in gate2"
    m3 = mod.copy()
    m3[2] *= -3.0
    _, x13 = M.block_forward(x, m3, w, heads, want=("x1",))
    assert _rel(x13 - x, -3.0 * (x1 - x)) < 1e-12, "linear in gate1"
    # no positional term and no mask: permuting tokens permutes the output
    perm = np.random.default_rng(3).permutation(x.shape[0])
    assert _rel(M.block_forward(x[perm], mod, w, heads), y[perm]) < 1e-12, "permutation"


def pin_int8_rows(M):
    rng = np.random.default_rng(9)
    q = rng.integers(-127, 127, size=(5, 7), endpoint=True).astype(np.int8)
    s = rng.uniform(1e-4, 1e-3, 5).astype(np.float32)
    wd = M.dequantize_rows(q, s)
    for r in range(5):
        for c in range(7):
            assert wd[r, c] == float(s[r]) * float(q[r, c]), "dequantised element"
    a = rng.standard_normal((3, 7))
    # a per-output-row scale factors out of the product
    assert _rel(M.linear(a, wd), M.linear(a, q.astype(np.float64)) * s.astype(np.float64)) < 1e-12


def pin_rows(M):
    x, mod, w, heads = _case(d=32, heads=2, ffn=64, n=40, seed=2)
    rows = np.array([1, 2, 17, 39])
    y, o, x1 = M.block_forward(x, mod, w, heads, want=("o", "x1"))
    yr, orow, x1r = M.block_rows(x, mod, w, heads, rows, want=("o", "x1"))
    assert _rel(yr, y[rows]) < 1e-12 and _rel(orow, o[rows]) < 1e-12 and _rel(x1r, x1[rows]) < 1e-12


def _qk_case(n=23, d=32, heads=2, ffn=64, seed=3):
    x, mod, w, heads = _case(d=d, heads=heads, ffn=ffn, n=n, seed=seed)
    sh = synth.BlockShape("t", d, heads, d // heads, ffn, n, "bf16")
    qk = {k: np.asarray(v, np.float64) for k, v in synth.make_qk_inputs(sh, seed).items()}
    return x, mod, w, heads, qk


def pin_rms_norm_heads(M):
    rng = np.random.default_rng(11)
    t = rng.standard_normal((9, 3 * 16)) * 2.5
    wv = 1.0 + 0.3 * rng.standard_normal(16)
    got = M.rms_norm_heads(t, wv, 3, 1e-6)
    ref = tF.rms_norm(torch.from_numpy(t).reshape(9, 3, 16), (16,), torch.from_numpy(wv), eps=1e-6)
    assert _rel(got, ref.reshape(9, 48).numpy()) < 1e-12, "rms_norm vs torch"
    unit = M.rms_norm_heads(t, np.ones(16), 3, 0.0).reshape(9, 3, 16)
    assert np.abs(np.sqrt((unit ** 2).mean(axis=2)) - 1).max() < 1e-12, "unit RMS per head"


def pin_rope(M):
    rng = np.random.default_rng(12)
    n, heads, dh = 7, 2, 8
    t = rng.standard_normal((n, heads * dh))
    ang = rng.uniform(-4, 4, (n, dh // 2))
    got = M.rope(t, np.cos(ang), np.sin(ang), heads)
    # the same rotation as a complex product (a + ib) e^{i angle}
    z = t.reshape(n, heads, dh // 2, 2)
    zc = (z[..., 0] + 1j * z[..., 1]) * np.exp(1j * ang)[:, None, :]
    ref = np.stack([zc.real, zc.imag], axis=-1).reshape(n, heads * dh)
    assert _rel(got, ref) < 1e-12, "rope vs complex rotation"
    assert np.array_equal(M.rope(t, np.ones((n, dh // 2)), np.zeros((n, dh // 2)), heads), t), "zero angle"
    # scores depend only on the position difference
    cos_a, sin_a = synth.rope_tables(n, dh, offset=0)
    cos_b, sin_b = synth.rope_tables(n, dh, offset=37)
    q, k = rng.standard_normal((n, heads * dh)), rng.standard_normal((n, heads * dh))
    sa = M.rope(q, cos_a, sin_a, heads) @ M.rope(k, cos_a, sin_a, heads).T
    sb = M.rope(q, cos_b, sin_b, heads) @ M.rope(k, cos_b, sin_b, heads).T
    assert np.abs(sa - sb).max() < 1e-5, "relative positions"  # tables are fp32


def pin_block_qk(M):
    x, mod, w, heads, qk = _qk_case()
    n, d = x.shape
    dh = d // heads
    X = torch.from_numpy(x)
    sh1, sc1 = torch.from_numpy(mod[0]), torch.from_numpy(mod[1])
    n1 = tF.layer_norm(X, (d,), eps=1e-6) * (1 + sc1) + sh1
    q, k, v = tF.linear(n1, torch.from_numpy(w["qkv"])).split(d, dim=1)

    def norm_rope(t, wv):
        th = tF.rms_norm(t.reshape(n, heads, dh), (dh,), torch.from_numpy(wv), eps=1e-6)
        zc = torch.view_as_complex(th.reshape(n, heads, dh // 2, 2).contiguous())
        rot = torch.polar(torch.ones(n, dh // 2, dtype=torch.float64),
                          torch.atan2(torch.from_numpy(qk["sin"]), torch.from_numpy(qk["cos"])))
        return torch.view_as_real(zc * rot[:, None, :]).reshape(n, d)

    q, k = norm_rope(q, qk["q_norm"]), norm_rope(k, qk["k_norm"])

    def hd(t):
        return t.reshape(n, heads, dh).transpose(0, 1).unsqueeze(0)

    o = tF.scaled_dot_product_attention(hd(q), hd(k), hd(v)).squeeze(0).transpose(0, 1).reshape(n, d)
    _, o_or = M.block_forward(x, mod, w, heads, want=("o",), qk=qk)
    # the fp32 tables are not exactly unit-norm pairs, so compare at the tables' precision
    assert _rel(o_or, o.numpy()) < 1e-6, "qk-norm + rope block vs torch"
    y = M.block_forward(x, mod, w, heads, qk=qk)
    rows = np.array([0, 5, n - 1])
    assert _rel(M.block_rows(x, mod, w, heads, rows, qk=qk), y[rows]) < 1e-12, "rows with qk"
    saved = M.matmul
    try:
        M.matmul = _order_stable
        y = M.block_forward(x, mod, w, heads, qk=qk)
        for ca, cm in ((5, 7), (0, n), (22, 3)):
            assert np.array_equal(M.block_forward_chunked(x, mod, w, heads, ca, cm, qk=qk), y), "chunked qk"
    finally:
        M.matmul = saved


def pin_final_layer(M):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((29, 48)) * 2.0
    sh, sc = rng.standard_normal(48) * 0.3, rng.standard_normal(48) * 0.3
    wf = rng.standard_normal((16, 48)) / np.sqrt(48)
    X = torch.from_numpy(x)
    ref = tF.linear(tF.layer_norm(X, (48,), eps=1e-6) * (1 + torch.from_numpy(sc)) + torch.from_numpy(sh),
                    torch.from_numpy(wf)).numpy()
    assert _rel(M.final_layer(x, sh, sc, wf), ref) < 1e-12, "final layer vs torch"
    saved = M.matmul
    try:
        M.matmul = _order_stable
        full = M.final_layer(x, sh, sc, wf)
        for c in (1, 5, 28, 0):
            assert np.array_equal(M.final_layer_chunked(x, sh, sc, wf, c), full), "final layer chunked"
    finally:
        M.matmul = saved


def _lora_case(dtype="bf16", d=32, heads=2, ffn=96, n=19, rank=16):
    x, mod, w, heads = _case(d=d, heads=heads, ffn=ffn, n=n, dtype=dtype)
    sh = synth.BlockShape("t", d, heads, d // heads, ffn, n, dtype)
    lora = {k: (synth.to_f64(a), synth.to_f64(b), al) for k, (a, b, al) in synth.make_lora(sh, rank).items()}
    return x, mod, w, heads, lora


def _merged(w, lora, d, ffn):
    """The same block with each adapter folded into its weight: W + alpha B A."""
    m = {k: np.array(v, copy=True) for k, v in w.items()}
    rows = {"q": ("qkv", 0), "k": ("qkv", d), "v": ("qkv", 2 * d), "o": ("o", 0),
            "gate": ("gu", 0), "up": ("gu", ffn), "down": ("down", 0)}
    for name, (a, b, alpha) in lora.items():
        key, r0 = rows[name]
        delta = alpha * (b @ a)
        m[key][r0:r0 + delta.shape[0]] += delta
    return m


def pin_lora(M):
    # the adapter term against torch: alpha * linear(linear(a, A), B)
    rng = np.random.default_rng(17)
    a_in = rng.standard_normal((9, 40))
    A, B = rng.standard_normal((16, 40)) / 6.0, rng.standard_normal((24, 16)) / 4.0
    ref = (0.75 * tF.linear(tF.linear(torch.from_numpy(a_in), torch.from_numpy(A)), torch.from_numpy(B))).numpy()
    assert _rel(M.lora_delta(a_in, (A, B, 0.75)), ref) < 1e-12, "lora delta vs torch"
    # activation-space adapters equal the same block with merged weights
    # W + alpha B A, on every projection at once and in every schedule
    for dtype in ("bf16", "w8_bf16"):
        x, mod, w, heads, lora = _lora_case(dtype)
        d, ffn = x.shape[1], w["down"].shape[1]
        ref = M.block_forward(x, mod, _merged(w, lora, d, ffn), heads)
        assert _rel(M.block_forward(x, mod, w, heads, lora=lora), ref) < 1e-12, f"lora vs merged ({dtype})"
        assert _rel(M.block_forward_chunked(x, mod, w, heads, 5, 7, lora=lora), ref) < 1e-12, "chunked lora"
        assert _rel(M.block_forward_chunked(x, mod, w, heads, 0, 4, 32, lora=lora), ref) < 1e-12, "ffn-sliced lora"
        rows = np.array([0, 6, x.shape[0] - 1])
        assert _rel(M.block_rows(x, mod, w, heads, rows, lora=lora), ref[rows]) < 1e-12, "rows lora"
        # each adapter alone, on its own projection
        for name in lora:
            one = {name: lora[name]}
            assert _rel(M.block_forward(x, mod, w, heads, lora=one),
                        M.block_forward(x, mod, _merged(w, one, d, ffn), heads)) < 1e-12, f"lora {name} alone"
    # zero B: exactly the block without adapters
    x, mod, w, heads, lora = _lora_case("bf16")
    zero = {k: (a, np.zeros_like(b), al) for k, (a, b, al) in lora.items()}
    assert np.array_equal(M.block_forward(x, mod, w, heads, lora=zero), M.block_forward(x, mod, w, heads)), "zero B"
    # the chunked schedule is bitwise when the matrix product is order-stable
    saved = M.matmul
    try:
        M.matmul = _order_stable
        y = M.block_forward(x, mod, w, heads, lora=lora)
        for ca, cm in ((5, 7), (0, 19), (3, 2)):
            assert np.array_equal(M.block_forward_chunked(x, mod, w, heads, ca, cm, lora=lora), y), "chunked lora bits"
    finally:
        M.matmul = saved


PINS = [pin_final_layer, pin_lora, pin_layer_norm, pin_silu, pin_attention_brute, pin_attention_sdpa, pin_block_torch,
        pin_chunked_schedule, pin_closed_forms, pin_int8_rows, pin_rows, pin_rms_norm_heads, pin_rope,
        pin_block_qk]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    pin(O)


# ----------------------------------------------------------------------------
# planted mistakes: each replaces one oracle function with a wrong variant

_orig = {name: getattr(O, name) for name in
         ("layer_norm", "modulate", "linear", "silu", "attention", "dequantize_rows",
          "block_forward", "block_forward_chunked", "rms_norm_heads", "rope", "qk_transform",
          "final_layer", "final_layer_chunked", "lora_delta", "_mlp_hidden")}


def _lora_alpha_dropped(a, ad):
    return 0.0 if ad is None else O.linear(O.linear(a, ad[0]), ad[1])


def _lora_alpha_twice(a, ad):
    return 0.0 if ad is None else ad[2] * _orig["lora_delta"](a, ad)


def _lora_factors_swapped(a, ad):
    # B's transpose as the down factor and A's transpose as the up factor
    return 0.0 if ad is None else ad[2] * O.linear(O.linear(a, ad[1].T), ad[0].T)


def _mlp_hidden_adapters_swapped(n2, w, ffn, f0, f1, lora):
    sw = dict(lora)
    sw["gate"], sw["up"] = lora.get("up"), lora.get("gate")
    return _orig["_mlp_hidden"](n2, w, ffn, f0, f1, {k: v for k, v in sw.items() if v is not None})


def _chunked_down_adapter_last_slice(x, mod, w, n_heads, attn_chunk, mlp_chunk, ffn_chunk=0, eps=1e-6, qk=None,
                                     lora=None):
    # the down adapter sees only the last FFN feature slice of h
    if not lora or "down" not in lora or ffn_chunk <= 0:
        return _orig["block_forward_chunked"](x, mod, w, n_heads, attn_chunk, mlp_chunk, ffn_chunk, eps, qk, lora)
    a, b, al = lora["down"]
    ffn = w["down"].shape[1]
    f0 = (ffn - 1) // ffn_chunk * ffn_chunk
    cut = dict(lora)
    cut["down"] = (np.where(np.arange(ffn)[None, :] >= f0, a, 0.0), b, al)
    return _orig["block_forward_chunked"](x, mod, w, n_heads, attn_chunk, mlp_chunk, ffn_chunk, eps, qk, cut)



def _final_shift_scale_swapped(x, shift, scale, w, eps=1e-6):
    return _orig["final_layer"](x, scale, shift, w, eps)


def _final_chunk_drops_tail(x, shift, scale, w, chunk, eps=1e-6):
    n = x.shape[0]
    c = n if chunk <= 0 else min(chunk, n)
    out = np.zeros((n, w.shape[0]))
    for s0 in range(0, n - c + 1, c):  # forgets a ragged last slab
        out[s0:s0 + c] = _orig["final_layer"](x[s0:s0 + c], shift, scale, w, eps)
    return out


def _rope_sin_flipped(t, cos, sin, n_heads):
    return _orig["rope"](t, cos, -np.asarray(sin), n_heads)


def _rope_halves(t, cos, sin, n_heads):
    # rotate (x_j, x_{j+dh/2}) instead of adjacent pairs
    n, d = t.shape
    dh = d // n_heads
    th = t.reshape(n, n_heads, 2, dh // 2).transpose(0, 1, 3, 2).reshape(n, d)
    return _orig["rope"](th, cos, sin, n_heads)


def _rms_over_d(t, w, n_heads, eps):
    ms = (t ** 2).mean(axis=1, keepdims=True)
    return t / np.sqrt(ms + eps) * np.tile(np.asarray(w, np.float64), n_heads)


def _qk_rope_first(t, norm_w, cos, sin, n_heads, eps):
    if cos is not None:
        t = _orig["rope"](t, cos, sin, n_heads)
    if norm_w is not None:
        t = _orig["rms_norm_heads"](t, norm_w, n_heads, eps)
    return t


def _ln_unbiased(x, eps):
    mu = x.mean(axis=1, keepdims=True)
    return (x - mu) / np.sqrt(x.var(axis=1, ddof=1, keepdims=True) + eps)


def _ln_no_eps(x, eps):
    mu = x.mean(axis=1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(axis=1, keepdims=True))


def _attn_variant(scale_pow=0.5, axis=1, use_k_for_v=False, strided_heads=False):
    def attn(q, k, v, n_heads):
        d = q.shape[1]
        dh = d // n_heads
        out = np.empty((q.shape[0], d))
        for h in range(n_heads):
            c = slice(h, d, n_heads) if strided_heads else slice(h * dh, (h + 1) * dh)
            s = q[:, c] @ k[:, c].T / dh ** scale_pow
            s = s - s.max(axis=axis, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=axis, keepdims=True)
            out[:, c] = p @ (k if use_k_for_v else v)[:, c]
        return out
    return attn


def _block_with_mod(perm):
    def bf(x, mod, w, n_heads, eps=1e-6, want=()):
        return _orig["block_forward"](x, np.asarray(mod)[list(perm)], w, n_heads, eps, want)
    return bf


def _block_gate_up_swapped(x, mod, w, n_heads, eps=1e-6, want=()):
    ffn = w["down"].shape[1]
    w2 = dict(w)
    w2["gu"] = np.concatenate([w["gu"][ffn:], w["gu"][:ffn]])
    return _orig["block_forward"](x, mod, w2, n_heads, eps, want)


def _block_mlp_residual_from_x(x, mod, w, n_heads, eps=1e-6, want=()):
    res = _orig["block_forward"](x, mod, w, n_heads, eps, ("x1",) + tuple(want))
    y, x1 = res[0], res[1]
    out = y - x1 + x
    return out if not want else (out,) + tuple(res[2:])


def _chunked_interleaved(x, mod, w, n_heads, attn_chunk, mlp_chunk, ffn_chunk=0, eps=1e-6):
    # Pass 1 fused into pass 2: each slice projects its own K/V and attends only
    # the keys projected so far, before the later slabs exist.
    n, d = x.shape
    ffn = w["down"].shape[1]
    ca = n if attn_chunk <= 0 else min(attn_chunk, n)
    sh1, sc1, g1, sh2, sc2, g2 = mod
    res = x.copy()
    k = np.zeros((n, d))
    v = np.zeros((n, d))
    for s0 in range(0, n, ca):
        s1 = min(n, s0 + ca)
        n1 = O.modulate(O.layer_norm(res[s0:s1], eps), sh1, sc1)
        k[s0:s1] = O.linear(n1, w["qkv"][d:2 * d])
        v[s0:s1] = O.linear(n1, w["qkv"][2 * d:])
        o = O.attention(O.linear(n1, w["qkv"][:d]), k[:s1], v[:s1], n_heads)
        res[s0:s1] += g1 * O.linear(o, w["o"])
    n2 = O.modulate(O.layer_norm(res, eps), sh2, sc2)
    h = O.silu(O.linear(n2, w["gu"][:ffn])) * O.linear(n2, w["gu"][ffn:])
    return res + g2 * O.linear(h, w["down"])


def _block_wo_transposed(x, mod, w, n_heads, eps=1e-6, want=()):
    w2 = dict(w)
    w2["o"] = np.ascontiguousarray(w["o"].T)
    return _orig["block_forward"](x, mod, w2, n_heads, eps, want)


MUTANTS = {
    "layer_norm: unbiased variance": ("layer_norm", _ln_unbiased),
    "layer_norm: eps dropped": ("layer_norm", _ln_no_eps),
    "modulate: scale instead of 1+scale": ("modulate", lambda nrm, sh, sc: nrm * sc + sh),
    "modulate: shift and scale swapped": ("modulate", lambda nrm, sh, sc: nrm * (1 + sh) + sc),
    "linear: weight not transposed": ("linear", lambda a, w: a @ w),
    "silu: sigmoid of -z": ("silu", lambda z: z / (1.0 + np.exp(z))),
    "attention: 1/dh scale": ("attention", _attn_variant(scale_pow=1.0)),
    "attention: no scale": ("attention", _attn_variant(scale_pow=0.0)),
    "attention: softmax over queries": ("attention", _attn_variant(axis=0)),
    "attention: keys used as values": ("attention", _attn_variant(use_k_for_v=True)),
    "attention: strided head columns": ("attention", _attn_variant(strided_heads=True)),
    "dequantize: per-column scale": ("dequantize_rows",
                                     lambda q, s: np.asarray(q, np.float64) * np.resize(
                                         np.asarray(s, np.float64), q.shape[1])[None, :]),
    "block: gates swapped": ("block_forward", _block_with_mod((0, 1, 5, 3, 4, 2))),
    "block: norm2 reuses shift1/scale1": ("block_forward", _block_with_mod((0, 1, 2, 0, 1, 5))),
    "block: gate and up swapped": ("block_forward", _block_gate_up_swapped),
    "block: square out-projection transposed": ("block_forward", _block_wo_transposed),
    "block: MLP residual from x, not x1": ("block_forward", _block_mlp_residual_from_x),
    "chunked: K/V interleaved with in-place writes": ("block_forward_chunked", _chunked_interleaved),
    "rope: sine sign flipped": ("rope", _rope_sin_flipped),
    "rope: halves instead of adjacent pairs": ("rope", _rope_halves),
    "qk-norm: RMS over all of d": ("rms_norm_heads", _rms_over_d),
    "qk: rope before the norm": ("qk_transform", _qk_rope_first),
    "final layer: shift and scale swapped": ("final_layer", _final_shift_scale_swapped),
    "final layer: ragged last slab dropped": ("final_layer_chunked", _final_chunk_drops_tail),
    "lora: alpha dropped": ("lora_delta", _lora_alpha_dropped),
    "lora: alpha applied twice": ("lora_delta", _lora_alpha_twice),
    "lora: factors transposed and swapped": ("lora_delta", _lora_factors_swapped),
    "lora: gate and up adapters swapped": ("_mlp_hidden", _mlp_hidden_adapters_swapped),
    "lora: down adapter sees only the last FFN slice": ("block_forward_chunked", _chunked_down_adapter_last_slice),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    monkeypatch.setattr(O, name, fn)
    failed = []
    for pin in PINS:
        try:
            pin(O)
        except Exception as e:  # an assertion or a shape error both expose it
            failed.append(f"{pin.__name__}: {type(e).__name__}")
    assert failed, f"no pin catches: {mutant}"


def test_block_draws_equal_single_draw(monkeypatch):
    sh = synth.BlockShape("t", 32, 2, 16, 64, 50, "bf16")
    a = synth.make_inputs(sh, 4)
    monkeypatch.setattr(synth, "_BLOCK_ELEMS", 100)
    b = synth.make_inputs(sh, 4)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
