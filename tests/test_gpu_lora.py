"""Activation-space adapters (LoRA in bypass mode) on the GPU block against the
fp64 oracle ("ComfyUI-StaticPipeline", section "Activation-space LoRA (bypass
mode)": y = W a + alpha * B (A a) with W untouched), plus the bit-identity
and zero-adapter properties (GPU).

Bars: as the block without adapters (fp32 max-abs and rel-L2 1e-4; bf16 and
int8-weight blocks ``check_bf16_bar``), and the adapter's own contribution
(output with adapters minus output without) within rel-L2 3e-2 (bf16) or
1e-3 (fp32) of the oracle's, so that a wrong or missing adapter term cannot
hide in the output's rounding.
"""
import numpy as np
import pytest
import torch

import oracle.dit_block as O
from _helpers import INT8_ADAPTER_SHAPES, bits, check_bf16_bar, half_ulp_bf16, max_abs, oracle_inputs, rel_l2, to_f64
from memory_bounded_chunked_amd import block as B
from memory_bounded_chunked_amd import synth

pytestmark = pytest.mark.gpu

SMALL = {
    "bf16": synth.BlockShape("small-bf16", 256, 2, 128, 512, 777, "bf16"),
    "f32": synth.BlockShape("small-f32", 256, 4, 64, 1024, 300, "f32"),
    "w8_bf16": synth.BlockShape("small-w8", 256, 2, 128, 512, 611, "w8_bf16"),
    "bf16-dh64": synth.BlockShape("small-dh64", 256, 4, 64, 768, 450, "bf16"),
}
RANKS = {"q": 16, "k": 32, "v": 48, "o": 16, "gate": 32, "up": 16, "down": 64}


def _run(shape, inputs, lora, ca, cm, fc=0, poison=False):
    blk, x, mod = B.block_from_inputs(shape, inputs)
    if lora is not None:
        blk.set_lora({k: (B.tensor_from_stored(a, "cuda"), B.tensor_from_stored(b, "cuda"), al)
                      for k, (a, b, al) in lora.items()})
    ws = torch.empty(blk.peak_workspace(shape.n_tokens, ca, cm, fc), dtype=torch.uint8, device="cuda")
    if poison:
        ws.fill_(0xFF)
    blk.forward(x, mod, ca, cm, fc, workspace=ws)
    torch.cuda.synchronize()
    out = x.cpu()
    blk.close()
    return out


def _lora_f64(lora):
    return O.lora_f64({k: (synth.to_f64(a), synth.to_f64(b), al) for k, (a, b, al) in lora.items()})


@pytest.fixture(scope="module", params=sorted(SMALL))
def case(request):
    shape = SMALL[request.param]
    inputs = synth.make_inputs(shape, seed=0)
    lora = synth.make_lora(shape, RANKS, seed=0)
    x, mod, w = oracle_inputs(inputs)
    y_ref = O.block_forward(x, mod, w, shape.n_heads, lora=_lora_f64(lora))
    y0_ref = O.block_forward(x, mod, w, shape.n_heads)
    return shape, inputs, lora, x, y_ref, y0_ref


def test_lora_block_matches_oracle(case):
    shape, inputs, lora, x, y_ref, y0_ref = case
    y = to_f64(_run(shape, inputs, lora, 256, 256))
    y0 = to_f64(_run(shape, inputs, None, 256, 256))
    if shape.dtype == "f32":
        assert max_abs(y, y_ref) <= 1e-4 and rel_l2(y, y_ref) <= 1e-4
        assert rel_l2(y - y0, y_ref - y0_ref) <= 1e-3
    else:
        check_bf16_bar(y, y_ref)
        assert rel_l2(y - y0, y_ref - y0_ref) <= 3e-2
    # the adapters matter at this scale: their term is far above the output's rounding
    assert rel_l2(y0_ref, y_ref) > 0.1


def test_lora_bit_identical_across_chunks(case):
    shape, inputs, lora, _, _, _ = case
    n = shape.n_tokens
    ref = bits(_run(shape, inputs, lora, 0, n))
    for ca, cm in ((256, 256), (100, 300), (n, 64), (1, 999)):
        assert bits(_run(shape, inputs, lora, ca, cm)) == ref, (ca, cm)
    assert bits(_run(shape, inputs, lora, 128, 192, poison=True)) == bits(_run(shape, inputs, lora, 128, 192))


def test_zero_adapters_equal_no_adapters(case):
    shape, inputs, lora, _, _, _ = case
    zero = {k: (a, np.zeros_like(b), al) for k, (a, b, al) in lora.items()}
    assert bits(_run(shape, inputs, zero, 200, 300)) == bits(_run(shape, inputs, None, 200, 300))


def test_lora_ffn_feature_slices(case):
    shape, inputs, lora, _, y_ref, _ = case
    y = to_f64(_run(shape, inputs, lora, 256, 256, fc=128))
    if shape.dtype == "f32":
        assert max_abs(y, y_ref) <= 1e-4 and rel_l2(y, y_ref) <= 1e-4
    else:
        check_bf16_bar(y, y_ref)


@pytest.mark.parametrize("key", ["bf16", "f32", "w8_bf16"])
def test_lora_with_qk_norm_rope_and_feature_slices(key):
    # every widening of the block at once: adapters on all seven projections,
    # QK RMSNorm + RoPE, and (in the second setting) FFN-feature slices
    shape = SMALL[key]
    inputs = synth.make_inputs(shape, 0)
    qk_in = synth.make_qk_inputs(shape, 0)
    lora = synth.make_lora(shape, RANKS, seed=2)
    x, mod, w = oracle_inputs(inputs)
    qk = {k: np.asarray(v, np.float64) for k, v in qk_in.items()}
    y_ref = O.block_forward(x, mod, w, shape.n_heads, qk=qk, lora=_lora_f64(lora))
    blk, xt, modt = B.block_from_inputs(shape, {**inputs, "q_norm": qk_in["q_norm"], "k_norm": qk_in["k_norm"]})
    blk.set_lora({k: (B.tensor_from_stored(a, "cuda"), B.tensor_from_stored(b, "cuda"), al)
                  for k, (a, b, al) in lora.items()})
    rope = (torch.from_numpy(qk_in["cos"]).cuda(), torch.from_numpy(qk_in["sin"]).cuda())
    n = shape.n_tokens
    outs = {}
    for ca, cm, fc in ((256, 256, 0), (0, n, 0), (100, 300, 0), (256, 256, 128)):
        xx = xt.clone()
        blk.forward(xx, modt, ca, cm, fc, rope=rope)
        torch.cuda.synchronize()
        outs[(ca, cm, fc)] = xx.cpu()
    blk.close()
    base = outs[(256, 256, 0)]
    assert all(bits(o) == bits(base) for k, o in outs.items() if k[2] == 0), "bit-identity across (Ca, Cm)"
    for o in (base, outs[(256, 256, 128)]):
        y = to_f64(o)
        if shape.dtype == "f32":
            assert max_abs(y, y_ref) <= 1e-4 and rel_l2(y, y_ref) <= 1e-4
        else:
            check_bf16_bar(y, y_ref)


@pytest.mark.parametrize("shape,bar", [
    # fp32: the adapter's term is resolved to ~1e-6, so every target is held tightly
    (synth.BlockShape("single-f32", 256, 4, 64, 1024, 300, "f32"), 1e-3),
    # bf16 with 64 tokens: attention's share of y is far above bf16 resolution,
    # so the q, k, v and o adapters (which act through attention) stay visible
    (synth.BlockShape("single-bf16", 256, 2, 128, 512, 64, "bf16"), 8e-2),
], ids=["f32", "bf16-64tok"])
def test_single_adapter_on_each_projection(shape, bar):
    inputs = synth.make_inputs(shape, seed=0)
    x, mod, w = oracle_inputs(inputs)
    y0 = to_f64(_run(shape, inputs, None, 128, 128))
    y0_ref = O.block_forward(x, mod, w, shape.n_heads)
    for name in synth.LORA_TARGETS:
        lora = synth.make_lora(shape, 32, seed=1, targets=(name,), alpha=2.0)
        y_ref = O.block_forward(x, mod, w, shape.n_heads, lora=_lora_f64(lora))
        y = to_f64(_run(shape, inputs, lora, 128, 128))
        if shape.dtype == "f32":
            assert max_abs(y, y_ref) <= 1e-4, name
        else:
            # alpha = 2 adapters make |y| reach 8 and more, where the output's own
            # half-ulp is 0.016-0.03, and push the error of the path's own bf16
            # rounding points past 2e-2 beyond that half-ulp (0.026 for the gate
            # adapter in an fp64 emulation of those points: test_tolerance.py),
            # so the bar per element is 3e-2 beyond the half-ulp (the "rarer than
            # 1e-4" count is meaningless on 16k elements)
            assert rel_l2(y, y_ref) <= 1e-2, name
            assert float((np.abs(y - y_ref) - half_ulp_bf16(y_ref)).max()) <= 3e-2, name
        assert rel_l2(y - y0, y_ref - y0_ref) <= bar, name


@pytest.mark.parametrize("rank", [80, 256])
def test_lora_rank_above_one_staging_chunk(rank):
    # bf16 adapters are staged through LDS in rank chunks of 64; ranks of 80
    # (a ragged second chunk) and 256 (four chunks), on every projection
    shape = SMALL["bf16"]
    inputs = synth.make_inputs(shape, seed=0)
    lora = synth.make_lora(shape, rank, seed=3)
    x, mod, w = oracle_inputs(inputs)
    y_ref = O.block_forward(x, mod, w, shape.n_heads, lora=_lora_f64(lora))
    y0_ref = O.block_forward(x, mod, w, shape.n_heads)
    y = to_f64(_run(shape, inputs, lora, 256, 256))
    y0 = to_f64(_run(shape, inputs, None, 256, 256))
    check_bf16_bar(y, y_ref)
    assert rel_l2(y - y0, y_ref - y0_ref) <= 3e-2
    assert bits(_run(shape, inputs, lora, 100, 300)) == bits(_run(shape, inputs, lora, 256, 256))


@pytest.mark.timeout(900)
def test_lora_mid_block_sampled_rows():
    # the 16k-token, d=3072 block with rank-64 adapters on every projection,
    # in its bench chunking, against the oracle on 256 sampled rows
    shape = synth.CONFIGS["mid"]
    inputs = synth.make_inputs(shape, seed=0)
    lora = synth.make_lora(shape, 64, seed=0)
    y = _run(shape, inputs, lora, shape.attn_chunk, shape.mlp_chunk)
    rows = synth.sample_rows(shape.n_tokens, 256, seed=1)
    x, mod, w = oracle_inputs(inputs)
    y_ref = O.block_rows(x, mod, w, shape.n_heads, rows, lora=_lora_f64(lora))
    check_bf16_bar(to_f64(y)[rows], y_ref)
    assert bits(_run(shape, inputs, lora, 0, shape.n_tokens)) == bits(y)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(INT8_ADAPTER_SHAPES))
@pytest.mark.parametrize("rank", [80, 256])
def test_int8_adapters_in_wide_tiles(name, rank):
    # int8 weights with adapters where the projections take 256-wide weight
    # tiles, whose adapter phase runs after the main loop (with all
    # accumulators live; LDS-staged in batches of 4 loads). d = 1024 with 16384
    # tokens: the Q, out, gate/up, down and feature-slice (ACCUM) projections
    # of a 16384-token slab run in 256-wide tiles, those of 4096-token slabs in
    # 128-wide ones; d = 4096: the fused K|V projection (2d = 8192 outputs)
    # runs in 256-wide tiles. Ranks 80 (a ragged second staging chunk) and 256
    # (four chunks). Against the oracle on 512 sampled rows with the bars that
    # the emulation of the path's rounding points derives (INT8_ADAPTER_SHAPES),
    # and bit-identical across chunk settings.
    (d, heads, dh, ffn, n), bars = INT8_ADAPTER_SHAPES[name]
    shape = synth.BlockShape(name, d, heads, dh, ffn, n, "w8_bf16")
    inputs = synth.make_inputs(shape, seed=0)
    lora = synth.make_lora(shape, rank, seed=3)
    sweep = [(n, n, 0), (n // 4, n // 4, 0), (0, 5000, 0)] if n >= 16384 else [(n, n, 0), (300, 500, 0), (100, 64, 0)]
    outs = [_run(shape, inputs, lora, ca, cm, fc) for ca, cm, fc in sweep]
    assert all(bits(o) == bits(outs[0]) for o in outs[1:]), "bit-identity across (Ca, Cm)"
    sliced = _run(shape, inputs, lora, n, n, ffn // 2)  # two FFN feature slices: EPI_ACCUM then EPI_FINAL
    rows = synth.sample_rows(n, 512)
    x, mod, w = oracle_inputs(inputs)
    y_ref = O.block_rows(x, mod, w, heads, rows, lora=_lora_f64(lora))
    for out in (outs[0], sliced):
        y = to_f64(out)[rows]
        assert rel_l2(y, y_ref) <= bars["y_rel"], rel_l2(y, y_ref)
        assert max_abs(y, y_ref) <= bars["y_max_frac"] * np.abs(y_ref).max(), max_abs(y, y_ref)
