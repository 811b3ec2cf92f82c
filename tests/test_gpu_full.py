"""Parity at the full workload sizes (GPU), on 512 sampled query rows, plus the
bit-identity sweep over chunk settings at full size.

For each workload: the block runs through the C ABI for every chunk setting of
its sweep, in the launch configuration ``bench.py`` times; the output bytes
must be identical across the sweep ("LayerStream: H3 Chunking": chunked output
is bit-identical). The oracle computes norm1 and K/V for all N tokens and the
remaining steps for the sampled rows (exact for them). The attention output O
is also recomputed through the step kernels for the sampled rows against all N
keys and checked directly, because its contribution to y sits near the bf16
resolution of y.
"""
import hashlib
import sys
import time

import numpy as np
import pytest
import torch

import oracle.dit_block as O
from _helpers import INT8_BARS, check_bf16_bar, max_abs, oracle_inputs, rel_l2, to_f64
from memory_bounded_chunked_amd import block as B
from memory_bounded_chunked_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

SWEEPS = {
    "mid": [(4096, 4096, 0), (0, 16384, 0), (3000, 5000, 0)],
    # key split of 4 ranges per query (dit_block_set_attention_splits), small slices
    "large-split4": [(2048, 2048, 0), (8192, 8192, 0), (1000, 3000, 0)],
    "large": [(8192, 8192, 0), (0, 32768, 0), (5000, 3000, 0)],
    "longclip": [(8192, 8192, 3456), (16384, 4096, 3456)],
    "int8": [(a, m, 0) for a in (0, 2048, 8192) for m in (2048, 8192)],
}


def _forward(blk, x0, mod, n, ca, cm, fc):
    x = x0.clone()
    ws = torch.empty(blk.peak_workspace(n, ca, cm, fc), dtype=torch.uint8, device="cuda")
    blk.forward(x, mod, ca, cm, fc, workspace=ws)
    torch.cuda.synchronize()
    del ws
    return x


def _gpu_attention_rows(shape, inputs, rows, x0, mod):
    """O for the sampled rows through the step kernels: norm1 of all tokens, K and
    V^T of all tokens, Q of the sampled rows, attention against all N keys."""
    n, d = shape.n_tokens, shape.d
    dt = shape.dtype
    dev = "cuda"
    w = {k: B.tensor_from_stored(v, dev) for k, v in inputs.items() if k[:2] in ("w_", "s_")}
    n1 = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
    B.modnorm(x0, mod[0], mod[1], n1, eps=shape.eps)
    sq = w.get("s_qkv")
    kk = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
    B.linear(dt, "store", n1, w["w_qkv"][d:2 * d], kk, d, w_scale=None if sq is None else sq[d:2 * d])
    ldv = (n + 63) // 64 * 64
    vt = torch.empty(d, ldv, dtype=torch.bfloat16, device=dev)
    B.linear(dt, "store_t", n1, w["w_qkv"][2 * d:], vt, d, w_scale=None if sq is None else sq[2 * d:])
    idx = torch.from_numpy(rows).to(dev)
    n1r = n1.index_select(0, idx).contiguous()
    del n1
    qr = torch.empty(len(rows), d, dtype=torch.bfloat16, device=dev)
    B.linear(dt, "store", n1r, w["w_qkv"][:d], qr, d, w_scale=None if sq is None else sq[:d])
    o = torch.empty(len(rows), d, dtype=torch.bfloat16, device=dev)
    B.attention(qr, kk, vt, o, shape.n_heads, n_kv=n)
    torch.cuda.synchronize()
    return to_f64(o)


@pytest.mark.parametrize("name", list(SWEEPS))
def test_full_size_parity_and_bit_identity(name):
    shape = synth.CONFIGS[name.split("-")[0]]
    n = shape.n_tokens
    inputs = synth.make_inputs(shape, seed=0)
    blk, x0, mod = B.block_from_inputs(shape, inputs, "cuda")
    if name.endswith("-split4"):
        blk.set_attention_splits(4)
    digests = []
    y_first = None
    for ca, cm, fc in SWEEPS[name]:
        y = _forward(blk, x0, mod, n, ca, cm, fc)
        digests.append(hashlib.sha256(y.view(torch.uint8).cpu().numpy().tobytes()).hexdigest())
        if y_first is None:
            y_first = y.cpu()
        del y
    assert len(set(digests)) == 1, f"{name}: outputs differ across {SWEEPS[name]}"

    rows = synth.sample_rows(n, 512)
    o_gpu = _gpu_attention_rows(shape, inputs, rows, x0, mod)
    blk.close()
    del x0
    torch.cuda.empty_cache()

    x, modf, w = oracle_inputs(inputs)
    y_ref, o_ref = O.block_rows(x, modf, w, shape.n_heads, rows, eps=shape.eps, want=("o",))
    y = to_f64(y_first[torch.from_numpy(rows)])
    o_rel = rel_l2(o_gpu, o_ref)
    print(f"\n{name}: y max_abs={max_abs(y, y_ref):.4g} rel_l2={rel_l2(y, y_ref):.4g} "
          f"max|y_ref|={np.abs(y_ref).max():.4g}; O rel_l2={o_rel:.4g}")
    if shape.dtype == "w8_bf16":
        # int8 weights (std ~0.045) push per-head logits to O(1e2): the bf16
        # rounding of norm1, Q and K that bf16 activations require moves the
        # softmax weights by tens of percent. An emulation of exactly this
        # block's rounding points on these rows (tests/test_tolerance.py) gives
        # rel-L2 0.0195 on y and 0.0149 on O; INT8_BARS are 1.5x those floors.
        assert rel_l2(y, y_ref) <= INT8_BARS["y_rel"]
        assert max_abs(y, y_ref) <= INT8_BARS["y_max_frac"] * np.abs(y_ref).max()
        assert o_rel <= INT8_BARS["o_rel"]
    else:
        check_bf16_bar(y, y_ref)
        assert o_rel <= 1e-2


def test_full_size_with_qk_norm_and_rope():
    shape = synth.CONFIGS["large"]
    n = shape.n_tokens
    inputs = synth.make_inputs(shape, seed=0)
    qk_in = synth.make_qk_inputs(shape, 0)
    blk, x0, mod = B.block_from_inputs(shape, {**inputs, "q_norm": qk_in["q_norm"], "k_norm": qk_in["k_norm"]},
                                       "cuda")
    rope = (torch.from_numpy(qk_in["cos"]).cuda(), torch.from_numpy(qk_in["sin"]).cuda())
    digests, y_first = [], None
    for ca, cm in ((8192, 8192), (5000, 3000)):
        x = x0.clone()
        ws = torch.empty(blk.peak_workspace(n, ca, cm, 0), dtype=torch.uint8, device="cuda")
        blk.forward(x, mod, ca, cm, workspace=ws, rope=rope)
        torch.cuda.synchronize()
        digests.append(hashlib.sha256(x.view(torch.uint8).cpu().numpy().tobytes()).hexdigest())
        if y_first is None:
            y_first = x.cpu()
        del x, ws
    assert digests[0] == digests[1]
    blk.close()
    del x0
    torch.cuda.empty_cache()
    rows = synth.sample_rows(n, 512)
    xf, modf, w = oracle_inputs(inputs)
    qk = {k: np.asarray(v, np.float64) for k, v in qk_in.items()}
    y_ref = O.block_rows(xf, modf, w, shape.n_heads, rows, eps=shape.eps, qk=qk)
    y = to_f64(y_first[torch.from_numpy(rows)])
    print(f"\nlarge+qk: y max_abs={max_abs(y, y_ref):.4g} rel_l2={rel_l2(y, y_ref):.4g}")
    check_bf16_bar(y, y_ref)


def test_mid_block_full_parity():
    # Every one of the 16384 x 3072 outputs of the mid block (bench chunking
    # 4096 / 4096) against the oracle: global K/V once, then the rows in slabs
    # of 4096 (the oracle takes about two minutes on 16 host cores; a line per
    # step goes to the terminal).
    shape = synth.CONFIGS["mid"]
    n = shape.n_tokens
    inputs = synth.make_inputs(shape, seed=0)
    blk, x0, mod = B.block_from_inputs(shape, inputs, "cuda")
    y_gpu = to_f64(_forward(blk, x0, mod, n, shape.attn_chunk, shape.mlp_chunk, 0).cpu())
    blk.close()
    del x0
    torch.cuda.empty_cache()
    x, modf, w = oracle_inputs(inputs)
    t0 = time.time()
    kv = O.global_kv(x, modf, w, shape.n_heads, eps=shape.eps)
    print(f"[mid full] oracle K/V of {n} tokens: {time.time() - t0:.0f} s", file=sys.__stderr__, flush=True)
    y_ref = np.empty_like(x)
    for r0 in range(0, n, 4096):
        rows = np.arange(r0, min(n, r0 + 4096))
        y_ref[rows] = O.block_rows(x, modf, w, shape.n_heads, rows, eps=shape.eps, kv=kv)
        print(f"[mid full] oracle rows {r0}-{rows[-1]}: {time.time() - t0:.0f} s", file=sys.__stderr__, flush=True)
    print(f"\nmid full: y max_abs={max_abs(y_gpu, y_ref):.4g} rel_l2={rel_l2(y_gpu, y_ref):.4g} "
          f"elements over 2e-2: {int((np.abs(y_gpu - y_ref) > 2e-2).sum())} of {y_ref.size}")
    check_bf16_bar(y_gpu, y_ref)
