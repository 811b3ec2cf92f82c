"""Per-kernel parity of the HIP steps against the fp64 oracle (GPU).

Each kernel is called through its C-ABI step entry point on seeded inputs
whose sizes span several tiles and end in ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle.dit_block as O
from _helpers import bf16_round, max_abs, rel_l2, to_f64
from memory_bounded_chunked_amd import block as B
from memory_bounded_chunked_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16(a: np.ndarray) -> torch.Tensor:
    return B.tensor_from_stored(synth.f64_to_bf16_bits(a), DEV)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# d = 8 and 520: a single 8-element group, and one group past a multiple of
# 64 lanes (the lanes past the row end re-read the last group and store nothing)
@pytest.mark.parametrize("rows,d", [(1, 256), (37, 256), (1000, 3072), (515, 5120), (5, 8), (33, 520)])
def test_modnorm_bf16(rows, d):
    rng = _rng(rows + d)
    x = synth.bf16_bits_to_f64(synth.f64_to_bf16_bits(rng.standard_normal((rows, d)) * 1.7 + 0.3))
    sh = (rng.standard_normal(d) * 0.3).astype(np.float32)
    sc = (rng.standard_normal(d) * 0.3).astype(np.float32)
    out = torch.empty(rows, d, dtype=torch.bfloat16, device=DEV)
    B.modnorm(_bf16(x), torch.from_numpy(sh).to(DEV), torch.from_numpy(sc).to(DEV), out)
    ref = O.modulate(O.layer_norm(x, 1e-6), sh.astype(np.float64), sc.astype(np.float64))
    got = to_f64(out)
    # bf16 output: within half an ulp of the reference plus fp32 statistics error
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-5)


@pytest.mark.parametrize("in_f32,out_f32", [(True, True), (True, False)])
def test_modnorm_f32_input(in_f32, out_f32):
    rows, d = 300, 1024
    rng = _rng(3)
    x = rng.standard_normal((rows, d)).astype(np.float32) * 2.0
    sh = (rng.standard_normal(d) * 0.3).astype(np.float32)
    sc = (rng.standard_normal(d) * 0.3).astype(np.float32)
    out = torch.empty(rows, d, dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    B.modnorm(torch.from_numpy(x).to(DEV), torch.from_numpy(sh).to(DEV), torch.from_numpy(sc).to(DEV), out)
    ref = O.modulate(O.layer_norm(x.astype(np.float64), 1e-6), sh.astype(np.float64), sc.astype(np.float64))
    got = to_f64(out)
    tol = 1e-5 if out_f32 else 2.0 ** -8
    assert np.all(np.abs(got - ref) <= np.abs(ref) * tol + 1e-5)


def _linear_case(dtype, m, n, k, seed, rows_w=None):
    rng = _rng(seed)
    rows_w = n if rows_w is None else rows_w
    a = rng.standard_normal((m, k))
    if dtype == "f32":
        a = a.astype(np.float32).astype(np.float64)
        w = (rng.standard_normal((rows_w, k)) / np.sqrt(k)).astype(np.float32).astype(np.float64)
        ta, tw, ts, wf = (torch.from_numpy(a.astype(np.float32)).to(DEV),
                          torch.from_numpy(w.astype(np.float32)).to(DEV), None, w)
    elif dtype == "bf16":
        a = bf16_round(a)
        w = bf16_round(rng.standard_normal((rows_w, k)) / np.sqrt(k))
        ta, tw, ts, wf = _bf16(a), _bf16(w), None, w
    else:
        a = bf16_round(a)
        q = rng.integers(-127, 127, size=(rows_w, k), endpoint=True, dtype=np.int8)
        s = rng.uniform(1e-4, 1e-3, rows_w).astype(np.float32)
        wf = O.dequantize_rows(q, s)
        ta, tw, ts = _bf16(a), torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)
    return a, wf, ta, tw, ts


def _act_dtype(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def _out_tol(dtype):
    return 1e-5 if dtype == "f32" else 2.0 ** -8


@pytest.mark.parametrize("dtype", ["bf16", "f32", "w8_bf16"])
# (257, 256, 64), (70, 512, 128), (33, 768, 192): one, two and three k-tiles in
# the 8-wave tiles, whose schedule reloads the last k-tile at the end
@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (300, 384, 512), (129, 256, 256), (257, 256, 64), (70, 512, 128),
                                   (33, 768, 192)])
def test_linear_store(dtype, m, n, k):
    a, wf, ta, tw, ts = _linear_case(dtype, m, n, k, m + n + k)
    out = torch.empty(m, n, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "store", ta, tw, out, n, w_scale=ts)
    ref = O.linear(a, wf)
    scale = np.abs(ref).max()
    assert np.all(np.abs(to_f64(out) - ref) <= np.abs(ref) * _out_tol(dtype) + 1e-5 * scale)


def _wide_columns(m: int, n: int, wb: int = 256, cus: int = 256) -> int:
    """Output columns the projection launcher gives 256-wide weight tiles (the
    rest take 128-wide ones): the split that fills whole rounds of the compute
    units, one round of 128-wide tiles costing 0.6 of a 256-wide round."""
    mt = -(-m // 256)
    best, na_best = None, 0
    for na in range(0, n + 1, wb):
        c = -(-mt * (na // wb) // cus) + 0.6 * -(-mt * ((n - na) // (wb // 2)) // cus)
        if best is None or c <= best:
            best, na_best = c, na
    return na_best


@pytest.mark.parametrize("dtype", ["bf16", "f32", "w8_bf16"])
def test_linear_tile_shape_does_not_change_bits(dtype):
    # The same output columns through launches that pick different tiles: the
    # full launch runs every column in 256-wide weight tiles (8 waves, 2 x 4;
    # the two-group schedule for bf16 weights), the slices in 128-wide (4 x 2
    # waves) and 64-wide (4 waves) ones. Every element takes the same k
    # sequence, so the bits must agree; the block's bit-identity across chunk
    # sizes relies on this.
    m, n, k = 16384, 1024, 512
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("tile choice below assumes 256 compute units")
    assert _wide_columns(m, n) == n  # the full launch: 256-wide tiles only
    a, wf, ta, tw, ts = _linear_case(dtype, m, n, k, 21)
    full = torch.empty(m, n, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "store", ta, tw, full, n, w_scale=ts)
    for c0, width in ((0, 64), (64, 128), (256, 256), (512, 512), (960, 64)):
        if width >= 128:
            assert _wide_columns(m, width) == 0  # 128-wide tiles only
        part = torch.empty(m, width, dtype=_act_dtype(dtype), device=DEV)
        B.linear(dtype, "store", ta, tw[c0:c0 + width], part, width, w_scale=None if ts is None else ts[c0:c0 + width])
        torch.cuda.synchronize()
        assert torch.equal(part.cpu(), full[:, c0:c0 + width].cpu()), (c0, width)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "w8_bf16"])
@pytest.mark.parametrize("m,n,k", [(300, 384, 512), (70, 512, 128), (16384, 1024, 512)])
def test_linear_selection_weights_exact(dtype, m, n, k):
    # Row j of W holds a single 0.5, at input column sel[j] (int8: q = 1 with
    # row scale 0.5). Each output is then one exact product plus exact zeros,
    # whatever the k order, so it must equal 0.5 * a[:, sel] bit for bit, in
    # the 64-, 128- and 256-wide tiles alike. A transposed or misplaced operand
    # fragment, a wrong k offset or a wrong row scale shows at once.
    rng = _rng(m + 3 * n + k)
    sel = rng.permutation(k)[:n] if n <= k else rng.integers(0, k, n)
    a = rng.standard_normal((m, k))
    a = a.astype(np.float32).astype(np.float64) if dtype == "f32" else bf16_round(a)
    wf = np.zeros((n, k))
    wf[np.arange(n), sel] = 0.5
    want = 0.5 * a[:, sel]
    if dtype == "f32":
        ta, tw = (torch.from_numpy(t.astype(np.float32)).to(DEV) for t in (a, wf))
        ts, expect = None, torch.from_numpy(want.astype(np.float32))
    elif dtype == "bf16":
        ta, tw, ts, expect = _bf16(a), _bf16(wf), None, _bf16(want).cpu()
    else:
        q = (wf != 0).astype(np.int8)
        ta, tw = _bf16(a), torch.from_numpy(q).to(DEV)
        ts = torch.full((n,), 0.5, dtype=torch.float32, device=DEV)
        expect = _bf16(want).cpu()
    out = torch.empty(m, n, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "store", ta, tw, out, n, w_scale=ts)
    # the transposed store (V^T of the K|V pass): the same values, columns
    # past the last token untouched
    ld = (m + 63) // 64 * 64
    out_t = torch.zeros(n, ld, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "store_t", ta, tw, out_t, n, w_scale=ts)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), expect)
    assert torch.equal(out_t[:, :m].cpu(), expect.T.contiguous())
    assert not out_t[:, m:].cpu().any()


@pytest.mark.parametrize("dtype", ["bf16", "f32", "w8_bf16"])
def test_linear_store_transposed(dtype):
    m, n, k, ld = 203, 128, 256, 256
    a, wf, ta, tw, ts = _linear_case(dtype, m, n, k, 11)
    out = torch.zeros(n, ld, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "store_t", ta, tw, out, n, w_scale=ts)
    ref = O.linear(a, wf).T
    got = to_f64(out)
    scale = np.abs(ref).max()
    assert np.all(np.abs(got[:, :m] - ref) <= np.abs(ref) * _out_tol(dtype) + 1e-5 * scale)
    assert np.all(got[:, m:] == 0)  # nothing written past the last token


@pytest.mark.parametrize("dtype", ["bf16", "f32", "w8_bf16"])
def test_linear_residual_epilogues(dtype):
    m, n, k = 333, 256, 512
    a, wf, ta, tw, ts = _linear_case(dtype, m, n, k, 12)
    rng = _rng(13)
    x = rng.standard_normal((m, n))
    x = x.astype(np.float32).astype(np.float64) if dtype == "f32" else bf16_round(x)
    tx = torch.from_numpy(x.astype(np.float32)).to(DEV) if dtype == "f32" else _bf16(x)
    gate = (rng.standard_normal(n) * 0.3).astype(np.float32)
    tg = torch.from_numpy(gate).to(DEV)
    acc = O.linear(a, wf)
    g64 = gate.astype(np.float64)
    # RESID: stage = x + gate * acc (fp32)
    stage = torch.empty(m, n, dtype=torch.float32, device=DEV)
    B.linear(dtype, "resid", ta, tw, stage, n, w_scale=ts, aux=tx, gate=tg)
    ref = x + g64 * acc
    assert max_abs(to_f64(stage), ref) <= 1e-5 * np.abs(ref).max()
    # ACCUM: stage += gate * acc
    base = to_f64(stage)
    B.linear(dtype, "accum", ta, tw, stage, n, w_scale=ts, gate=tg)
    ref2 = base + g64 * acc
    assert max_abs(to_f64(stage), ref2) <= 1e-5 * np.abs(ref2).max()
    # FINAL: out = stage + gate * acc, rounded once to the activation type
    out = torch.empty(m, n, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "final", ta, tw, out, n, w_scale=ts, aux=stage, gate=tg)
    ref3 = ref2 + g64 * acc
    got = to_f64(out)
    assert np.all(np.abs(got - ref3) <= np.abs(ref3) * _out_tol(dtype) + 1e-5 * np.abs(ref3).max())


@pytest.mark.parametrize("dtype", ["bf16", "f32", "w8_bf16"])
def test_linear_gateup(dtype):
    m, f, k = 301, 192, 256
    a, wf, ta, tw, ts = _linear_case(dtype, m, f, k, 14, rows_w=2 * f)
    out = torch.empty(m, f, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "gateup", ta, tw, out, f, w_scale=ts, up_offset=f)
    ref = O.silu(O.linear(a, wf[:f])) * O.linear(a, wf[f:])
    got = to_f64(out)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * _out_tol(dtype) + 1e-4 * np.abs(ref).max())
    # a feature slice [64, 192) addressed through the weight pointer offset
    sub = torch.empty(m, 128, dtype=_act_dtype(dtype), device=DEV)
    B.linear(dtype, "gateup", ta, tw[64:], sub, 128, w_scale=None if ts is None else ts[64:], up_offset=f)
    torch.cuda.synchronize()
    assert torch.equal(sub.cpu(), out[:, 64:].cpu())


def _attn_inputs(dtype, n_q, n_kv, heads, dh, seed, scale=1.0, key_growth=0.0):
    # key_growth: keys of 64-key tile t scaled by 1 + key_growth * t, so later
    # tiles hold ever larger logits and running maxima keep moving
    rng = _rng(seed)
    d = heads * dh
    q, k, v = (rng.standard_normal((n, d)) * scale for n in (n_q, n_kv, n_kv))
    k = k * (1.0 + key_growth * (np.arange(n_kv) // 64))[:, None]
    ld_vt = (n_kv + 63) // 64 * 64
    if dtype == "f32":
        q, k, v = (t.astype(np.float32).astype(np.float64) for t in (q, k, v))
        mk = lambda a: torch.from_numpy(a.astype(np.float32)).to(DEV)  # noqa: E731
        tdt = torch.float32
    else:
        q, k, v = (bf16_round(t) for t in (q, k, v))
        mk = _bf16
        tdt = torch.bfloat16
    vt = torch.zeros(d, ld_vt, dtype=tdt, device=DEV)
    vt[:, :n_kv] = mk(v).T
    return q, k, v, mk(q), mk(k), vt, tdt


@pytest.mark.parametrize("dtype,heads,dh,n_q,n_kv", [
    ("bf16", 3, 128, 300, 1000), ("bf16", 2, 128, 1, 1), ("bf16", 2, 128, 129, 64),
    ("bf16", 2, 64, 257, 333), ("f32", 4, 64, 300, 1000), ("f32", 2, 64, 5, 7), ("f32", 2, 128, 70, 200)])
def test_attention(dtype, heads, dh, n_q, n_kv):
    q, k, v, tq, tk, tvt, tdt = _attn_inputs(dtype, n_q, n_kv, heads, dh, n_q * 7 + n_kv)
    out = torch.empty(n_q, heads * dh, dtype=tdt, device=DEV)
    B.attention(tq, tk, tvt, out, heads, n_kv=n_kv)
    ref = O.attention(q, k, v, heads)
    got = to_f64(out)
    if dtype == "f32":
        assert max_abs(got, ref) <= 1e-5 * max(1.0, np.abs(ref).max())
    else:
        assert rel_l2(got, ref) <= 1e-2
        assert max_abs(got, ref) <= 2e-2 * max(np.abs(ref).max(), 1e-3)
        # no worse than twice what rounding the exact result to bf16 costs, plus P's rounding
        assert rel_l2(got, ref) <= 2 * rel_l2(bf16_round(ref), ref) + 4e-3


def test_attention_sharp_logits():
    # large logits (near one-hot softmax); the running max stays where the
    # first tile put it (moves: test_attention_moving_maxima)
    q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", 200, 700, 2, 128, 5, scale=3.0)
    out = torch.empty(200, 256, dtype=tdt, device=DEV)
    B.attention(tq, tk, tvt, out, 2, n_kv=700)
    ref = O.attention(q, k, v, 2)
    assert rel_l2(to_f64(out), ref) <= 1e-2


def test_attention_query_slices_bit_identical():
    n_q, n_kv = 400, 900
    q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", n_q, n_kv, 2, 128, 21)
    full = torch.empty(n_q, 256, dtype=tdt, device=DEV)
    B.attention(tq, tk, tvt, full, 2, n_kv=n_kv)
    for a, b in ((0, 1), (1, 130), (77, 400), (128, 256)):
        part = torch.empty(b - a, 256, dtype=tdt, device=DEV)
        B.attention(tq[a:b], tk, tvt, part, 2, n_kv=n_kv)
        torch.cuda.synchronize()
        assert torch.equal(part.cpu().view(torch.int16), full[a:b].cpu().view(torch.int16)), (a, b)


@pytest.mark.parametrize("dh", [64, 128])
def test_attention_every_tile_count_with_poisoned_padding(dh):
    # one to six 64-key tiles, full and ragged (every peeled path of the
    # pipelined kernel); V^T columns past n_kv hold NaN, which must not reach O
    for n_kv in (1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 320, 383):
        q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", 70, n_kv, 2, dh, n_kv)
        tvt[:, n_kv:] = float("nan")
        out = torch.empty(70, 2 * dh, dtype=tdt, device=DEV)
        B.attention(tq, tk, tvt, out, 2, n_kv=n_kv)
        ref = O.attention(q, k, v, 2)
        got = to_f64(out)
        assert np.isfinite(got).all(), n_kv
        assert rel_l2(got, ref) <= 1e-2, n_kv


def test_attention_query_slices_bit_identical_sharp_logits():
    # near one-hot softmax, sliced at offsets that are not multiples of 32
    # queries (slices with moving maxima: test_attention_moving_maxima)
    n_q, n_kv = 300, 1000
    q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", n_q, n_kv, 2, 128, 5, scale=3.0)
    full = torch.empty(n_q, 256, dtype=tdt, device=DEV)
    B.attention(tq, tk, tvt, full, 2, n_kv=n_kv)
    for a, b in ((0, 1), (1, 130), (33, 97), (77, 300), (255, 300)):
        part = torch.empty(b - a, 256, dtype=tdt, device=DEV)
        B.attention(tq[a:b], tk, tvt, part, 2, n_kv=n_kv)
        torch.cuda.synchronize()
        assert torch.equal(part.cpu().view(torch.int16), full[a:b].cpu().view(torch.int16)), (a, b)


def _moves_after_first_tile(q, k, heads, dh, bar_log2=64.0):
    """Per (query, head): how many times the kernel's rule moves the running
    max after the first 64-key tile (fp64 emulation of the rule: tile 0 sets
    the max; a later tile whose sum of exp2((s - m) c) exceeds 2^bar_log2
    moves it to that tile's max). Used to check that inputs exercise moves."""
    c = np.log2(np.e) / np.sqrt(dh)
    n_kv = k.shape[0]
    moves = np.zeros((q.shape[0], heads), dtype=np.int64)
    for h in range(heads):
        s = q[:, h * dh:(h + 1) * dh] @ k[:, h * dh:(h + 1) * dh].T
        m = s[:, :64].max(axis=1)
        for t0 in range(64, n_kv, 64):
            st = s[:, t0:t0 + 64]
            tmax = st.max(axis=1)
            lsum = np.log2(np.exp2((st - tmax[:, None]) * c).sum(axis=1)) + (tmax - m) * c
            mv = lsum > bar_log2
            moves[mv, h] += 1
            m = np.where(mv, np.maximum(m, tmax), m)
    return moves


def test_attention_moving_maxima():
    # keys whose tiles grow in scale: each query's running max moves several
    # times after tile 0, at tiles that differ between queries of one
    # wavefront; the result must meet the bar and be the same bits in any
    # query slice (slices not multiples of 32 queries, single rows)
    n_q, n_kv, heads, dh = 300, 1000, 2, 128
    q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", n_q, n_kv, heads, dh, 11, scale=3.0, key_growth=0.5)
    moves = _moves_after_first_tile(q, k, heads, dh)
    assert (moves > 0).mean() > 0.9 and moves.max() >= 2, np.bincount(moves.ravel())
    assert len(np.unique(moves[:32].ravel())) > 1  # queries of one wavefront move differently
    full = torch.empty(n_q, heads * dh, dtype=tdt, device=DEV)
    B.attention(tq, tk, tvt, full, heads, n_kv=n_kv)
    ref = O.attention(q, k, v, heads)
    assert rel_l2(to_f64(full), ref) <= 1e-2
    for a, b in ((0, 1), (1, 130), (33, 97), (77, 300), (255, 300), (296, 297)):
        part = torch.empty(b - a, heads * dh, dtype=tdt, device=DEV)
        B.attention(tq[a:b], tk, tvt, part, heads, n_kv=n_kv)
        torch.cuda.synchronize()
        assert torch.equal(part.cpu().view(torch.int16), full[a:b].cpu().view(torch.int16)), (a, b)


def test_attention_split_with_moving_maxima():
    # key ranges whose maxima differ by hundreds of units (growing key scales):
    # the merge weights exp2((m_p - m) c) span a wide range; the result meets
    # the bar and is the same bits in any query slice
    n_q, n_kv, heads, dh = 300, 1000, 2, 128
    q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", n_q, n_kv, heads, dh, 23, scale=3.0, key_growth=0.5)
    assert (_moves_after_first_tile(q, k, heads, dh) > 0).mean() > 0.9
    full = torch.empty(n_q, heads * dh, dtype=tdt, device=DEV)
    B.attention_split(tq, tk, tvt, full, heads, 3, n_kv=n_kv)
    ref = O.attention(q, k, v, heads)
    assert rel_l2(to_f64(full), ref) <= 1e-2
    for a, b in ((0, 1), (33, 97), (255, 300)):
        part = torch.empty(b - a, heads * dh, dtype=tdt, device=DEV)
        B.attention_split(tq[a:b], tk, tvt, part, heads, 3, n_kv=n_kv)
        torch.cuda.synchronize()
        assert torch.equal(part.cpu().view(torch.int16), full[a:b].cpu().view(torch.int16)), (a, b)


def test_attention_overflowing_logits():
    # one key tile whose logits exceed the first tile's max by hundreds of
    # log2 units: its exponentials overflow fp32 (inf), which must move the
    # running max (the sum test is false for inf), not reach O; and a first
    # tile far above the rest, whose later exponentials underflow to zero
    n_q, n_kv, heads, dh = 96, 640, 2, 128
    q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", n_q, n_kv, heads, dh, 17, scale=3.0)
    for hot in (5, 0):
        k2 = k.copy()
        k2[64 * hot:64 * hot + 64] *= 20.0
        k2 = bf16_round(k2)
        moves = _moves_after_first_tile(q, k2, heads, dh)
        if hot:
            assert (moves > 0).all()
        out = torch.empty(n_q, heads * dh, dtype=tdt, device=DEV)
        B.attention(tq, _bf16(k2), tvt, out, heads, n_kv=n_kv)
        ref = O.attention(q, k2, v, heads)
        got = to_f64(out)
        assert np.isfinite(got).all(), hot
        assert rel_l2(got, ref) <= 1e-2, hot


@pytest.mark.parametrize("dtype,heads,dh,n_q,n_kv,splits", [
    ("bf16", 3, 128, 300, 1000, 4), ("bf16", 2, 128, 129, 64, 4), ("bf16", 2, 64, 257, 333, 3),
    ("bf16", 2, 128, 70, 200, 7), ("f32", 4, 64, 300, 1000, 4), ("f32", 2, 128, 70, 200, 2), ("f32", 2, 64, 5, 7, 8)])
def test_attention_split_matches_oracle(dtype, heads, dh, n_q, n_kv, splits):
    # each query's keys in contiguous ranges of 64-key tiles, attended
    # separately and merged: the same bars as the unsplit kernel; fewer tiles
    # than ranges fall back to one range per tile (n_kv = 64: one range)
    q, k, v, tq, tk, tvt, tdt = _attn_inputs(dtype, n_q, n_kv, heads, dh, n_q * 5 + n_kv + splits)
    out = torch.empty(n_q, heads * dh, dtype=tdt, device=DEV)
    B.attention_split(tq, tk, tvt, out, heads, splits, n_kv=n_kv)
    ref = O.attention(q, k, v, heads)
    got = to_f64(out)
    if dtype == "f32":
        assert max_abs(got, ref) <= 1e-5 * max(1.0, np.abs(ref).max())
    else:
        assert rel_l2(got, ref) <= 1e-2
        assert max_abs(got, ref) <= 2e-2 * max(np.abs(ref).max(), 1e-3)
        assert rel_l2(got, ref) <= 2 * rel_l2(bf16_round(ref), ref) + 4e-3
    one = torch.empty_like(out)
    B.attention_split(tq, tk, tvt, one, heads, 1, n_kv=n_kv)
    plain = torch.empty_like(out)
    B.attention(tq, tk, tvt, plain, heads, n_kv=n_kv)
    torch.cuda.synchronize()
    assert torch.equal(one.cpu(), plain.cpu())  # one range is the unsplit kernel


@pytest.mark.parametrize("dh,n_q,n_kv,splits", [(128, 300, 1000, 1), (64, 257, 333, 1), (128, 70, 700, 3),
                                                 (64, 33, 130, 2), (128, 1, 1, 1)])
def test_attention_identical_keys_return_v_exactly(dh, n_q, n_kv, splits):
    # Every key row equal and every value row equal: all of a query's scores
    # are equal, so each P is exp2 of at most the rounding error of one score
    # times the scale and rounds to exactly 1 in bf16; the row sum is the key
    # count, and O = (count * v) / count = v, exact in fp32 (v has 8
    # significant bits, the count at most 10). So the output holds v's bits
    # for every query, also with a ragged last tile (its masked keys give P = 0)
    # and with key ranges merged (every range has the same max, weight 1).
    heads = 2
    d = heads * dh
    rng = _rng(n_q * 3 + n_kv + dh + splits)
    q = bf16_round(rng.standard_normal((n_q, d)))
    k1, v1 = (bf16_round(rng.standard_normal((1, d))) for _ in range(2))
    k, v = np.repeat(k1, n_kv, axis=0), np.repeat(v1, n_kv, axis=0)
    ld_vt = (n_kv + 63) // 64 * 64
    vt = torch.zeros(d, ld_vt, dtype=torch.bfloat16, device=DEV)
    vt[:, :n_kv] = _bf16(v).T
    out = torch.empty(n_q, d, dtype=torch.bfloat16, device=DEV)
    if splits == 1:
        B.attention(_bf16(q), _bf16(k), vt, out, heads, n_kv=n_kv)
    else:
        B.attention_split(_bf16(q), _bf16(k), vt, out, heads, splits, n_kv=n_kv)
    torch.cuda.synchronize()
    want = np.repeat(v1, n_q, axis=0)
    assert torch.equal(out.cpu(), _bf16(want).cpu())
    assert max_abs(O.attention(q, k, v, heads), want) <= 1e-12  # the textbook result


@pytest.mark.parametrize("dh,n_q,n_kv,splits", [(64, 300, 1000, 1), (128, 70, 200, 1), (64, 33, 130, 3)])
def test_attention_identical_keys_return_v_f32(dh, n_q, n_kv, splits):
    # The same closed form through the fp32 kernel. Its P is exp2 of at most
    # the rounding error of one score times the scale, so 1 to within a few
    # units of 2^-24, but v has 24 significant bits and the n_kv products p*v
    # and the n_kv terms of the row sum are rounded as they accumulate: O is v
    # to within 2 * n_kv * 2^-24 relative. A row sum off by one key, or a
    # masked key counted, would miss by 1/n_kv, far above that.
    heads = 2
    d = heads * dh
    rng = _rng(n_q * 5 + n_kv + dh + splits)
    q = rng.standard_normal((n_q, d)).astype(np.float32).astype(np.float64)
    k1, v1 = (rng.standard_normal((1, d)).astype(np.float32).astype(np.float64) for _ in range(2))
    k, v = np.repeat(k1, n_kv, axis=0), np.repeat(v1, n_kv, axis=0)
    ld_vt = (n_kv + 63) // 64 * 64
    vt = torch.zeros(d, ld_vt, dtype=torch.float32, device=DEV)
    vt[:, :n_kv] = torch.from_numpy(v.astype(np.float32)).to(DEV).T
    tq, tk = (torch.from_numpy(t.astype(np.float32)).to(DEV) for t in (q, k))
    out = torch.empty(n_q, d, dtype=torch.float32, device=DEV)
    if splits == 1:
        B.attention(tq, tk, vt, out, heads, n_kv=n_kv)
    else:
        B.attention_split(tq, tk, vt, out, heads, splits, n_kv=n_kv)
    got = to_f64(out)
    want = np.repeat(v1, n_q, axis=0)
    assert np.all(np.abs(got - want) <= 2.0 * n_kv * 2.0 ** -24 * np.abs(want) + 1e-30)


@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_attention_split_query_slices_bit_identical(scale):
    # with the key cut fixed by n_kv and the range count, a query's bits do not
    # depend on the other queries of the call (slices at any offset), also
    # with near one-hot softmax, and the ragged last range holds the ragged tile
    n_q, n_kv = 300, 1000
    q, k, v, tq, tk, tvt, tdt = _attn_inputs("bf16", n_q, n_kv, 2, 128, 9, scale=scale)
    full = torch.empty(n_q, 256, dtype=tdt, device=DEV)
    B.attention_split(tq, tk, tvt, full, 2, 4, n_kv=n_kv)
    assert rel_l2(to_f64(full), O.attention(q, k, v, 2)) <= 1e-2
    for a, b in ((0, 1), (1, 130), (33, 97), (77, 300), (255, 300)):
        part = torch.empty(b - a, 256, dtype=tdt, device=DEV)
        B.attention_split(tq[a:b], tk, tvt, part, 2, 4, n_kv=n_kv)
        torch.cuda.synchronize()
        assert torch.equal(part.cpu().view(torch.int16), full[a:b].cpu().view(torch.int16)), (a, b)


@pytest.mark.parametrize("dtype,heads,dh,rows", [("bf16", 40, 128, 300), ("bf16", 4, 64, 77), ("f32", 4, 64, 130),
                                                 ("f32", 2, 128, 33)])
@pytest.mark.parametrize("mode", ["norm", "rope", "both"])
def test_qk_transform(dtype, heads, dh, rows, mode):
    rng = _rng(rows + dh)
    d = heads * dh
    t = rng.standard_normal((rows, d)) * 1.5
    wv = (1.0 + 0.1 * rng.standard_normal(dh)).astype(np.float32)
    cos, sin = synth.rope_tables(rows, dh, offset=1000)
    if dtype == "f32":
        t = t.astype(np.float32).astype(np.float64)
        x = torch.from_numpy(t.astype(np.float32)).to(DEV)
    else:
        t = bf16_round(t)
        x = _bf16(t)
    use_norm = mode in ("norm", "both")
    use_rope = mode in ("rope", "both")
    B.qk_transform(x, heads, torch.from_numpy(wv).to(DEV) if use_norm else None,
                   (torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV)) if use_rope else None)
    ref = O.qk_transform(t, wv.astype(np.float64) if use_norm else None, cos if use_rope else None,
                         sin if use_rope else None, heads, 1e-6)
    got = to_f64(x)
    tol = 1e-5 if dtype == "f32" else 2.0 ** -8
    assert np.all(np.abs(got - ref) <= np.abs(ref) * tol + tol * 1e-2 * np.abs(ref).max())


def test_attention_query_independent_of_wave_mates_with_moving_maxima():
    # Q, K and V^T of an int8-weight block (d = 4096, 32 heads x 128, 1024
    # tokens) through the step kernels: per-head logits reach tens of units.
    # A query's O must not depend on the queries that share its wavefront:
    # slices starting at offsets that are not multiples of 32, and single
    # rows, must give the bits of the full launch. (Under the earlier move bar
    # of 2^16 these logits moved running maxima in later tiles, and with the
    # second exponentiation compiled differently from the first, query 296 of
    # head 23 did not; under the 2^64 bar moves are exercised by
    # test_attention_moving_maxima.)
    shape = synth.BlockShape("att-mates", 4096, 32, 128, 2048, 1024, "w8_bf16")
    inp = synth.make_inputs(shape, 0)
    t = {k: B.tensor_from_stored(v, DEV) for k, v in inp.items()}
    n, d = shape.n_tokens, shape.d
    w, sc = t["w_qkv"], t["s_qkv"]
    n1 = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    B.modnorm(t["x"], t["mod"][0], t["mod"][1], n1)
    q = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    vt = torch.zeros(d, n, dtype=torch.bfloat16, device=DEV)
    B.linear("w8_bf16", "store", n1, w[:d], q, d, w_scale=sc[:d])
    B.linear("w8_bf16", "store", n1, w[d:2 * d], k, d, w_scale=sc[d:2 * d])
    B.linear("w8_bf16", "store_t", n1, w[2 * d:], vt, d, w_scale=sc[2 * d:])
    full = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    B.attention(q, k, vt, full, shape.n_heads)
    for s0, c in ((0, 300), (300, 300), (600, 300), (200, 100), (5, 1019), (296, 1), (567, 1)):
        part = torch.empty(c, d, dtype=torch.bfloat16, device=DEV)
        B.attention(q[s0:s0 + c].contiguous(), k, vt, part, shape.n_heads)
        torch.cuda.synchronize()
        assert torch.equal(part.cpu(), full[s0:s0 + c].cpu()), (s0, c)
