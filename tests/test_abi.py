"""The C-ABI library on the host: it loads, exports every declared symbol,
and validates arguments before touching the GPU (CPU only)."""
import ctypes
import os
import re

import pytest

from memory_bounded_chunked_amd import block as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.listdir(os.path.join(ROOT, "include")))


def _declared():
    names = set()
    for h in HEADERS:
        src = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"^(?:const\s+)?\w+\*?\s+\*?(dit_\w+)\(", src, flags=re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"dit_block_create", "dit_block_forward", "dit_block_peak_workspace",
            "dit_modnorm", "dit_attention", "dit_linear", "dit_profile_read"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(B.EXPORTS)


def _handle(lib, d=256, heads=2, hd=128, ffn=512, dtype=1, eps=1e-6, wptr=0x10000, scales=True):
    desc = B._Desc(d, heads, hd, ffn, dtype, eps)
    s = wptr if scales else 0
    w = B._Weights(wptr, wptr, wptr, wptr, s, s, s, s)
    h = ctypes.c_void_p()
    rc = lib.dit_block_create(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(h))
    return rc, h


def test_create_validation(lib):
    rc, h = _handle(lib)
    assert rc == B.DIT_OK and h.value
    lib.dit_block_destroy(h)
    bad = [dict(d=250), dict(hd=96, d=192, heads=2), dict(ffn=100), dict(ffn=0), dict(dtype=7),
           dict(eps=0.0), dict(wptr=0x10008), dict(wptr=0), dict(dtype=2, scales=False), dict(d=16384, heads=128)]
    for kw in bad:
        rc, _ = _handle(lib, **kw)
        assert rc == B.DIT_EINVAL, kw


def _ws(lib, h, n, ca, cm, fc):
    out = ctypes.c_size_t()
    rc = lib.dit_block_peak_workspace(h, n, ca, cm, fc, ctypes.byref(out))
    return rc, out.value


def _closed_form(n, d, ffn, e, ca, cm, fc):
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    ca = n if ca == 0 else min(ca, n)
    cm = min(cm, n)
    fc = ffn if fc == 0 else min(fc, ffn)
    s = max(ca, cm)
    np_ = (n + 63) // 64 * 64
    return (r(n * d * e) + r(d * np_ * e) + r(s * d * 4)
            + max(2 * r(ca * d * e), r(cm * d * e) + r(cm * fc * e)))


@pytest.mark.parametrize("n,ca,cm,fc", [(1000, 256, 256, 0), (1000, 0, 1000, 0), (777, 100, 300, 128),
                                        (5, 8192, 8192, 0), (32768, 8192, 8192, 0), (131072, 8192, 8192, 3456)])
def test_workspace_closed_form(lib, n, ca, cm, fc):
    for dtype, e in ((1, 2), (0, 4), (2, 2)):
        d, ffn = (5120, 13824) if n >= 32768 else (256, 1024)
        rc, h = _handle(lib, d=d, heads=d // 128, ffn=ffn, dtype=dtype)
        assert rc == 0
        rc, ws = _ws(lib, h, n, ca, cm, fc)
        assert rc == 0 and ws == _closed_form(n, d, ffn, e, ca, cm, fc)
        lib.dit_block_destroy(h)


def test_token_count_limit_of_the_attention_offsets(lib):
    # bf16, head_dim 128: 128 * Np * 2 bytes must stay below 2^32
    rc, h = _handle(lib)
    assert rc == B.DIT_OK
    try:
        assert _ws(lib, h, (1 << 24) - 64, 256, 256, 0)[0] == B.DIT_OK
        assert _ws(lib, h, (1 << 24) - 63, 256, 256, 0)[0] == B.DIT_EINVAL
    finally:
        lib.dit_block_destroy(h)


def test_weight_size_limit_of_the_projection_offsets(lib):
    # one gate/up tile spans rows f .. f + F + 255 of the [2F][d] weight, addressed
    # with 32-bit byte offsets: (F + 256) * d * (weight bytes) must stay below 2^32
    for dtype, wb in ((1, 2), (0, 4), (2, 1)):
        f_max = (1 << 32) // (8192 * wb) - 256  # first F whose span reaches 2^32
        f_ok = f_max - 64 if f_max % 64 == 0 else f_max // 64 * 64
        rc, h = _handle(lib, d=8192, heads=64, ffn=f_ok, dtype=dtype)
        assert rc == B.DIT_OK, (dtype, f_ok)
        lib.dit_block_destroy(h)
        rc, _ = _handle(lib, d=8192, heads=64, ffn=(f_max + 63) // 64 * 64, dtype=dtype)
        assert rc == B.DIT_EINVAL, dtype


def test_workspace_figures_at_32k():
    # headline block (d=5120, F=13824, N=32768, chunks 8192/8192): K,V 640 MiB,
    # fp32 staging 160 MiB, slabs max(160, 296) MiB -> 1096 MiB; only K/V grow with N
    assert _closed_form(32768, 5120, 13824, 2, 8192, 8192, 0) == 1096 * 2 ** 20
    assert _closed_form(32768, 5120, 13824, 2, 0, 32768, 0) == 2464 * 2 ** 20
    grow = _closed_form(65536, 5120, 13824, 2, 8192, 8192, 0) - _closed_form(32768, 5120, 13824, 2, 8192, 8192, 0)
    assert grow == 2 * 32768 * 5120 * 2


def test_forward_rejects_before_launch(lib):
    rc, h = _handle(lib)
    assert rc == 0
    _, need = _ws(lib, h, 1000, 256, 256, 0)
    x, mod, ws = 0x20000, 0x30000, 0x40000
    f = lib.dit_block_forward
    cases = [
        ((None, x, mod, 1000, 256, 256, 0, ws, need, None), B.DIT_EINVAL),
        ((h, None, mod, 1000, 256, 256, 0, ws, need, None), B.DIT_EINVAL),
        ((h, x, None, 1000, 256, 256, 0, ws, need, None), B.DIT_EINVAL),
        ((h, x, mod, 0, 256, 256, 0, ws, need, None), B.DIT_EINVAL),
        ((h, x, mod, 1000, -1, 256, 0, ws, need, None), B.DIT_EINVAL),
        ((h, x, mod, 1000, 256, 0, 0, ws, need, None), B.DIT_EINVAL),
        ((h, x, mod, 1000, 256, 256, 100, ws, need, None), B.DIT_EINVAL),
        ((h, x, mod, 1000, 256, 256, -64, ws, need, None), B.DIT_EINVAL),
        ((h, x + 2, mod, 1000, 256, 256, 0, ws, need, None), B.DIT_EINVAL),
        ((h, x, mod, 1000, 256, 256, 0, ws + 8, need, None), B.DIT_EINVAL),
        ((h, x, mod, 1000, 256, 256, 0, None, need, None), B.DIT_EINVAL),
        ((h, x, mod, 1000, 256, 256, 0, ws, need - 1, None), B.DIT_ENOSPC),
        ((h, x, mod, 1000, 256, 256, 0, ws, 0, None), B.DIT_ENOSPC),
    ]
    for args, want in cases:
        assert f(*args) == want, args
    lib.dit_block_destroy(h)


def test_noalloc_forward_rejects_before_any_device_call(lib):
    # argument errors and sizes beyond the static workspace are host decisions:
    # they return before the entry point looks up its device buffer
    rc, h = _handle(lib)
    assert rc == 0
    x, mod = 0x20000, 0x30000
    f = lib.dit_block_forward_noalloc
    assert f(None, x, mod, None, None, 1000, 256, 256, 0, None) == B.DIT_EINVAL
    assert f(h, x, mod, None, None, 0, 256, 256, 0, None) == B.DIT_EINVAL
    assert f(h, x, mod, None, None, 1000, 256, 0, 0, None) == B.DIT_EINVAL
    assert f(h, x, mod, None, None, 1000, 256, 256, 100, None) == B.DIT_EINVAL
    n_big = 1 << 17  # d=256 bf16: global K and V alone are 128 MiB
    _, need = _ws(lib, h, n_big, 8192, 8192, 0)
    assert need > B.STATIC_WORKSPACE_BYTES
    assert f(h, x, mod, None, None, n_big, 8192, 8192, 0, None) == B.DIT_ETOOBIG
    assert B.STATIC_WORKSPACE_BYTES == 64 << 20
    lib.dit_block_destroy(h)


def test_attention_splits_workspace_and_validation(lib):
    rc, h = _handle(lib)
    assert rc == 0
    for bad in (0, -1, 65):
        assert lib.dit_block_set_attention_splits(h, bad) == B.DIT_EINVAL
    n, ca, cm, d, heads = 1000, 256, 256, 256, 2
    _, base = _ws(lib, h, n, ca, cm, 0)
    assert base == _closed_form(n, d, 512, 2, ca, cm, 0)
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    for splits, eff in ((1, 1), (4, 4), (64, 16)):  # at most one range per 64-key tile (ceil(1000/64) = 16)
        assert lib.dit_block_set_attention_splits(h, splits) == 0
        _, ws = _ws(lib, h, n, ca, cm, 0)
        extra = 0 if eff == 1 else r(eff * ca * d * 4) + r(eff * ca * heads * 2 * 4)
        assert ws == base + extra, splits
        out = ctypes.c_size_t()
        assert lib.dit_attention_split_workspace(ca, n, heads, 128, splits, ctypes.byref(out)) == 0
        assert out.value == extra
    lib.dit_block_destroy(h)
    p = 0x10000
    f = lib.dit_attention_split
    assert f(1, p, 256, p, 256, p, 1000, p, 256, 10, 1000, 2, 128, 0, p, 1 << 20, None) == B.DIT_EINVAL
    assert f(1, p, 256, p, 256, p, 1000, p, 256, 10, 1000, 2, 128, 4, p, 100, None) == B.DIT_ENOSPC
    assert f(1, p, 256, p, 256, p, 1000, p, 256, 10, 1000, 2, 128, 4, p + 8, 1 << 20, None) == B.DIT_EINVAL
    assert f(1, p, 256, p, 256, p, 1000, p, 256, 0, 1000, 2, 128, 4, p, 1 << 20, None) == B.DIT_OK


def test_step_entry_points_reject_before_launch(lib):
    p = 0x10000
    assert lib.dit_modnorm(1, 1, p, 256, p, p, p, 256, 10, 250, 1e-6, None) == B.DIT_EINVAL
    assert lib.dit_modnorm(1, 3, p, 256, p, p, p, 256, 10, 256, 1e-6, None) == B.DIT_EINVAL
    assert lib.dit_modnorm(1, 1, p, 128, p, p, p, 256, 10, 256, 1e-6, None) == B.DIT_EINVAL
    assert lib.dit_modnorm(1, 1, p, 256, p, p, p, 256, 0, 256, 1e-6, None) == B.DIT_OK  # nothing to do
    assert lib.dit_attention(1, p, 256, p, 256, p, 64, p, 256, 10, 0, 2, 128, None) == B.DIT_EINVAL
    assert lib.dit_attention(1, p, 256, p, 256, p, 64, p, 256, 10, 100, 2, 128, None) == B.DIT_EINVAL
    assert lib.dit_attention(1, p, 256, p, 256, p, 104, p, 256, 10, 100, 2, 96, None) == B.DIT_EINVAL
    assert lib.dit_attention(2, p, 256, p, 256, p, 104, p, 256, 10, 100, 2, 128, None) == B.DIT_EINVAL
    assert lib.dit_attention(1, p, 256, p, 256, p, 104, p, 256, 0, 100, 2, 128, None) == B.DIT_OK
    # 32-bit offsets within a head's V^T rows: head_dim * ldvt * element bytes < 2^32
    assert lib.dit_attention(1, p, 256, p, 256, p, 1 << 24, p, 256, 0, 100, 2, 128, None) == B.DIT_EINVAL
    assert lib.dit_attention(1, p, 256, p, 256, p, (1 << 24) - 8, p, 256, 0, 100, 2, 128, None) == B.DIT_OK
    assert lib.dit_attention(0, p, 256, p, 256, p, 1 << 23, p, 256, 0, 100, 2, 128, None) == B.DIT_EINVAL
    # dit_linear: k not a multiple of 64, n not a multiple of 64, int8 without scale, missing gate
    assert lib.dit_linear(1, 0, p, 256, p, 256, None, 0, 10, 256, 100, p, 256, None, 0, None, None) == B.DIT_EINVAL
    assert lib.dit_linear(1, 0, p, 256, p, 256, None, 0, 10, 200, 256, p, 256, None, 0, None, None) == B.DIT_EINVAL
    assert lib.dit_linear(2, 0, p, 256, p, 256, None, 0, 10, 256, 256, p, 256, None, 0, None, None) == B.DIT_EINVAL
    assert lib.dit_linear(1, 2, p, 256, p, 256, None, 0, 10, 256, 256, p, 256, p, 256, None, None) == B.DIT_EINVAL
    assert lib.dit_linear(1, 3, p, 256, p, 256, None, 100, 10, 256, 256, p, 256, None, 0, None, None) == B.DIT_EINVAL
    assert lib.dit_linear(1, 0, p, 256, p, 256, None, 0, 0, 256, 256, p, 256, None, 0, None, None) == B.DIT_OK
    # dit_linear: 32-bit tile offsets, 256 * lda * 2 and R * ldw * (weight bytes) below 2^32
    big = 1 << 23
    assert lib.dit_linear(1, 0, p, big - 8, p, 256, None, 0, 0, 256, 256, p, 256, None, 0, None, None) == B.DIT_OK
    assert lib.dit_linear(1, 0, p, big, p, 256, None, 0, 0, 256, 256, p, 256, None, 0, None, None) == B.DIT_EINVAL
    assert lib.dit_linear(1, 0, p, 256, p, big, None, 0, 0, 256, 256, p, 256, None, 0, None, None) == B.DIT_EINVAL
    assert lib.dit_linear(2, 0, p, 256, p, big, p, 0, 0, 256, 256, p, 256, None, 0, None, None) == B.DIT_OK
    up = (1 << 32) // (8192 * 2) - 256  # gate/up span (up_offset + 256) rows of 8192 bf16
    assert lib.dit_linear(1, 3, p, 8192, p, 8192, None, up - 8, 0, 256, 256, p, 256, None, 0, None, None) == B.DIT_OK
    assert lib.dit_linear(1, 3, p, 8192, p, 8192, None, up, 0, 256, 256, p, 256, None, 0, None, None) == B.DIT_EINVAL


def test_final_layer_rejects_before_launch(lib):
    p = 0x10000
    fl = lib.dit_final_layer
    # (dtype, x, ldx, n, d, shift, scale, w, out_dim, out, ldo, eps)
    ok = (1, p, 256, 10, 256, p, p, p, 64, p, 64, 1e-6)
    assert fl(*ok[:3], 0, *ok[4:], None) == B.DIT_OK  # no rows: nothing enqueued
    assert fl(1, None, 256, 0, 256, p, p, p, 64, None, 64, 1e-6, None) == B.DIT_OK  # empty range, NULL rows
    bad = [
        (2,) + ok[1:],                       # int8 activations are not an input type of the head
        ok[:1] + (None,) + ok[2:],           # null x
        ok[:9] + (None,) + ok[10:],          # null out
        ok[:5] + (None,) + ok[6:],           # null shift
        ok[:2] + (200,) + ok[3:],            # ldx < d
        ok[:3] + (-1,) + ok[4:],             # negative n
        ok[:4] + (96,) + ok[5:],             # d not a multiple of 64
        ok[:4] + (8256,) + ok[5:],           # d above 8192
        ok[:8] + (0,) + ok[9:],              # out_dim 0
        ok[:8] + (129,) + ok[9:],            # out_dim above 128
        ok[:10] + (63,) + ok[11:],           # ldo < out_dim
        ok[:11] + (0.0,),                    # eps
        ok[:7] + (p + 4,) + ok[8:],          # w_out not 16-byte aligned
        ok[:9] + (p + 2,) + ok[10:],         # out not 4-byte aligned
    ]
    for args in bad:
        assert fl(*args, None) == B.DIT_EINVAL, args


def test_profile_read_without_records(lib):
    assert lib.dit_profile_enable(1) == 0
    t, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.dit_profile_read(3, ctypes.byref(t), ctypes.byref(n)) == 0 and n.value == 0
    assert lib.dit_profile_read(len(B.PROFILE_KINDS), ctypes.byref(t), ctypes.byref(n)) == B.DIT_EINVAL
    assert lib.dit_profile_enable(0) == 0


def test_strerror(lib):
    assert B.strerror(B.DIT_ENOSPC) == "workspace too small"
    assert B.strerror(B.DIT_EINVAL) == "invalid argument"


def test_defaults_follow_the_pages():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "chunk_knobs.json")))
    assert B.DEFAULT_ATTN_CHUNK == g["attn_chunk_tokens"]["default"]
    assert B.DEFAULT_MLP_CHUNK == g["mlp_chunk_tokens"]["default"]


def _plan(lib, h, n, budget):
    a, m, f = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib.dit_block_plan_chunks(h, n, budget, ctypes.byref(a), ctypes.byref(m), ctypes.byref(f))
    return rc, a.value, m.value, f.value


@pytest.mark.parametrize("n,dtype", [(32768, 1), (131072, 1), (65536, 2), (1000, 0)])
def test_plan_chunks_fits_and_is_maximal(lib, n, dtype):
    d, ffn = (256, 1024) if n == 1000 else (5120, 13824)
    rc, h = _handle(lib, d=d, heads=d // 128, ffn=ffn, dtype=dtype)
    assert rc == 0
    e = 4 if dtype == 0 else 2
    kv = _closed_form(n, d, ffn, e, n, 1, 64) - (n * d * 4) - max(2 * n * d * e, d * e + 64 * e)
    for extra_mib in (1, 64, 300, 1200, 4000, 100000):
        budget = kv + extra_mib * 2 ** 20
        rc, ca, cm, fc = _plan(lib, h, n, budget)
        if rc == B.DIT_ENOSPC:
            # not even a 256-token chunk at the narrowest candidate feature width fits
            fc_min = ffn
            while fc_min % 128 == 0 and (fc_min // 2) % 64 == 0:
                fc_min //= 2
            assert _ws(lib, h, n, min(256, n), min(256, n), fc_min)[1] > budget
            continue
        assert rc == 0
        c = n if ca == 0 else ca
        assert cm == c and (c == n or c % 256 == 0)
        rc, ws = _ws(lib, h, n, ca, cm, fc)
        assert rc == 0 and ws <= budget
        if c < n:  # one more step of 256 tokens does not fit at any candidate feature width
            for f2 in (0, ffn // 2, ffn // 4, ffn // 8):
                if f2 and f2 % 64:
                    continue
                nxt = min(n, c + 256)
                assert _ws(lib, h, n, 0 if nxt == n else nxt, nxt, f2)[1] > budget
    # a budget below the global K/V floor is refused
    assert _plan(lib, h, n, kv // 2)[0] == B.DIT_ENOSPC
    # ample memory: one slice of all tokens, no feature slicing
    assert _plan(lib, h, n, 1 << 50)[1:] == (0, n, 0)
    lib.dit_block_destroy(h)


def test_plan_chunks_rejects(lib):
    rc, h = _handle(lib)
    a = ctypes.c_int64()
    assert lib.dit_block_plan_chunks(h, 0, 1 << 30, ctypes.byref(a), ctypes.byref(a), ctypes.byref(a)) == B.DIT_EINVAL
    assert lib.dit_block_plan_chunks(None, 10, 1 << 30, ctypes.byref(a), ctypes.byref(a), ctypes.byref(a)) == B.DIT_EINVAL
    lib.dit_block_destroy(h)


def _lora_struct(ranks, ptr=0x10000, alpha=0.5):
    st = B._BlockLora()
    for name, r in ranks.items():
        setattr(st, name, B._Lora(ptr if r else 0, ptr if r else 0, r, alpha))
    return st


def test_set_lora_validation(lib):
    rc, h = _handle(lib)
    assert rc == 0
    try:
        ok = _lora_struct({"q": 16, "k": 32, "gate": 64, "down": 256})
        assert lib.dit_block_set_lora(h, ctypes.byref(ok)) == B.DIT_OK
        assert lib.dit_block_set_lora(h, None) == B.DIT_OK
        for bad in ({"q": 8}, {"v": 272}, {"o": -16}, {"up": 17}):
            assert lib.dit_block_set_lora(h, ctypes.byref(_lora_struct(bad))) == B.DIT_EINVAL, bad
        assert lib.dit_block_set_lora(h, ctypes.byref(_lora_struct({"q": 16}, ptr=0x10008))) == B.DIT_EINVAL
        assert lib.dit_block_set_lora(h, ctypes.byref(_lora_struct({"q": 16}, alpha=float("nan")))) == B.DIT_EINVAL
        null = B._BlockLora()
        null.k = B._Lora(0x10000, 0, 16, 1.0)  # B missing
        assert lib.dit_block_set_lora(h, ctypes.byref(null)) == B.DIT_EINVAL
        assert lib.dit_block_set_lora(None, ctypes.byref(ok)) == B.DIT_EINVAL
    finally:
        lib.dit_block_destroy(h)


@pytest.mark.parametrize("n,ca,cm,fc", [(1000, 256, 256, 0), (777, 100, 300, 128), (32768, 8192, 8192, 0)])
def test_workspace_closed_form_with_adapters(lib, n, ca, cm, fc):
    ranks = {"q": 16, "k": 32, "v": 48, "o": 64, "gate": 16, "up": 32, "down": 128}
    d, ffn = (5120, 13824) if n >= 32768 else (256, 1024)
    rc, h = _handle(lib, d=d, heads=d // 128, ffn=ffn, dtype=1)
    assert rc == 0
    try:
        base = _ws(lib, h, n, ca, cm, fc)[1]
        assert lib.dit_block_set_lora(h, ctypes.byref(_lora_struct(ranks))) == B.DIT_OK
        rc, got = _ws(lib, h, n, ca, cm, fc)
        assert rc == 0
        a = n if ca == 0 else min(ca, n)
        m = min(cm, n)
        t = 4 * max(a * max(ranks["k"] + ranks["v"], ranks["q"], ranks["o"]),
                    m * (ranks["gate"] + ranks["up"] + ranks["down"]))
        assert got == base + (t + 255) // 256 * 256
        assert lib.dit_block_set_lora(h, None) == B.DIT_OK
        assert _ws(lib, h, n, ca, cm, fc)[1] == base
    finally:
        lib.dit_block_destroy(h)
