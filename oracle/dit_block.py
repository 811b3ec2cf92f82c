"""fp64 CPU oracle for the forward pass of one token-chunked DiT transformer block.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it. It shares no code with the HIP library.

What it computes is the plain definition of the block that the pages chunk:

* "LayerStream: H3 Chunking" (comfy.icu/node/LayerStreamH3Chunking), section
  "How the slicing works": norms, modulation, the projections and the MLP are
  token-wise and add into the residual stream; attention needs every key and
  value for every query.
* "Proposal: Generic memory-aware streaming execution for transformer models"
  (github.com/Comfy-Org/ComfyUI/discussions/15920), sections "MLP planning" and
  "Attention requires a stronger contract": a gated MLP followed by a linear
  down projection, and attention over global K/V.

Readings the pages leave open (each also listed in the design notes):
LayerNorm without its own affine, biased variance, eps = 1e-6; DiT adaLN
modulation ``norm * (1 + scale) + shift`` and a ``gate`` multiplying each
branch before its residual add; no biases, no QK-norm, no positional transform,
no mask; head h owns columns [h*dh, (h+1)*dh) of Q, K and V; scale 1/sqrt(dh);
SwiGLU = silu(gate) * up with gate rows [0, F) and up rows [F, 2F) of ``w_gu``.

Optional activation-space adapters ("ComfyUI-StaticPipeline", section
"Activation-space LoRA (bypass mode)"): a projection y = W a becomes
y = W a + alpha * B (A a) on any of q, k, v, o, gate, up and down, without
touching W. Pinned against the same block with merged weights W + alpha B A.

Everything is fp64. A library matmul (numpy/OpenBLAS) serves as the matrix
product step. Parity of every function here is pinned by the CPU tests
(brute force, torch fp64 library routines, closed forms and invariants).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "layer_norm", "modulate", "linear", "silu", "attention", "dequantize_rows",
    "rms_norm_heads", "rope", "qk_transform", "final_layer", "final_layer_chunked",
    "lora_delta", "lora_f64", "block_weights_f64", "block_forward", "block_forward_chunked", "global_kv",
    "block_rows",
]

# Projections an adapter can attach to, in the block's own names.
LORA_TARGETS = ("q", "k", "v", "o", "gate", "up", "down")

# The matrix-product step. Every product in this module goes through this one
# name, so a test can substitute an order-stable product.
matmul = np.matmul

# Query rows per group when materialising scores: each query row's softmax is
# independent of every other row, so rows are handled a group at a time only
# to bound host memory.
_SCORE_ELEMS = 1 << 25


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """Per token row: (x - mean) / sqrt(biased variance + eps); no affine.

    The block's normalisation, applied per token ("How the slicing works";
    "How it works", step 1, of the H3 MultiStream page). Two-pass statistics.
    """
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(nrm: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """adaLN modulation of a normalised row: nrm * (1 + scale) + shift."""
    return nrm * (1.0 + scale) + shift


def linear(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """a [T, in] times w [out, in] transposed: y[t, o] = sum_i a[t, i] * w[o, i]."""
    return matmul(a, w.T)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int) -> np.ndarray:
    """Bidirectional multi-head softmax attention, exact two-pass softmax.

    For each head h and query row i:
        s_ij = <q_i^h, k_j^h> / sqrt(dh)         for every key j,
        p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij),
        o_i^h = sum_j p_ij v_j^h.
    Every query sees every key ("How the slicing works": attention is not
    token-wise). ``q`` may hold any subset of query rows; ``k`` and ``v`` hold
    all N keys.
    """
    t, d = q.shape
    dh = d // n_heads
    out = np.empty((t, d), dtype=np.float64)
    rows = max(1, _SCORE_ELEMS // max(1, k.shape[0]))
    inv = 1.0 / np.sqrt(dh)
    for h in range(n_heads):
        c = slice(h * dh, (h + 1) * dh)
        kh_t = np.ascontiguousarray(k[:, c].T)
        vh = np.ascontiguousarray(v[:, c])
        for r0 in range(0, t, rows):
            r1 = min(t, r0 + rows)
            s = matmul(q[r0:r1, c], kh_t) * inv
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r1, c] = matmul(p, vh)
    return out


def rms_norm_heads(t: np.ndarray, w: np.ndarray, n_heads: int, eps: float) -> np.ndarray:
    """Per token and head: t_h / sqrt(mean(t_h^2) + eps) * w, w of length dh.

    The optional Q/K normalization step of the streamed-Q plan (streaming
    proposal, "Attention requires a stronger contract": apply the model's Q
    normalization/positional transform to each bounded Q region).
    """
    n, d = t.shape
    dh = d // n_heads
    th = t.reshape(n, n_heads, dh)
    ms = (th ** 2).mean(axis=2, keepdims=True)
    return (th / np.sqrt(ms + eps) * np.asarray(w, np.float64)).reshape(n, d)


def rope(t: np.ndarray, cos: np.ndarray, sin: np.ndarray, n_heads: int) -> np.ndarray:
    """Rotary positional transform on adjacent pairs of every head.

    For token i and pair j of a head: (a, b) = (t[2j], t[2j+1]) becomes
    (a cos_ij - b sin_ij, a sin_ij + b cos_ij); ``cos``/``sin`` are [N, dh/2],
    shared by all heads (the "positional encoding/RoPE step" of the same plan).
    """
    n, d = t.shape
    dh = d // n_heads
    th = t.reshape(n, n_heads, dh // 2, 2)
    a, b = th[..., 0], th[..., 1]
    c = np.asarray(cos, np.float64)[:, None, :]
    s = np.asarray(sin, np.float64)[:, None, :]
    out = np.empty_like(th)
    out[..., 0] = a * c - b * s
    out[..., 1] = a * s + b * c
    return out.reshape(n, d)


def qk_transform(t: np.ndarray, norm_w, cos, sin, n_heads: int, eps: float) -> np.ndarray:
    """RMSNorm (if a weight is given), then RoPE (if tables are given)."""
    if norm_w is not None:
        t = rms_norm_heads(t, norm_w, n_heads, eps)
    if cos is not None:
        t = rope(t, cos, sin, n_heads)
    return t


def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Weight-only int8: W[n, k] = s[n] * q[n, k], one scale per output row.

    The TensorWiseINT8 layout of the Ascend port article (m.qwbw.cn/news/87515,
    section 2.2) keeps one ``weight_scale`` per output row; slicing rows keeps
    the projection exact ("How it works", step 3, of the H3 MultiStream page).
    """
    return np.asarray(s, np.float64)[:, None] * np.asarray(q, np.float64)


def lora_delta(a: np.ndarray, ad) -> np.ndarray:
    """The activation-space adapter term alpha * B (A a) of one projection.

    "ComfyUI-StaticPipeline", section "Activation-space LoRA (bypass mode)":
    the adapter is applied to activations, y = W x + alpha * B (A x), so the
    packed (for example int8) weight W is never rewritten. ``ad`` is
    (A [rank, in], B [out, rank], alpha); None means no adapter (term 0).
    """
    if ad is None:
        return 0.0
    a_mat, b_mat, alpha = ad
    return alpha * linear(linear(a, a_mat), b_mat)


def lora_f64(lora: dict | None) -> dict:
    """fp64 copies of the adapters: {target: (A, B, alpha)} for the targets present."""
    out = {}
    for name, ad in (lora or {}).items():
        if name not in LORA_TARGETS:
            raise ValueError(f"unknown adapter target {name!r}")
        if ad is not None:
            a_mat, b_mat, alpha = ad
            out[name] = (np.asarray(a_mat, np.float64), np.asarray(b_mat, np.float64), float(alpha))
    return out


def _adapter_rows(ad, r0: int, r1: int):
    """The adapter restricted to output rows [r0, r1) (B rows; A unchanged)."""
    return None if ad is None else (ad[0], ad[1][r0:r1], ad[2])


def block_weights_f64(w: dict) -> dict:
    """fp64 weight matrices from already-decoded arrays (dequantising int8 ones)."""
    out = {}
    for name in ("qkv", "o", "gu", "down"):
        m = w["w_" + name]
        if ("s_" + name) in w:
            out[name] = dequantize_rows(m, w["s_" + name])
        else:
            out[name] = np.asarray(m, np.float64)
    return out


def _split(w: dict, d: int):
    wqkv = w["qkv"]
    return wqkv[:d], wqkv[d:2 * d], wqkv[2 * d:3 * d]


def _mlp_hidden(n2: np.ndarray, w: dict, ffn: int, f0: int, f1: int, lora: dict) -> np.ndarray:
    """silu(gate) * up for FFN features [f0, f1), each projection with its adapter."""
    g = linear(n2, w["gu"][f0:f1]) + lora_delta(n2, _adapter_rows(lora.get("gate"), f0, f1))
    u = linear(n2, w["gu"][ffn + f0:ffn + f1]) + lora_delta(n2, _adapter_rows(lora.get("up"), f0, f1))
    return silu(g) * u


def _mlp_delta(n2: np.ndarray, w: dict, ffn: int, f0: int = 0, f1: int | None = None,
               lora: dict | None = None) -> np.ndarray:
    """W_down[:, f0:f1] h[f0:f1] for FFN features [f0, f1), h = silu(gate) * up.

    The down projection's adapter is not included: its A acts on all of h, so
    a feature-sliced schedule accumulates A h over the slices (see
    block_forward_chunked)."""
    f1 = ffn if f1 is None else f1
    return linear(_mlp_hidden(n2, w, ffn, f0, f1, lora or {}), w["down"][:, f0:f1])


def block_forward(x: np.ndarray, mod: np.ndarray, w: dict, n_heads: int,
                  eps: float = 1e-6, want: tuple = (), qk: dict | None = None,
                  lora: dict | None = None) -> np.ndarray | tuple:
    """Unchunked block forward; returns y [N, d] (and the named intermediates).

    n1 = modulate(LN(x); shift1, scale1);  q, k, v = n1 W_{q,k,v}^T
    o  = attention(q, k, v);               x1 = x + gate1 * (o W_o^T)
    n2 = modulate(LN(x1); shift2, scale2); h = silu(n2 W_g^T) * (n2 W_u^T)
    y  = x1 + gate2 * (h W_down^T)
    ``want`` may name any of n1, q, k, v, o, x1, n2, h. ``qk`` optionally holds
    ``q_norm`` / ``k_norm`` ([dh] RMSNorm weights) and ``cos`` / ``sin``
    ([N, dh/2] RoPE tables), applied to q and k before attention. ``lora``
    optionally maps targets q, k, v, o, gate, up, down to adapters (A, B,
    alpha), each adding alpha * B (A a) to its projection of a.
    """
    d = x.shape[1]
    ffn = w["down"].shape[1]
    sh1, sc1, g1, sh2, sc2, g2 = (np.asarray(m, np.float64) for m in mod)
    wq, wk, wv = _split(w, d)
    lo = lora or {}
    n1 = modulate(layer_norm(x, eps), sh1, sc1)
    q = linear(n1, wq) + lora_delta(n1, lo.get("q"))
    k = linear(n1, wk) + lora_delta(n1, lo.get("k"))
    v = linear(n1, wv) + lora_delta(n1, lo.get("v"))
    if qk:
        q = qk_transform(q, qk.get("q_norm"), qk.get("cos"), qk.get("sin"), n_heads, eps)
        k = qk_transform(k, qk.get("k_norm"), qk.get("cos"), qk.get("sin"), n_heads, eps)
    o = attention(q, k, v, n_heads)
    x1 = x + g1 * (linear(o, w["o"]) + lora_delta(o, lo.get("o")))
    n2 = modulate(layer_norm(x1, eps), sh2, sc2)
    h = _mlp_hidden(n2, w, ffn, 0, ffn, lo)
    y = x1 + g2 * (linear(h, w["down"]) + lora_delta(h, lo.get("down")))
    if not want:
        return y
    loc = dict(n1=n1, q=q, k=k, v=v, o=o, x1=x1, n2=n2, h=h)
    return (y,) + tuple(loc[name] for name in want)


def block_forward_chunked(x: np.ndarray, mod: np.ndarray, w: dict, n_heads: int,
                          attn_chunk: int, mlp_chunk: int, ffn_chunk: int = 0,
                          eps: float = 1e-6, qk: dict | None = None, lora: dict | None = None) -> np.ndarray:
    """The pages' two-pass, token-chunked schedule of the same block, in place.

    Follows "How the slicing works" (LayerStream: H3 Chunking) and "Attention
    requires a stronger contract" (streaming proposal):
      pass 1: for each slab of ``attn_chunk`` tokens, norm1 and project K and V
              only, kept for the whole sequence;
      pass 2: for each slice, recompute norm1 and Q, attend the slice against
              the full K/V, out-project, and add the gated result into the
              residual rows of that slice in place;
      MLP:    for each slab of ``mlp_chunk`` tokens, norm2, SwiGLU and add the
              gated result in place; with ``ffn_chunk`` > 0 the FFN features
              are taken a slice at a time and the down-projected partials
              accumulated ("MLP planning"). An adapter on the down projection
              then accumulates its A h over the slices too and applies B once.
    ``attn_chunk`` = 0 means one slice of all N tokens. The input is not
    modified; the returned array is the residual stream after the block.
    """
    n, d = x.shape
    ffn = w["down"].shape[1]
    ca = n if attn_chunk <= 0 else min(attn_chunk, n)
    cm = min(mlp_chunk, n)
    fc = ffn if ffn_chunk <= 0 else min(ffn_chunk, ffn)
    sh1, sc1, g1, sh2, sc2, g2 = (np.asarray(m, np.float64) for m in mod)
    wq, wk, wv = _split(w, d)
    lo = lora or {}
    res = np.array(x, dtype=np.float64, copy=True)

    k = np.empty((n, d))
    v = np.empty((n, d))
    qk = qk or {}
    cos, sin = qk.get("cos"), qk.get("sin")

    def rows(tab, a, b):
        return None if tab is None else tab[a:b]

    for s0 in range(0, n, ca):                      # pass 1: K and V only
        s1 = min(n, s0 + ca)
        n1 = modulate(layer_norm(res[s0:s1], eps), sh1, sc1)
        k[s0:s1] = qk_transform(linear(n1, wk) + lora_delta(n1, lo.get("k")), qk.get("k_norm"),
                                rows(cos, s0, s1), rows(sin, s0, s1), n_heads, eps)
        v[s0:s1] = linear(n1, wv) + lora_delta(n1, lo.get("v"))
    for s0 in range(0, n, ca):                      # pass 2: Q slice vs global K/V
        s1 = min(n, s0 + ca)
        n1 = modulate(layer_norm(res[s0:s1], eps), sh1, sc1)
        q = qk_transform(linear(n1, wq) + lora_delta(n1, lo.get("q")), qk.get("q_norm"), rows(cos, s0, s1),
                         rows(sin, s0, s1), n_heads, eps)
        o = attention(q, k, v, n_heads)
        res[s0:s1] += g1 * (linear(o, w["o"]) + lora_delta(o, lo.get("o")))
    for m0 in range(0, n, cm):                      # MLP, token slabs
        m1 = min(n, m0 + cm)
        n2 = modulate(layer_norm(res[m0:m1], eps), sh2, sc2)
        acc = np.zeros((m1 - m0, d))
        ad = lo.get("down")
        t = 0.0 if ad is None else np.zeros((m1 - m0, ad[0].shape[0]))
        for f0 in range(0, ffn, fc):                # optional FFN feature slices
            f1 = min(ffn, f0 + fc)
            h = _mlp_hidden(n2, w, ffn, f0, f1, lo)
            acc += linear(h, w["down"][:, f0:f1])
            if ad is not None:
                t = t + linear(h, ad[0][:, f0:f1])  # A h, accumulated over the slices
        if ad is not None:
            acc += ad[2] * linear(t, ad[1])
        res[m0:m1] += g2 * acc
    return res


def global_kv(x: np.ndarray, mod: np.ndarray, w: dict, n_heads: int, eps: float = 1e-6,
              qk: dict | None = None, lora: dict | None = None) -> tuple:
    """K and V of all N tokens (K after its QK transform, if any): what every
    query row attends to."""
    d = x.shape[1]
    _, wk, wv = _split(w, d)
    qk = qk or {}
    lo = lora or {}
    n1_all = modulate(layer_norm(x, eps), np.asarray(mod[0], np.float64), np.asarray(mod[1], np.float64))
    k = linear(n1_all, wk) + lora_delta(n1_all, lo.get("k"))
    v = linear(n1_all, wv) + lora_delta(n1_all, lo.get("v"))
    del n1_all
    k = qk_transform(k, qk.get("k_norm"), qk.get("cos"), qk.get("sin"), n_heads, eps)
    return k, v


def block_rows(x: np.ndarray, mod: np.ndarray, w: dict, n_heads: int, rows: np.ndarray,
               eps: float = 1e-6, want: tuple = (), qk: dict | None = None,
               lora: dict | None = None, kv: tuple | None = None) -> np.ndarray | tuple:
    """The block output for the query rows ``rows`` only (exact for those rows).

    norm1 and K/V are computed for all N tokens, because every query attends
    every key (``global_kv``; ``kv`` passes them in when several row sets share
    them); every later step is per token, so it runs on the chosen rows.
    """
    d = x.shape[1]
    ffn = w["down"].shape[1]
    sh1, sc1, g1, sh2, sc2, g2 = (np.asarray(m, np.float64) for m in mod)
    wq, _, _ = _split(w, d)
    qk = qk or {}
    lo = lora or {}
    cos, sin = qk.get("cos"), qk.get("sin")
    k, v = global_kv(x, mod, w, n_heads, eps, qk, lora) if kv is None else kv
    xr = x[rows]
    n1 = modulate(layer_norm(xr, eps), sh1, sc1)
    q = qk_transform(linear(n1, wq) + lora_delta(n1, lo.get("q")), qk.get("q_norm"),
                     None if cos is None else cos[rows], None if sin is None else sin[rows], n_heads, eps)
    o = attention(q, k, v, n_heads)
    x1 = xr + g1 * (linear(o, w["o"]) + lora_delta(o, lo.get("o")))
    n2 = modulate(layer_norm(x1, eps), sh2, sc2)
    h = _mlp_hidden(n2, w, ffn, 0, ffn, lo)
    y = x1 + g2 * (linear(h, w["down"]) + lora_delta(h, lo.get("down")))
    if not want:
        return y
    loc = dict(n1=n1, q=q, k=k[rows], v=v[rows], o=o, x1=x1, n2=n2, h=h)
    return (y,) + tuple(loc[name] for name in want)


def final_layer(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """The output head after the last block: LN(x) * (1 + scale) + shift, then
    projected by w [out, d]: out[t] = w n[t].

    "LayerStream: H3 Chunking", "How the slicing works": the fp32 output head
    runs stock and is sliced by tokens only when memory runs out; the streaming
    proposal's "Summary": final projection/modulation is similarly bounded.
    """
    return linear(modulate(layer_norm(x, eps), np.asarray(shift, np.float64), np.asarray(scale, np.float64)), w)


def final_layer_chunked(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, w: np.ndarray, chunk: int,
                        eps: float = 1e-6) -> np.ndarray:
    """The same head, one slab of ``chunk`` tokens at a time (0 = all tokens)."""
    n = x.shape[0]
    c = n if chunk <= 0 else min(chunk, n)
    out = np.empty((n, w.shape[0]))
    for s0 in range(0, n, c):
        out[s0:s0 + c] = final_layer(x[s0:s0 + c], shift, scale, w, eps)
    return out
