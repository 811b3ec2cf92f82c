"""Seeded synthetic inputs for one DiT transformer block.

This module only draws and encodes numbers; it holds none of the block's
arithmetic. The GPU path and the fp64 oracle both take their inputs from here.

Recipe (one ``numpy.random.Generator(PCG64(seed))``, fixed draw order):

* ``x``    [N, d]    ~ N(0, 1)
* ``mod``  [6, d]    ~ N(0, variance 0.1)  (shift1, scale1, gate1, shift2, scale2, gate2)
* ``w_qkv`` [3d, d], ``w_o`` [d, d], ``w_gu`` [2F, d], ``w_down`` [d, F]
  ~ N(0, variance 1/d), in that order.

Draws are fp64. Activations and weights are rounded once, round-to-nearest-even,
to the storage type (fp32 for the "f32" block, bf16 otherwise); ``mod`` is
always fp32. For the weight-only int8 block each weight matrix is replaced by
integers drawn uniformly from [-127, 127] followed by one fp32 scale per output
row drawn uniformly from [1e-4, 1e-3). Large arrays are drawn in row blocks from
the same generator; ``standard_normal`` consumes the stream one value at a time,
so block draws equal a single draw (checked in the tests).

bf16 arrays are returned as their raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["BlockShape", "CONFIGS", "make_inputs", "make_qk_inputs", "make_lora", "LORA_TARGETS", "rope_tables",
           "bf16_bits_to_f64", "f64_to_bf16_bits", "sample_rows", "to_f64"]

# Projections an activation-space adapter can attach to, in draw order.
LORA_TARGETS = ("q", "k", "v", "o", "gate", "up", "down")

_BLOCK_ELEMS = 1 << 23  # values per draw call when filling large arrays


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """Shape and chunking of one DiT-block workload."""
    name: str
    d: int
    n_heads: int
    head_dim: int
    ffn: int
    n_tokens: int
    dtype: str               # "f32", "bf16" or "w8_bf16"
    attn_chunk: int = 0      # query tokens per attention slice (0 = one slice)
    mlp_chunk: int = 0       # tokens per MLP slice (0 = all tokens)
    ffn_chunk: int = 0       # FFN features per slice (0 = all features)
    eps: float = 1e-6

    def replace(self, **kw) -> "BlockShape":
        return dataclasses.replace(self, **kw)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of one forward: QKV 6Nd^2, out 2Nd^2, attention 4N^2d, MLP 6NdF."""
        n, d, f = self.n_tokens, self.d, self.ffn
        return 8.0 * n * d * d + 4.0 * n * n * d + 6.0 * n * d * f


# The five workloads: a tiny fp32 block, a mid bf16 block, the 32k-token
# headline block, a 131k-token long clip with FFN-feature slicing, and a
# weight-only int8 block at 65k tokens.
CONFIGS = {
    "tiny": BlockShape("tiny", 256, 4, 64, 1024, 1024, "f32", 256, 256, 0),
    "mid": BlockShape("mid", 3072, 24, 128, 8192, 16384, "bf16", 4096, 4096, 0),
    "large": BlockShape("large", 5120, 40, 128, 13824, 32768, "bf16", 8192, 8192, 0),
    "longclip": BlockShape("longclip", 5120, 40, 128, 13824, 131072, "bf16", 8192, 8192, 3456),
    "int8": BlockShape("int8", 5120, 40, 128, 13824, 65536, "w8_bf16", 8192, 8192, 0),
}


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp64 values once, to nearest-even, to bf16; return the uint16 bit patterns.

    bf16 keeps 8 significant bits. ``frexp`` puts the significand in [0.5, 1);
    scaling by 256 and ``np.round`` (ties to even) keeps exactly 8 bits. The
    rounded value is then exact in fp32, whose top half is the bf16 pattern.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.round(m * 256.0) / 256.0, e)
    tiny = (r != 0) & (np.abs(r) < 2.0 ** -126)
    if tiny.any():
        raise ValueError("value below the normal bf16 range")
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact conversion of bf16 bit patterns to fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _normal(rng: np.random.Generator, shape, std: float, store: str) -> np.ndarray:
    rows, cols = shape
    out = np.empty(shape, dtype=np.uint16 if store == "bf16" else np.float32)
    step = max(1, _BLOCK_ELEMS // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = rng.standard_normal((r1 - r0, cols)) * std
        out[r0:r1] = f64_to_bf16_bits(z) if store == "bf16" else z.astype(np.float32)
    return out


def _int8_weight(rng: np.random.Generator, shape):
    rows, cols = shape
    q = np.empty(shape, dtype=np.int8)
    step = max(1, _BLOCK_ELEMS // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        q[r0:r1] = rng.integers(-127, 127, size=(r1 - r0, cols), endpoint=True, dtype=np.int8)
    s = rng.uniform(1e-4, 1e-3, size=rows).astype(np.float32)
    return q, s


def make_inputs(shape: BlockShape, seed: int = 0, with_x: bool = True) -> dict:
    """Draw x, mod and the four weight matrices for ``shape``.

    Returns a dict with ``x`` (uint16 bf16 bits or fp32), ``mod`` (fp32 [6, d])
    and ``w_qkv``, ``w_o``, ``w_gu``, ``w_down`` (bf16 bits, fp32, or int8).
    For "w8_bf16" it also holds ``s_qkv``, ``s_o``, ``s_gu``, ``s_down`` (fp32).
    ``with_x=False`` still consumes the x draws, so weights stay identical.
    """
    d, f, n = shape.d, shape.ffn, shape.n_tokens
    if shape.n_heads * shape.head_dim != d:
        raise ValueError("d must equal n_heads * head_dim")
    rng = np.random.Generator(np.random.PCG64(seed))
    act = "f32" if shape.dtype == "f32" else "bf16"
    out = {}
    x = _normal(rng, (n, d), 1.0, act)
    if with_x:
        out["x"] = x
    del x
    out["mod"] = (rng.standard_normal((6, d)) * np.sqrt(0.1)).astype(np.float32)
    wstd = 1.0 / np.sqrt(d)
    for name, wshape in (("qkv", (3 * d, d)), ("o", (d, d)), ("gu", (2 * f, d)), ("down", (d, f))):
        if shape.dtype == "w8_bf16":
            out["w_" + name], out["s_" + name] = _int8_weight(rng, wshape)
        else:
            out["w_" + name] = _normal(rng, wshape, wstd, act)
    return out


def rope_tables(n_tokens: int, head_dim: int, base: float = 10000.0, offset: int = 0):
    """fp32 cos/sin tables [N, head_dim/2] for 1-D token positions offset..offset+N-1:
    angle(i, j) = (offset + i) * base^(-2j / head_dim), drawn in fp64, rounded once."""
    pos = np.arange(offset, offset + n_tokens, dtype=np.float64)[:, None]
    freq = base ** (-2.0 * np.arange(head_dim // 2, dtype=np.float64) / head_dim)
    ang = pos * freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_qk_inputs(shape: BlockShape, seed: int = 0) -> dict:
    """Optional QK-norm weights and RoPE tables for ``shape``: ``q_norm`` and
    ``k_norm`` [head_dim] fp32 ~ 1 + N(0, variance 0.01), drawn from
    PCG64(seed + 1000) (so the block's own draws are unchanged), and ``cos`` /
    ``sin`` from ``rope_tables``."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    q_norm = (1.0 + 0.1 * rng.standard_normal(shape.head_dim)).astype(np.float32)
    k_norm = (1.0 + 0.1 * rng.standard_normal(shape.head_dim)).astype(np.float32)
    cos, sin = rope_tables(shape.n_tokens, shape.head_dim)
    return {"q_norm": q_norm, "k_norm": k_norm, "cos": cos, "sin": sin}


def make_final_inputs(n_tokens: int, d: int, out_dim: int, act: str = "bf16", seed: int = 0) -> dict:
    """Inputs of the output head, drawn from PCG64(seed + 2000) in this order:
    ``x`` [N, d] (bf16 bits or fp32) = N(0, 1) per element plus one N(0, 0.25)
    offset per row (so row means are far from zero), ``shift`` and ``scale``
    [d] fp32 ~ N(0, variance 0.1) (like the block's modulation), ``w_out``
    [out_dim, d] fp32 ~ N(0, variance 1/d)."""
    rng = np.random.Generator(np.random.PCG64(seed + 2000))
    step = max(1, _BLOCK_ELEMS // d)
    x = np.empty((n_tokens, d), dtype=np.uint16 if act == "bf16" else np.float32)
    for r0 in range(0, n_tokens, step):
        r1 = min(n_tokens, r0 + step)
        z = rng.standard_normal((r1 - r0, d)) + 0.5 * rng.standard_normal((r1 - r0, 1))
        x[r0:r1] = f64_to_bf16_bits(z) if act == "bf16" else z.astype(np.float32)
    shift = (rng.standard_normal(d) * np.sqrt(0.1)).astype(np.float32)
    scale = (rng.standard_normal(d) * np.sqrt(0.1)).astype(np.float32)
    w_out = (rng.standard_normal((out_dim, d)) / np.sqrt(d)).astype(np.float32)
    return {"x": x, "shift": shift, "scale": scale, "w_out": w_out}


def make_lora(shape: BlockShape, rank, seed: int = 0, targets=LORA_TARGETS, alpha: float = 0.5) -> dict:
    """Activation-space adapters for ``shape``, drawn from PCG64(seed + 3000).

    For each target in LORA_TARGETS order (targets not asked for are skipped
    without drawing): ``A`` [rank, in] ~ N(0, variance 1/in), then ``B``
    [out, rank] ~ N(0, variance 1/rank), stored like the block's activations
    (fp32 for the "f32" block, bf16 bits otherwise); in/out are d/d for q, k,
    v, o, d/F for gate and up, F/d for down. ``rank`` is an int or a
    {target: rank} dict. Returns {target: (A, B, alpha)}.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 3000))
    act = "f32" if shape.dtype == "f32" else "bf16"
    d, f = shape.d, shape.ffn
    dims = {"q": (d, d), "k": (d, d), "v": (d, d), "o": (d, d), "gate": (d, f), "up": (d, f), "down": (f, d)}
    out = {}
    for name in LORA_TARGETS:
        if name not in targets:
            continue
        r = rank[name] if isinstance(rank, dict) else rank
        n_in, n_out = dims[name]
        a = _normal(rng, (r, n_in), 1.0 / np.sqrt(n_in), act)
        b = _normal(rng, (n_out, r), 1.0 / np.sqrt(r), act)
        out[name] = (a, b, float(np.float32(alpha)))
    return out


def to_f64(arr: np.ndarray) -> np.ndarray:
    """Decode a stored array (bf16 bits, fp32 or int8) exactly to fp64."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


def sample_rows(n_tokens: int, count: int = 512, seed: int = 1) -> np.ndarray:
    """Sorted query rows checked at full size: ``count`` distinct rows from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    count = min(count, n_tokens)
    return np.sort(rng.choice(n_tokens, count, replace=False))
