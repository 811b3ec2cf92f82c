"""Thin ctypes binding over the C ABI in ``include/dit_block.h``,
``include/dit_block_steps.h``, ``include/dit_block_profile.h`` and
``include/dit_final_layer.h``.

Argument marshalling only: every step of the block runs in the HIP library.
torch supplies device memory and the stream. If the library is not built the
calls raise; there is no other path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit_block.so")
_lib = None

DIT_OK, DIT_EINVAL, DIT_ENOSPC, DIT_EHIP, DIT_ETOOBIG = 0, -1, -2, -3, -4
# bytes of the library-owned workspace of dit_block_forward_noalloc (per GPU)
STATIC_WORKSPACE_BYTES = 64 << 20
DTYPES = {"f32": 0, "bf16": 1, "w8_bf16": 2}
EPILOGUES = {"store": 0, "store_t": 1, "resid": 2, "gateup": 3, "accum": 4, "final": 5}

# Chunk sizes the pages' node starts from ("LayerStream: H3 Chunking",
# section "The two numbers you set").
DEFAULT_ATTN_CHUNK = 8192
DEFAULT_MLP_CHUNK = 8192

EXPORTS = ("dit_block_create", "dit_block_peak_workspace", "dit_block_plan_chunks", "dit_block_forward",
           "dit_block_forward_rope", "dit_block_destroy", "dit_block_strerror", "dit_modnorm", "dit_attention",
           "dit_qk_transform", "dit_linear", "dit_profile_enable", "dit_profile_read", "dit_final_layer",
           "dit_block_set_lora", "dit_block_forward_noalloc", "dit_block_set_attention_splits",
           "dit_attention_split", "dit_attention_split_workspace")
PROFILE_KINDS = ("modnorm", "kv_proj", "q_proj", "attention", "out_proj", "gate_up", "down", "qk", "final", "lora",
                 "norm2")


class DitError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class _Desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("n_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("ffn", ctypes.c_int64), ("dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


class _Weights(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("w_gu", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_qkv", ctypes.c_void_p), ("s_o", ctypes.c_void_p),
                ("s_gu", ctypes.c_void_p), ("s_down", ctypes.c_void_p), ("q_norm", ctypes.c_void_p),
                ("k_norm", ctypes.c_void_p)]


class _Lora(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("rank", ctypes.c_int64), ("alpha", ctypes.c_float)]


class _BlockLora(ctypes.Structure):
    _fields_ = [(name, _Lora) for name in ("q", "k", "v", "o", "gate", "up", "down")]


LORA_TARGETS = ("q", "k", "v", "o", "gate", "up", "down")


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load ``libdit_block.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} (run python -m memory_bounded_chunked_amd.build)")
    lib = ctypes.CDLL(p)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
    lib.dit_block_create.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Weights), ctypes.POINTER(vp)]
    lib.dit_block_create.restype = ctypes.c_int
    lib.dit_block_peak_workspace.argtypes = [vp, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.dit_block_peak_workspace.restype = ctypes.c_int
    lib.dit_block_plan_chunks.argtypes = [vp, i64, ctypes.c_size_t, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                          ctypes.POINTER(i64)]
    lib.dit_block_plan_chunks.restype = ctypes.c_int
    lib.dit_block_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.dit_block_forward.restype = ctypes.c_int
    lib.dit_block_forward_rope.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.dit_block_forward_rope.restype = ctypes.c_int
    lib.dit_block_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp]
    lib.dit_block_forward_noalloc.restype = ctypes.c_int
    lib.dit_block_set_attention_splits.argtypes = [vp, i64]
    lib.dit_block_set_attention_splits.restype = ctypes.c_int
    lib.dit_attention_split.argtypes = [i32, vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, i64, i64, vp,
                                        ctypes.c_size_t, vp]
    lib.dit_attention_split.restype = ctypes.c_int
    lib.dit_attention_split_workspace.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.dit_attention_split_workspace.restype = ctypes.c_int
    lib.dit_qk_transform.argtypes = [i32, vp, i64, i64, i64, i64, vp, vp, vp, i64, ctypes.c_float, vp]
    lib.dit_qk_transform.restype = ctypes.c_int
    lib.dit_block_set_lora.argtypes = [vp, ctypes.POINTER(_BlockLora)]
    lib.dit_block_set_lora.restype = ctypes.c_int
    lib.dit_block_destroy.argtypes = [vp]
    lib.dit_block_destroy.restype = None
    lib.dit_block_strerror.argtypes = [ctypes.c_int]
    lib.dit_block_strerror.restype = ctypes.c_char_p
    lib.dit_modnorm.argtypes = [i32, i32, vp, i64, vp, vp, vp, i64, i64, i64, ctypes.c_float, vp]
    lib.dit_modnorm.restype = ctypes.c_int
    lib.dit_attention.argtypes = [i32, vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, i64, vp]
    lib.dit_attention.restype = ctypes.c_int
    lib.dit_linear.argtypes = [i32, i32, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp, i64, vp, i64, vp, vp]
    lib.dit_linear.restype = ctypes.c_int
    lib.dit_final_layer.argtypes = [i32, vp, i64, i64, i64, vp, vp, vp, i64, vp, i64, ctypes.c_float, vp]
    lib.dit_final_layer.restype = ctypes.c_int
    lib.dit_profile_enable.argtypes = [ctypes.c_int]
    lib.dit_profile_enable.restype = ctypes.c_int
    lib.dit_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.dit_profile_read.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().dit_block_strerror(code).decode()


def _check(code: int, what: str) -> None:
    if code != DIT_OK:
        raise DitError(code, what)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class DitBlock:
    """One DiT block with borrowed device weights.

    ``weights``: ``w_qkv`` [3d, d], ``w_o`` [d, d], ``w_gu`` [2F, d], ``w_down``
    [d, F] (torch tensors on the GPU, fp32 / bf16 / int8 by ``dtype``) and for
    "w8_bf16" the fp32 per-row scales ``s_qkv``, ``s_o``, ``s_gu``, ``s_down``.
    The tensors are kept referenced for the life of the block.
    """

    def __init__(self, d: int, n_heads: int, head_dim: int, ffn: int, dtype: str, weights: dict,
                 eps: float = 1e-6):
        self._lib = load_library()
        self.d, self.n_heads, self.head_dim, self.ffn, self.dtype = d, n_heads, head_dim, ffn, dtype
        self._weights = dict(weights)
        desc = _Desc(d, n_heads, head_dim, ffn, DTYPES[dtype], eps)
        w = _Weights(*(_ptr(self._weights.get(k)) for k in
                       ("w_qkv", "w_o", "w_gu", "w_down", "s_qkv", "s_o", "s_gu", "s_down", "q_norm", "k_norm")))
        h = ctypes.c_void_p()
        _check(self._lib.dit_block_create(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(h)),
               "dit_block_create")
        self._h = h

    def set_lora(self, adapters: dict | None) -> None:
        """Attach activation-space adapters: ``{target: (A, B, alpha)}`` for targets
        among q, k, v, o, gate, up, down, with A [rank, in] and B [out, rank]
        device tensors in the activation type (see ``dit_block_set_lora``).
        ``None`` or ``{}`` detaches. The tensors stay referenced by the block."""
        if not adapters:
            _check(self._lib.dit_block_set_lora(self._h, None), "dit_block_set_lora")
            self._lora = {}
            return
        unknown = set(adapters) - set(LORA_TARGETS)
        if unknown:
            raise ValueError(f"unknown adapter targets {sorted(unknown)}")
        st = _BlockLora()
        for name, (a, b, alpha) in adapters.items():
            setattr(st, name, _Lora(a.data_ptr(), b.data_ptr(), a.shape[0], float(alpha)))
        _check(self._lib.dit_block_set_lora(self._h, ctypes.byref(st)), "dit_block_set_lora")
        self._lora = dict(adapters)

    def set_attention_splits(self, splits: int) -> None:
        """Key ranges per query in this block's attention (see
        ``dit_block_set_attention_splits``); 1 = none."""
        _check(self._lib.dit_block_set_attention_splits(self._h, splits), "dit_block_set_attention_splits")

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.dit_block_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def peak_workspace(self, n_tokens: int, attn_chunk_tokens: int = DEFAULT_ATTN_CHUNK,
                       mlp_chunk_tokens: int = DEFAULT_MLP_CHUNK, ffn_chunk_features: int = 0) -> int:
        out = ctypes.c_size_t()
        _check(self._lib.dit_block_peak_workspace(self._h, n_tokens, attn_chunk_tokens, mlp_chunk_tokens,
                                                  ffn_chunk_features, ctypes.byref(out)),
               "dit_block_peak_workspace")
        return out.value

    def plan_chunks(self, n_tokens: int, budget_bytes: int) -> tuple:
        """(attn_chunk_tokens, mlp_chunk_tokens, ffn_chunk_features): the largest chunks
        whose workspace fits ``budget_bytes`` (see ``dit_block_plan_chunks``)."""
        a, m, f = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(self._lib.dit_block_plan_chunks(self._h, n_tokens, budget_bytes, ctypes.byref(a), ctypes.byref(m),
                                               ctypes.byref(f)), "dit_block_plan_chunks")
        return a.value, m.value, f.value

    def forward(self, x: torch.Tensor, mod: torch.Tensor, attn_chunk_tokens: int = DEFAULT_ATTN_CHUNK,
                mlp_chunk_tokens: int = DEFAULT_MLP_CHUNK, ffn_chunk_features: int = 0,
                workspace: torch.Tensor | None = None, stream=None, rope: tuple | None = None) -> torch.Tensor:
        """Run the block in place on ``x`` [N, d]; returns ``x``. ``rope`` = (cos, sin)
        fp32 [N, head_dim/2] device tables for the rotary transform of Q and K."""
        n = x.shape[0]
        if workspace is None:
            nbytes = self.peak_workspace(n, attn_chunk_tokens, mlp_chunk_tokens, ffn_chunk_features)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
        cs, sn = (None, None) if rope is None else rope
        _check(self._lib.dit_block_forward_rope(self._h, x.data_ptr(), mod.data_ptr(), _ptr(cs), _ptr(sn), n,
                                                attn_chunk_tokens, mlp_chunk_tokens, ffn_chunk_features,
                                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                                _stream(stream)),
               "dit_block_forward_rope")
        return x


    def forward_noalloc(self, x: torch.Tensor, mod: torch.Tensor, attn_chunk_tokens: int = DEFAULT_ATTN_CHUNK,
                        mlp_chunk_tokens: int = DEFAULT_MLP_CHUNK, ffn_chunk_features: int = 0, stream=None,
                        rope: tuple | None = None) -> torch.Tensor:
        """``forward`` with the library-owned static workspace (no device allocation;
        see ``dit_block_forward_noalloc``). Raises ``DitError`` with DIT_ETOOBIG when
        the sizes need more than ``STATIC_WORKSPACE_BYTES``."""
        cs, sn = (None, None) if rope is None else rope
        _check(self._lib.dit_block_forward_noalloc(self._h, x.data_ptr(), mod.data_ptr(), _ptr(cs), _ptr(sn),
                                                   x.shape[0], attn_chunk_tokens, mlp_chunk_tokens,
                                                   ffn_chunk_features, _stream(stream)),
               "dit_block_forward_noalloc")
        return x


def modnorm(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor, out: torch.Tensor,
            eps: float = 1e-6, stream=None) -> torch.Tensor:
    """Modulated LayerNorm of the rows of ``x`` into ``out`` (one kernel)."""
    lib = load_library()
    code = {torch.float32: 0, torch.bfloat16: 1}
    _check(lib.dit_modnorm(code[x.dtype], code[out.dtype], x.data_ptr(), x.stride(0), shift.data_ptr(),
                           scale.data_ptr(), out.data_ptr(), out.stride(0), x.shape[0], x.shape[1], eps,
                           _stream(stream)), "dit_modnorm")
    return out


def qk_transform(x: torch.Tensor, n_heads: int, norm_w: torch.Tensor | None = None, rope: tuple | None = None,
                 eps: float = 1e-6, stream=None) -> torch.Tensor:
    """QK RMSNorm and/or RoPE in place on the rows of ``x`` (one kernel)."""
    lib = load_library()
    dt = {torch.float32: 0, torch.bfloat16: 1}[x.dtype]
    cs, sn = (None, None) if rope is None else rope
    _check(lib.dit_qk_transform(dt, x.data_ptr(), x.stride(0), x.shape[0], n_heads, x.shape[1] // n_heads,
                                _ptr(norm_w), _ptr(cs), _ptr(sn), 0 if cs is None else cs.stride(0), eps,
                                _stream(stream)), "dit_qk_transform")
    return x


def attention(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, out: torch.Tensor, n_heads: int,
              n_kv: int | None = None, stream=None) -> torch.Tensor:
    """Attention of the rows of ``q`` against ``k`` and transposed ``vt`` (one kernel)."""
    lib = load_library()
    dt = {torch.float32: 0, torch.bfloat16: 1}[q.dtype]
    n_kv = k.shape[0] if n_kv is None else n_kv
    head_dim = q.shape[1] // n_heads
    _check(lib.dit_attention(dt, q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), vt.data_ptr(),
                             vt.stride(0), out.data_ptr(), out.stride(0), q.shape[0], n_kv, n_heads, head_dim,
                             _stream(stream)), "dit_attention")
    return out


def attention_split(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, out: torch.Tensor, n_heads: int,
                    splits: int, n_kv: int | None = None, workspace: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Attention with each query's keys in ``splits`` ranges merged afterwards
    (two kernels; see ``dit_attention_split``)."""
    lib = load_library()
    dt = {torch.float32: 0, torch.bfloat16: 1}[q.dtype]
    n_kv = k.shape[0] if n_kv is None else n_kv
    head_dim = q.shape[1] // n_heads
    need = ctypes.c_size_t()
    _check(lib.dit_attention_split_workspace(q.shape[0], n_kv, n_heads, head_dim, splits, ctypes.byref(need)),
           "dit_attention_split_workspace")
    if workspace is None:
        workspace = torch.empty(max(need.value, 16), dtype=torch.uint8, device=q.device)
    _check(lib.dit_attention_split(dt, q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), vt.data_ptr(),
                                   vt.stride(0), out.data_ptr(), out.stride(0), q.shape[0], n_kv, n_heads, head_dim,
                                   splits, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "dit_attention_split")
    return out


def linear(dtype: str, epilogue: str, a: torch.Tensor, w: torch.Tensor, out: torch.Tensor, n: int,
           k: int | None = None, w_scale: torch.Tensor | None = None, up_offset: int = 0,
           aux: torch.Tensor | None = None, gate: torch.Tensor | None = None, m: int | None = None,
           stream=None) -> torch.Tensor:
    """One projection with a fused epilogue (one kernel); see ``dit_linear``."""
    lib = load_library()
    m = a.shape[0] if m is None else m
    k = a.shape[1] if k is None else k
    _check(lib.dit_linear(DTYPES[dtype], EPILOGUES[epilogue], a.data_ptr(), a.stride(0), w.data_ptr(),
                          w.stride(0), _ptr(w_scale), up_offset, m, n, k, out.data_ptr(), out.stride(0),
                          _ptr(aux), 0 if aux is None else aux.stride(0), _ptr(gate), _stream(stream)),
           "dit_linear")
    return out


def final_layer(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor, w_out: torch.Tensor,
                out: torch.Tensor | None = None, eps: float = 1e-6, stream=None) -> torch.Tensor:
    """Output head of the rows of ``x`` [n, d] (fp32 or bf16): modulated LayerNorm, then
    the fp32 projection by ``w_out`` [out_dim, d] into ``out`` [n, out_dim] fp32 (one kernel)."""
    lib = load_library()
    n, d = x.shape
    out_dim = w_out.shape[0]
    if out is None:
        out = torch.empty((n, out_dim), dtype=torch.float32, device=x.device)
    dt = {torch.float32: 0, torch.bfloat16: 1}[x.dtype]
    _check(lib.dit_final_layer(dt, x.data_ptr(), x.stride(0), n, d, shift.data_ptr(), scale.data_ptr(),
                               w_out.data_ptr(), out_dim, out.data_ptr(), out.stride(0), eps, _stream(stream)),
           "dit_final_layer")
    return out


def profile_enable(on: bool) -> None:
    """Start (clearing old records) or stop per-kernel event timing of forwards."""
    _check(load_library().dit_profile_enable(1 if on else 0), "dit_profile_enable")


def profile_read() -> dict:
    """{step: (total_ms, launches)} over the records since the last enable."""
    lib = load_library()
    out = {}
    for i, name in enumerate(PROFILE_KINDS):
        t, n = ctypes.c_double(), ctypes.c_int64()
        _check(lib.dit_profile_read(i, ctypes.byref(t), ctypes.byref(n)), "dit_profile_read")
        out[name] = (t.value, n.value)
    return out


def tensor_from_stored(arr, device) -> torch.Tensor:
    """Host array from ``synth`` (bf16 bit patterns, fp32, int8) -> device tensor."""
    import numpy as np
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def block_from_inputs(shape, inputs: dict, device="cuda") -> tuple:
    """(DitBlock, x, mod) on ``device`` from a ``synth.BlockShape`` and its inputs."""
    w = {k: tensor_from_stored(v, device) for k, v in inputs.items()
         if k[:2] in ("w_", "s_") or k in ("q_norm", "k_norm")}
    blk = DitBlock(shape.d, shape.n_heads, shape.head_dim, shape.ffn, shape.dtype, w, shape.eps)
    x = tensor_from_stored(inputs["x"], device) if "x" in inputs else None
    mod = tensor_from_stored(inputs["mod"], device)
    return blk, x, mod
