"""Thin ctypes binding of ``libbiattn.so`` (argument marshalling only).

Every function here has the name of the C entry point it calls (``include/bi_attn.h``) and
does nothing but turn torch tensors into pointers, sizes and the current HIP stream; all of
the work runs in the library's HIP kernels. A non-OK status raises ``BiAttnError``. There is
no fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbiattn.so")

BI_F32, BI_BF16 = 0, 1
BI_SPLIT_FIXED, BI_SPLIT_BY_BATCH, BI_SPLIT_BY_BATCH_FILL = 0, 1, 2
BI_OK, BI_EINVAL, BI_EUNSUPPORTED, BI_EWORKSPACE, BI_EHIP = 0, 1, 2, 3, 4

NOALLOC_SCRATCH_BYTES = 64 << 20   # BI_NOALLOC_SCRATCH_BYTES

EXPORTED = ("bi_kv_page_update", "bi_attn_workspace_bytes", "bi_attn_decode", "bi_attn_decode_noalloc",
            "bi_attn_decode_partials", "bi_attn_decode_combine", "bi_attn_decode_append",
            "bi_attn_decode_append_partials", "bi_attn_prefill",
            "bi_attn_varlen", "bi_status_string", "bi_rmsnorm", "bi_gemm")


class BiAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bi_status_string(status)} (status {status})")


class _Cfg(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("split_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("split_policy", ctypes.c_int32)]


@dataclass(frozen=True)
class AttnConfig:
    """Python mirror of ``bi_attn_cfg``."""

    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 16
    split_size: int = 256
    dtype: int = BI_BF16
    softmax_scale: float = 0.0
    split_policy: int = BI_SPLIT_FIXED

    def c(self) -> _Cfg:
        return _Cfg(self.num_q_heads, self.num_kv_heads, self.head_dim, self.page_size,
                    self.split_size, self.dtype, self.softmax_scale, self.split_policy)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == BI_BF16 else torch.float32


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    CP = ctypes.POINTER(_Cfg)
    lib.bi_status_string.restype = ctypes.c_char_p
    lib.bi_status_string.argtypes = [ctypes.c_int]
    lib.bi_attn_workspace_bytes.restype = Z
    lib.bi_attn_workspace_bytes.argtypes = [CP, I, I]
    lib.bi_kv_page_update.restype = ctypes.c_int
    lib.bi_kv_page_update.argtypes = [CP, P, P, P, P, P, I, I, I, I, P, P, P]
    lib.bi_attn_decode.restype = ctypes.c_int
    lib.bi_attn_decode.argtypes = [CP, P, P, P, P, I, I, P, I, I, P, P, Z, P]
    lib.bi_attn_decode_noalloc.restype = ctypes.c_int
    lib.bi_attn_decode_noalloc.argtypes = [CP, P, P, P, P, I, I, P, I, I, P, P]
    lib.bi_attn_decode_partials.restype = ctypes.c_int
    lib.bi_attn_decode_partials.argtypes = [CP, P, P, P, P, I, I, P, I, I, P, Z, P]
    lib.bi_attn_decode_combine.restype = ctypes.c_int
    lib.bi_attn_decode_combine.argtypes = [CP, P, I, I, P, P, Z, P]
    lib.bi_attn_decode_append.restype = ctypes.c_int
    lib.bi_attn_decode_append.argtypes = [CP, P, P, P, P, P, P, I, I, P, I, I, P, P, Z, P]
    lib.bi_attn_decode_append_partials.restype = ctypes.c_int
    lib.bi_attn_decode_append_partials.argtypes = [CP, P, P, P, P, P, P, I, I, P, I, I, P, Z, P]
    lib.bi_attn_prefill.restype = ctypes.c_int
    lib.bi_attn_prefill.argtypes = [CP, P, P, P, P, I, I, P, P, I, I, I, I, P, P, Z, P]
    lib.bi_attn_varlen.restype = ctypes.c_int
    lib.bi_rmsnorm.restype = ctypes.c_int
    lib.bi_gemm.restype = ctypes.c_int
    lib.bi_gemm.argtypes = [P, P, P, I, I, I, I, P]
    lib.bi_rmsnorm.argtypes = [P, P, P, I, I, I, ctypes.c_float, P]
    lib.bi_attn_varlen.argtypes = [CP, P, P, P, P, P, I, I, I, I, I, P, P]
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    """Device address of a dense GPU tensor: the kernels index plain row-major memory, so a
    strided view or a host tensor is refused here rather than read wrongly."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise BiAttnError(BI_EINVAL, "tensor arguments must be contiguous GPU tensors")
    return t.data_ptr()


def _expect(t: Optional[torch.Tensor], where: str, name: str, dtype: torch.dtype,
            shape: tuple) -> None:
    """Refuse a tensor of the wrong dtype or shape (``None`` in ``shape`` matches any size)
    before anything reaches the library: the kernels index raw memory by the sizes they are
    given, so a mismatch would be read or written past the tensor instead of failing."""
    if t is None:
        raise BiAttnError(BI_EINVAL, f"{where}: {name} is missing")
    if t.dtype != dtype:
        raise BiAttnError(BI_EINVAL, f"{where}: {name} must be {dtype}, got {t.dtype}")
    if t.dim() != len(shape) or any(want is not None and int(got) != want
                                    for got, want in zip(t.shape, shape)):
        raise BiAttnError(BI_EINVAL, f"{where}: {name} must have shape {shape}, got {tuple(t.shape)}")


def _check_cache(cfg: "AttnConfig", where: str, k_cache: torch.Tensor, v_cache: torch.Tensor) -> int:
    """Both caches ``[num_pages][Hkv][page_size][D]`` of the configured dtype; returns
    num_pages."""
    dt = cfg.torch_dtype
    _expect(k_cache, where, "k_cache", dt, (None, cfg.num_kv_heads, cfg.page_size, cfg.head_dim))
    _expect(v_cache, where, "v_cache", dt, tuple(k_cache.shape))
    return int(k_cache.shape[0])


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status: int, where: str) -> None:
    if status != BI_OK:
        raise BiAttnError(status, where)


def bi_status_string(status: int) -> str:
    return load().bi_status_string(int(status)).decode()


def bi_attn_workspace_bytes(cfg: AttnConfig, rows_tokens: int, max_seq_len: int) -> int:
    return int(load().bi_attn_workspace_bytes(ctypes.byref(cfg.c()), int(rows_tokens), int(max_seq_len)))


def bi_kv_page_update(cfg: AttnConfig, k_new: torch.Tensor, v_new: torch.Tensor,
                      q_starts: torch.Tensor, seq_lens: torch.Tensor, page_table: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Write a step's new K/V rows into their pages (before attention, same stream)."""
    w = "bi_kv_page_update"
    _check_cache(cfg, w, k_cache, v_cache)
    _expect(k_new, w, "k_new", cfg.torch_dtype, (None, cfg.num_kv_heads, cfg.head_dim))
    _expect(v_new, w, "v_new", cfg.torch_dtype, tuple(k_new.shape))
    _expect(seq_lens, w, "seq_lens", torch.int32, (None,))
    B = int(seq_lens.shape[0])
    _expect(q_starts, w, "q_starts", torch.int32, (B + 1,))
    _expect(page_table, w, "page_table", torch.int32, (B, None))
    st = load().bi_kv_page_update(
        ctypes.byref(cfg.c()), _ptr(k_new), _ptr(v_new), _ptr(q_starts), _ptr(seq_lens),
        _ptr(page_table), page_table.shape[1], k_cache.shape[0], seq_lens.shape[0],
        k_new.shape[0], _ptr(k_cache), _ptr(v_cache), _stream(stream))
    _check(st, "bi_kv_page_update")


def bi_attn_decode(cfg: AttnConfig, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                   out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """One query token per sequence; ``out`` fp32 ``[batch][Hq][D]``."""
    _check_decode(cfg, "bi_attn_decode", q, k_cache, v_cache, page_table, seq_lens, out)
    st = load().bi_attn_decode(
        ctypes.byref(cfg.c()), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        page_table.shape[1], k_cache.shape[0], _ptr(seq_lens), seq_lens.shape[0],
        int(max_seq_len), _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "bi_attn_decode")


def bi_attn_decode_noalloc(cfg: AttnConfig, q: torch.Tensor, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                           max_seq_len: int, out: torch.Tensor, stream=None) -> None:
    """``bi_attn_decode`` with the split partials in the library's static device array (no
    workspace, nothing allocated); calls that overlap on one device race."""
    _check_decode(cfg, "bi_attn_decode_noalloc", q, k_cache, v_cache, page_table, seq_lens, out)
    st = load().bi_attn_decode_noalloc(
        ctypes.byref(cfg.c()), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        page_table.shape[1], k_cache.shape[0], _ptr(seq_lens), seq_lens.shape[0],
        int(max_seq_len), _ptr(out), _stream(stream))
    _check(st, "bi_attn_decode_noalloc")


def _check_decode(cfg: AttnConfig, w: str, q, k_cache, v_cache, page_table, seq_lens, out) -> None:
    _expect(seq_lens, w, "seq_lens", torch.int32, (None,))
    B = int(seq_lens.shape[0])
    if q is not None or k_cache is not None:
        _check_cache(cfg, w, k_cache, v_cache)
        _expect(q, w, "q", cfg.torch_dtype, (B, cfg.num_q_heads, cfg.head_dim))
        _expect(page_table, w, "page_table", torch.int32, (B, None))
    if out is not None:
        _expect(out, w, "out", torch.float32, (B, cfg.num_q_heads, cfg.head_dim))


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def bi_attn_decode_partials(cfg: AttnConfig, q: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, page_table: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, workspace: torch.Tensor,
                            stream=None) -> None:
    """First phase of decode: split partials into ``workspace``."""
    _check_decode(cfg, "bi_attn_decode_partials", q, k_cache, v_cache, page_table, seq_lens, None)
    st = load().bi_attn_decode_partials(
        ctypes.byref(cfg.c()), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        page_table.shape[1], k_cache.shape[0], _ptr(seq_lens), seq_lens.shape[0],
        int(max_seq_len), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "bi_attn_decode_partials")


def bi_attn_decode_combine(cfg: AttnConfig, seq_lens: torch.Tensor, max_seq_len: int,
                           out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """Second phase of decode: ascending fold of the partials into ``out``."""
    _check_decode(cfg, "bi_attn_decode_combine", None, None, None, None, seq_lens, out)
    st = load().bi_attn_decode_combine(
        ctypes.byref(cfg.c()), _ptr(seq_lens), seq_lens.shape[0], int(max_seq_len), _ptr(out),
        _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "bi_attn_decode_combine")


def _check_append(cfg: AttnConfig, w: str, k_new, v_new, seq_lens) -> None:
    shape = (int(seq_lens.shape[0]), cfg.num_kv_heads, cfg.head_dim)
    _expect(k_new, w, "k_new", cfg.torch_dtype, shape)
    _expect(v_new, w, "v_new", cfg.torch_dtype, shape)


def bi_attn_decode_append(cfg: AttnConfig, q: torch.Tensor, k_new: torch.Tensor,
                          v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                          out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """Decode step with the page update folded in: writes row b of ``k_new``/``v_new``
    (``[batch][Hkv][D]``) at position ``seq_lens[b] - 1`` and attends, bit-identical to
    ``bi_kv_page_update`` then ``bi_attn_decode``."""
    w = "bi_attn_decode_append"
    _check_decode(cfg, w, q, k_cache, v_cache, page_table, seq_lens, out)
    _check_append(cfg, w, k_new, v_new, seq_lens)
    st = load().bi_attn_decode_append(
        ctypes.byref(cfg.c()), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), page_table.shape[1], k_cache.shape[0], _ptr(seq_lens),
        seq_lens.shape[0], int(max_seq_len), _ptr(out), _ptr(workspace), _nbytes(workspace),
        _stream(stream))
    _check(st, w)


def bi_attn_decode_append_partials(cfg: AttnConfig, q: torch.Tensor, k_new: torch.Tensor,
                                   v_new: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, page_table: torch.Tensor,
                                   seq_lens: torch.Tensor, max_seq_len: int,
                                   workspace: torch.Tensor, stream=None) -> None:
    """First phase of ``bi_attn_decode_append``: page update and split partials."""
    w = "bi_attn_decode_append_partials"
    _check_decode(cfg, w, q, k_cache, v_cache, page_table, seq_lens, None)
    _check_append(cfg, w, k_new, v_new, seq_lens)
    st = load().bi_attn_decode_append_partials(
        ctypes.byref(cfg.c()), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), page_table.shape[1], k_cache.shape[0], _ptr(seq_lens),
        seq_lens.shape[0], int(max_seq_len), _ptr(workspace), _nbytes(workspace),
        _stream(stream))
    _check(st, w)


def bi_attn_prefill(cfg: AttnConfig, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    page_table: torch.Tensor, q_starts: torch.Tensor, seq_lens: torch.Tensor,
                    max_q_len: int, max_seq_len: int, out: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Chunked prefill of ``q [T][Hq][D]``; ``out`` fp32 ``[T][Hq][D]``."""
    w = "bi_attn_prefill"
    _check_cache(cfg, w, k_cache, v_cache)
    _expect(q, w, "q", cfg.torch_dtype, (None, cfg.num_q_heads, cfg.head_dim))
    _expect(out, w, "out", torch.float32, tuple(q.shape))
    _expect(seq_lens, w, "seq_lens", torch.int32, (None,))
    B = int(seq_lens.shape[0])
    _expect(q_starts, w, "q_starts", torch.int32, (B + 1,))
    _expect(page_table, w, "page_table", torch.int32, (B, None))
    st = load().bi_attn_prefill(
        ctypes.byref(cfg.c()), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        page_table.shape[1], k_cache.shape[0], _ptr(q_starts), _ptr(seq_lens),
        seq_lens.shape[0], q.shape[0], int(max_q_len), int(max_seq_len), _ptr(out),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "bi_attn_prefill")


def bi_attn_varlen(cfg: AttnConfig, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   q_starts: torch.Tensor, k_starts: torch.Tensor, max_q_len: int,
                   max_seq_len: int, out: torch.Tensor, stream=None) -> None:
    """Dense varlen attention: ``k``, ``v`` ``[total_k][Hkv][D]``, sequence ``b`` owning rows
    ``k_starts[b] .. k_starts[b+1]-1``; ``q [T][Hq][D]``; ``out`` fp32 ``[T][Hq][D]``."""
    w = "bi_attn_varlen"
    _expect(q, w, "q", cfg.torch_dtype, (None, cfg.num_q_heads, cfg.head_dim))
    _expect(out, w, "out", torch.float32, tuple(q.shape))
    _expect(k, w, "k", cfg.torch_dtype, (None, cfg.num_kv_heads, cfg.head_dim))
    _expect(v, w, "v", cfg.torch_dtype, tuple(k.shape))
    _expect(k_starts, w, "k_starts", torch.int32, (None,))
    _expect(q_starts, w, "q_starts", torch.int32, tuple(k_starts.shape))
    st = load().bi_attn_varlen(
        ctypes.byref(cfg.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(q_starts), _ptr(k_starts),
        k_starts.shape[0] - 1, q.shape[0], k.shape[0], int(max_q_len), int(max_seq_len),
        _ptr(out), _stream(stream))
    _check(st, "bi_attn_varlen")


def bi_rmsnorm(x: torch.Tensor, weight: torch.Tensor, y: torch.Tensor, eps: float,
               stream=None) -> None:
    """Batch-invariant RMSNorm of ``x [rows][hidden]`` (bf16 or fp32) into ``y`` (same shape
    and dtype) with ``weight [hidden]``; one wavefront reduces each row."""
    if x.dtype not in (torch.bfloat16, torch.float32) or y.dtype != x.dtype or weight.dtype != x.dtype:
        raise BiAttnError(BI_EINVAL, "bi_rmsnorm")
    if x.dim() != 2 or tuple(y.shape) != tuple(x.shape) or tuple(weight.shape) != (x.shape[1],):
        raise BiAttnError(BI_EINVAL, "bi_rmsnorm")
    st = load().bi_rmsnorm(_ptr(x), _ptr(weight), _ptr(y), x.shape[0], x.shape[1],
                           BI_BF16 if x.dtype == torch.bfloat16 else BI_F32, float(eps),
                           _stream(stream))
    _check(st, "bi_rmsnorm")


def bi_gemm(a: torch.Tensor, w: torch.Tensor, c: torch.Tensor, stream=None) -> None:
    """Batch-invariant ``c = a @ w.T``: ``a [M][K]``, ``w [N][K]`` bf16, ``c [M][N]`` fp32 or
    bf16; N a multiple of 128, K a multiple of 64."""
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16 or c.dtype not in (torch.float32, torch.bfloat16):
        raise BiAttnError(BI_EINVAL, "bi_gemm")
    if a.dim() != 2 or w.dim() != 2 or c.dim() != 2 or a.shape[1] != w.shape[1] or \
            c.shape[0] != a.shape[0] or c.shape[1] != w.shape[0]:
        raise BiAttnError(BI_EINVAL, "bi_gemm")
    st = load().bi_gemm(_ptr(a), _ptr(w), _ptr(c), a.shape[0], w.shape[0], a.shape[1],
                        1 if c.dtype == torch.bfloat16 else 0, _stream(stream))
    _check(st, "bi_gemm")
