"""Seeded synthetic workloads for paged attention (inputs only, no attention arithmetic).

Every value a request ever has is a function of ``(seed, request id, tensor, position)``:
token values come from ``numpy.random.default_rng([seed, req, tensor, block])`` in blocks of
``BLOCK`` positions, so any range of any request can be regenerated alone. That is what
lets a probe request carry the same bits whatever batch it is placed in, while its page
placement and batch position change.

Recipe (all configs): values are N(0, 1) float32, multiplied by a power-of-two scale where a
workload asks for a peaked softmax, then rounded to bfloat16 (round to nearest even) for the
bf16 workloads. Physical pages come from a seeded permutation of the pool; unused slots and
spare pages are filled with NaN so that any read of a slot that should not be read shows up.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 256
_TENSOR_ID = {"q": 1, "k": 2, "v": 3}


@dataclass(frozen=True)
class AttnShape:
    """Head geometry and cache layout of one workload."""

    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 16
    split_size: int = 256
    dtype: str = "bf16"  # "bf16" or "f32": type of q, k, v and the caches

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# The five workloads: tiny fp32, decode sweep, chunked prefill, long-context decode and
# the mixed continuous-batching trace.
CONFIG_SHAPES: Dict[str, AttnShape] = {
    "tiny_f32": AttnShape(1, 1, 64, 16, 32, "f32"),
    "decode_bf16": AttnShape(32, 4, 128, 16, 256, "bf16"),
    "prefill_bf16": AttnShape(64, 4, 128, 16, 256, "bf16"),
    "long_decode_bf16": AttnShape(64, 4, 128, 16, 256, "bf16"),
    "mixed_trace_bf16": AttnShape(64, 4, 128, 16, 256, "bf16"),
}


# ----------------------------------------------------------------------------- bf16 helpers
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 value, returned as float32."""
    return from_bf16_bits(bf16_bits(x))


# ----------------------------------------------------------------------------- token values
def token_values(seed: int, req: int, tensor: str, start: int, stop: int, heads: int,
                 dim: int, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Values of ``tensor`` ('q', 'k' or 'v') of request ``req`` at positions [start, stop).

    Returns float32 ``[stop - start][heads][dim]``; bf16-exact when ``dtype == 'bf16'``.
    """
    if stop <= start:
        return np.zeros((0, heads, dim), np.float32)
    tid = _TENSOR_ID[tensor]
    b0, b1 = start // BLOCK, (stop - 1) // BLOCK
    parts = []
    for blk in range(b0, b1 + 1):
        rng = np.random.default_rng([int(seed), int(req), tid, blk])
        parts.append(rng.standard_normal((BLOCK, heads, dim), dtype=np.float32))
    vals = np.concatenate(parts, axis=0) if len(parts) > 1 else parts[0]
    vals = vals[start - b0 * BLOCK: stop - b0 * BLOCK]
    if scale != 1.0:
        vals = vals * np.float32(scale)
    if dtype == "bf16":
        vals = bf16_round(vals)
    return np.ascontiguousarray(vals, dtype=np.float32)


# ----------------------------------------------------------------------------- batches
@dataclass(frozen=True)
class SeqSpec:
    """One sequence of a step: ``cached`` tokens already in the cache, ``n_new`` arriving now."""

    req: int
    cached: int
    n_new: int

    @property
    def seq_len(self) -> int:
        return self.cached + self.n_new


@dataclass
class Batch:
    """One attention step over a paged pool, as numpy arrays (float32 values, int32 indices).

    Layouts: ``q [T][Hq][D]``, ``k_new/v_new [T][Hkv][D]``,
    ``k_pool/v_pool [num_pages][Hkv][page_size][D]``, ``page_table [B][max_pages]`` (unused
    entries are -1), ``seq_lens [B]`` (after this step's tokens), ``q_starts [B+1]``.
    The pools hold the cached prefixes only; the new tokens' slots hold NaN until the
    page update writes them.
    """

    shape: AttnShape
    seqs: List[SeqSpec]
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    page_table: np.ndarray
    seq_lens: np.ndarray
    q_starts: np.ndarray
    seed: int = 0
    q_scale: float = 1.0

    @property
    def batch(self) -> int:
        return len(self.seqs)

    @property
    def total_tokens(self) -> int:
        return int(self.q_starts[-1])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_q_len(self) -> int:
        return max([s.n_new for s in self.seqs] + [0])

    @property
    def max_seq_len(self) -> int:
        return max([s.seq_len for s in self.seqs] + [0])

    def token_rows(self, b: int) -> Tuple[int, int]:
        return int(self.q_starts[b]), int(self.q_starts[b + 1])

    def positions(self) -> np.ndarray:
        """Absolute position of every new token, ``[T]``."""
        pos = np.empty(self.total_tokens, np.int64)
        for b, s in enumerate(self.seqs):
            r0, r1 = self.token_rows(b)
            pos[r0:r1] = np.arange(s.cached, s.seq_len)
        return pos


def poisoned_pool(num_pages: int, shape: AttnShape) -> Tuple[np.ndarray, np.ndarray]:
    """Two NaN-filled pools ``[num_pages][Hkv][page_size][D]`` (float32)."""
    dims = (num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim)
    return np.full(dims, np.nan, np.float32), np.full(dims, np.nan, np.float32)


def _pages_for(n_tokens: int, page_size: int) -> int:
    return (n_tokens + page_size - 1) // page_size


def build_batch(shape: AttnShape, seqs: Sequence[SeqSpec], seed: int, *, page_seed: int = 0,
                extra_pages: int = 0, max_pages: Optional[int] = None, q_scale: float = 1.0,
                fill_prefix: bool = True) -> Batch:
    """Place ``seqs`` in a seeded permutation of a NaN-poisoned pool.

    Token values depend on ``(seed, req, position)`` only; page placement depends on
    ``page_seed`` and on the order of ``seqs``.
    """
    P, Hq, Hkv, D = shape.page_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    seqs = list(seqs)
    B = len(seqs)
    npages = [_pages_for(s.seq_len, P) for s in seqs]
    num_pages = sum(npages) + extra_pages
    mp = max(npages + [1]) if max_pages is None else max_pages
    perm = np.random.default_rng([int(page_seed), 0x9A6E, B]).permutation(max(num_pages, 1))
    page_table = np.full((B, mp), -1, np.int32)
    off = 0
    for b, n in enumerate(npages):
        page_table[b, :n] = perm[off: off + n]
        off += n
    k_pool, v_pool = poisoned_pool(max(num_pages, 1), shape)
    seq_lens = np.array([s.seq_len for s in seqs], np.int32)
    q_starts = np.zeros(B + 1, np.int32)
    q_starts[1:] = np.cumsum([s.n_new for s in seqs])
    T = int(q_starts[-1])
    q = np.empty((T, Hq, D), np.float32)
    k_new = np.empty((T, Hkv, D), np.float32)
    v_new = np.empty((T, Hkv, D), np.float32)
    # generate every prefix in parallel (numpy releases the GIL while filling arrays)
    jobs = [(b, s, tensor) for b, s in enumerate(seqs) if fill_prefix and s.cached > 0
            for tensor in ("k", "v")]
    with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        prefix = dict(zip([(b, t) for b, _, t in jobs],
                          ex.map(lambda j: token_values(seed, j[1].req, j[2], 0, j[1].cached, Hkv, D,
                                                        shape.dtype), jobs)))
    for b, s in enumerate(seqs):
        if fill_prefix and s.cached > 0:
            for tensor, pool in (("k", k_pool), ("v", v_pool)):
                vals = prefix.pop((b, tensor))
                npre = _pages_for(s.cached, P)
                padded = np.full((npre * P, Hkv, D), np.nan, np.float32)
                padded[: s.cached] = vals
                # [page][slot][Hkv][D] -> [page][Hkv][slot][D]
                blocks = padded.reshape(npre, P, Hkv, D).transpose(0, 2, 1, 3)
                pages = page_table[b, :npre]
                full = s.cached // P
                pool[pages[:full]] = blocks[:full]
                if npre > full:  # partial last page: keep the NaN in its unused slots
                    pool[pages[full], :, : s.cached - full * P] = blocks[full, :, : s.cached - full * P]
        r0, r1 = int(q_starts[b]), int(q_starts[b + 1])
        if r1 > r0:
            q[r0:r1] = token_values(seed, s.req, "q", s.cached, s.seq_len, Hq, D, shape.dtype, q_scale)
            k_new[r0:r1] = token_values(seed, s.req, "k", s.cached, s.seq_len, Hkv, D, shape.dtype)
            v_new[r0:r1] = token_values(seed, s.req, "v", s.cached, s.seq_len, Hkv, D, shape.dtype)
    return Batch(shape, seqs, q, k_new, v_new, k_pool, v_pool, page_table, seq_lens, q_starts,
                 seed=seed, q_scale=q_scale)


# ----------------------------------------------------------------------------- mixed trace
@dataclass
class TraceStep:
    """One continuous-batching step: decode tokens first, then prefill chunks (FCFS)."""

    decode: List[Tuple[int, int]] = field(default_factory=list)        # (req, position)
    prefill: List[Tuple[int, int, int]] = field(default_factory=list)  # (req, start, n)
    finished: List[int] = field(default_factory=list)                  # reqs done after this step

    @property
    def tokens(self) -> int:
        return len(self.decode) + sum(n for _, _, n in self.prefill)


@dataclass
class Trace:
    prompts: np.ndarray
    outputs: np.ndarray
    steps: List[TraceStep]


def mixed_trace(seed: int, n_requests: int = 256, n_steps: int = 64, budget: int = 8192,
                prompt_range: Tuple[int, int] = (64, 32768),
                output_range: Tuple[int, int] = (16, 1024)) -> Trace:
    """Schedule of the mixed decode/prefill trace.

    All requests arrive at step 0. Each step gives one token to every request that has
    finished its prompt and still has outputs to produce (in request order), then fills the
    rest of the token budget with prompt chunks, first come first served, splitting a prompt
    across steps when it does not fit. Prompt lengths are floor(exp(U[ln lo, ln hi])) and
    output lengths U[lo, hi] (inclusive).
    """
    rng = np.random.default_rng([int(seed), 0x7ACE])
    lo, hi = prompt_range
    prompts = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), n_requests))).astype(np.int64)
    prompts = np.clip(prompts, lo, hi)
    outputs = rng.integers(output_range[0], output_range[1], n_requests, endpoint=True)
    done_prompt = np.zeros(n_requests, np.int64)
    decoded = np.zeros(n_requests, np.int64)
    steps: List[TraceStep] = []
    for _ in range(n_steps):
        st = TraceStep()
        room = budget
        for r in range(n_requests):
            if room == 0:
                break
            if done_prompt[r] == prompts[r] and decoded[r] < outputs[r]:
                st.decode.append((r, int(prompts[r] + decoded[r])))
                room -= 1
        for r in range(n_requests):
            if room == 0:
                break
            if done_prompt[r] < prompts[r]:
                n = int(min(room, prompts[r] - done_prompt[r]))
                st.prefill.append((r, int(done_prompt[r]), n))
                room -= n
        for r, _ in st.decode:
            decoded[r] += 1
            if decoded[r] == outputs[r]:
                st.finished.append(r)
        for r, _, n in st.prefill:
            done_prompt[r] += n
        steps.append(st)
    return Trace(prompts, outputs, steps)


class PageAllocator:
    """FIFO free list over a seeded permutation of ``num_pages`` physical pages."""

    def __init__(self, num_pages: int, seed: int):
        self.free = list(np.random.default_rng([int(seed), 0xA11C]).permutation(num_pages))
        self.owned: Dict[int, List[int]] = {}

    def ensure(self, req: int, n_tokens: int, page_size: int) -> List[int]:
        pages = self.owned.setdefault(req, [])
        need = _pages_for(n_tokens, page_size)
        while len(pages) < need:
            if not self.free:
                raise RuntimeError("page pool exhausted")
            pages.append(int(self.free.pop(0)))
        return pages

    def release(self, req: int) -> None:
        self.free.extend(self.owned.pop(req, []))


# ----------------------------------------------------------------------------- RMSNorm inputs
def norm_inputs(seed: int, rows: int, hidden: int, dtype: str):
    """Seeded RMSNorm inputs: activations ``x [rows][hidden]`` ~ N(0,1) and a weight vector
    ``[hidden]`` ~ U[0.5, 1.5], as float32 arrays holding values exact in ``dtype``. Row r's
    values depend on (seed, r) only, so a row is the same whatever rows surround it."""
    x = np.empty((rows, hidden), np.float32)
    for r in range(rows):
        x[r] = np.random.default_rng([int(seed), 0x4E4F, r]).standard_normal(hidden)
    w = np.random.default_rng([int(seed), 0x5747]).uniform(0.5, 1.5, hidden).astype(np.float32)
    if dtype == "bf16":
        x, w = bf16_round(x), bf16_round(w)
    return x, w


# ----------------------------------------------------------------------------- GEMM inputs
def gemm_inputs(seed: int, m: int, n: int, k: int):
    """Seeded linear-layer inputs: activations ``A [m][k]`` ~ N(0,1) (row i depends on (seed, i)
    only) and a weight ``W [n][k]`` ~ N(0, 1/k), as float32 arrays holding bf16 values."""
    a = np.empty((m, k), np.float32)
    for i in range(m):
        a[i] = np.random.default_rng([int(seed), 0x4745, i]).standard_normal(k)
    w = (np.random.default_rng([int(seed), 0x5745]).standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    return bf16_round(a), bf16_round(w)
