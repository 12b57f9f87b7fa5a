"""fp64 CPU oracle for causal grouped-query attention over a paged KV cache.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package. It
shares no code with the HIP library and imports nothing from it.

What it follows. The write-ups of "Defeating Nondeterminism in LLM Inference" describe
attention as two matrix products, one reducing over the feature dimension and one over the
sequence dimension, run over a KV cache whose page table is updated before the kernel is
launched (neican.ai insight page, section 技术原理与创新点解析, batch-invariant attention
item). They give no formula; this oracle takes the plainest reading, the textbook
``softmax(q k^T / sqrt(D)) V`` with a causal mask that includes the query's own key, with
consecutive query heads sharing a KV head (grouped-query attention), evaluated in float64
on the exact input values the GPU receives. The splitting and folding that make the GPU
path batch invariant change only rounding, so the plain definition is the oracle for every
route (decode, chunked prefill, any batch).

Pins (tests/test_oracle_pins.py): a pure-Python brute force on tiny inputs, torch's
``scaled_dot_product_attention`` in float64 with an explicit mask, hand-derived closed forms
(tests/golden/closed_forms.json), and invariants (weights sum to one, constant V, dominant
key, page permutation, causality, GQA == MHA with repeated heads, q = 0 gives the mean).
``split_fold_attention`` (the fixed-size split and ascending fold, in float64) is pinned
against the plain result. Every function here is pinned; none is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------- page update
def kv_page_update(k_new: np.ndarray, v_new: np.ndarray, q_starts: np.ndarray,
                   seq_lens: np.ndarray, page_table: np.ndarray, k_cache: np.ndarray,
                   v_cache: np.ndarray) -> None:
    """Write each sequence's new tokens into the cache through its page table (in place).

    The page table is brought up to date before the attention launch, so that the kernel
    always sees one consistent KV layout (neican.ai insight page, section
    技术原理与创新点解析, batch-invariant attention item). Sequence ``b``'s new tokens are
    rows ``q_starts[b]:q_starts[b+1]`` of ``k_new``/``v_new`` (``[T][Hkv][D]``); they occupy
    absolute positions ``[seq_lens[b] - n_new, seq_lens[b])`` and position ``pos`` lives in
    page ``page_table[b][pos // P]``, slot ``pos % P`` of ``cache[page][kv_head][slot][:]``.
    """
    P = k_cache.shape[2]
    for b in range(len(seq_lens)):
        r0, r1 = int(q_starts[b]), int(q_starts[b + 1])
        first = int(seq_lens[b]) - (r1 - r0)
        for i in range(r1 - r0):
            pos = first + i
            page = int(page_table[b][pos // P])
            k_cache[page, :, pos % P, :] = k_new[r0 + i]
            v_cache[page, :, pos % P, :] = v_new[r0 + i]


def gather_kv(cache: np.ndarray, table_row: np.ndarray, seq_len: int) -> np.ndarray:
    """The first ``seq_len`` positions of one sequence, ``[seq_len][Hkv][D]`` float64."""
    P = cache.shape[2]
    n_pages = (seq_len + P - 1) // P
    pages = np.asarray(table_row[:n_pages], np.int64)
    blocks = cache[pages].astype(np.float64)           # [page][Hkv][slot][D]
    flat = blocks.transpose(0, 2, 1, 3).reshape(n_pages * P, cache.shape[1], cache.shape[3])
    return flat[:seq_len]


# ----------------------------------------------------------------------------- attention
def _softmax_rows(s: np.ndarray) -> np.ndarray:
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def paged_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    page_table: np.ndarray, q_starts: np.ndarray, seq_lens: np.ndarray,
                    num_kv_heads: int, scale: Optional[float] = None,
                    row_block: int = 64) -> np.ndarray:
    """Causal GQA attention of every new token, float64 ``[T][Hq][D]``.

    For sequence ``b`` with ``n`` new tokens, token ``i`` sits at ``pos = seq_lens[b] - n + i``
    and query head ``h`` reads KV head ``h // (Hq / Hkv)``:
    ``out = softmax(K[0..pos] q * scale) V[0..pos]`` with ``scale = 1/sqrt(D)`` by default.
    Tokens are taken ``row_block`` at a time only to bound memory; each row is the plain
    definition (one matrix product for the scores, one for the output).
    """
    T, Hq, D = q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.empty((T, Hq, D), np.float64)
    for b in range(len(seq_lens)):
        r0, r1 = int(q_starts[b]), int(q_starts[b + 1])
        if r1 == r0:
            continue
        L = int(seq_lens[b])
        K = gather_kv(k_cache, page_table[b], L)
        V = gather_kv(v_cache, page_table[b], L)
        _causal_rows(q, K, V, r0, r1, num_kv_heads, sc, row_block, out)
    return out


def _causal_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, r0: int, r1: int,
                 num_kv_heads: int, sc: float, row_block: int, out: np.ndarray) -> None:
    """Rows ``r0 .. r1-1`` of ``q`` are the last ``r1 - r0`` positions of one sequence whose
    keys and values are ``K``, ``V`` ``[L][Hkv][D]`` float64; writes their outputs."""
    D = q.shape[2]
    G = q.shape[1] // num_kv_heads
    first = K.shape[0] - (r1 - r0)
    for t0 in range(r0, r1, row_block):
        t1 = min(t0 + row_block, r1)
        pos = first + np.arange(t0 - r0, t1 - r0)            # absolute positions
        nk = int(pos[-1]) + 1                                 # keys any row may see
        masked = np.arange(nk)[None, :] > pos[:, None]        # [rows][keys]
        mask_rows = np.repeat(masked, G, axis=0)                # row = token * G + head
        for g in range(num_kv_heads):
            Qg = q[t0:t1, g * G:(g + 1) * G, :].astype(np.float64).reshape(-1, D)
            S = (Qg @ K[:nk, g, :].T) * sc
            S[mask_rows] = -np.inf
            W = _softmax_rows(S)
            out[t0:t1, g * G:(g + 1) * G, :] = (W @ V[:nk, g, :]).reshape(t1 - t0, G, D)


def varlen_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_starts: np.ndarray,
                     k_starts: np.ndarray, num_kv_heads: int, scale: Optional[float] = None,
                     row_block: int = 64) -> np.ndarray:
    """The same causal GQA attention with dense keys: ``k``, ``v`` ``[total_k][Hkv][D]``,
    sequence ``b`` owning rows ``k_starts[b] .. k_starts[b+1]-1``, its queries being its last
    ``q_starts[b+1] - q_starts[b]`` positions. float64 ``[T][Hq][D]``.

    A trainer computes this form; the sampler computes the paged one, and on-policy training
    needs the two to agree (xitu-tech.com report, section 强化学习的突破). Mathematically it is
    ``paged_attention`` with the sequence's pages laid end to end.
    """
    T, Hq, D = q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.empty((T, Hq, D), np.float64)
    for b in range(len(k_starts) - 1):
        r0, r1 = int(q_starts[b]), int(q_starts[b + 1])
        if r1 == r0:
            continue
        k0, k1 = int(k_starts[b]), int(k_starts[b + 1])
        _causal_rows(q, k[k0:k1].astype(np.float64), v[k0:k1].astype(np.float64), r0, r1,
                     num_kv_heads, sc, row_block, out)
    return out


def paged_attention_rows(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                         page_table: np.ndarray, q_starts: np.ndarray, seq_lens: np.ndarray,
                         num_kv_heads: int, rows: Iterable[Tuple[int, int]],
                         scale: Optional[float] = None) -> np.ndarray:
    """The same definition for selected ``(token, q_head)`` rows only, float64 ``[n][D]``.

    Used at full workload sizes, where only sampled outputs are checked one by one.
    """
    T, Hq, D = q.shape
    G = Hq // num_kv_heads
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    starts = np.asarray(q_starts, np.int64)
    rows = list(rows)
    out = np.empty((len(rows), D), np.float64)
    cache = {}
    for n, (t, h) in enumerate(rows):
        b = int(np.searchsorted(starts, t, side="right") - 1)
        L = int(seq_lens[b])
        pos = L - int(starts[b + 1] - starts[b]) + (t - int(starts[b]))
        g = h // G
        if (b, g) not in cache:
            cache.clear()
            cache[(b, g)] = (gather_kv(k_cache, page_table[b], L)[:, g, :],
                             gather_kv(v_cache, page_table[b], L)[:, g, :])
        K, V = cache[(b, g)]
        s = K[: pos + 1] @ q[t, h].astype(np.float64) * sc
        w = np.exp(s - s.max())
        out[n] = (w / w.sum()) @ V[: pos + 1]
    return out


# ----------------------------------------------------------------------------- split and fold
def split_bounds(pos: int, split_size: int) -> List[Tuple[int, int]]:
    """Key ranges of the fixed-size splits of a row at absolute position ``pos``.

    The split *size* is fixed, not the number of splits (xitu-tech.com report, section
    构建确定性解决方案, attention item; neican.ai insight page, section 技术原理与创新点解析).
    Splits are aligned to absolute position 0: split ``j`` is ``[j S, min(j S + S, pos + 1))``
    for ``j = 0 .. pos // S``, so the decomposition depends on ``pos`` and ``S`` only.
    """
    return [(j * split_size, min(j * split_size + split_size, pos + 1))
            for j in range(pos // split_size + 1)]


def split_partial(s_log2: np.ndarray, v: np.ndarray) -> Tuple[float, float, np.ndarray]:
    """Softmax state of one split: running max ``m``, ``l = sum 2^(s - m)``, ``acc = sum 2^(s - m) v``.

    ``s_log2`` are scores in base-2 units (``q.k * scale * log2(e)``) for the split's keys.
    """
    m = float(np.max(s_log2))
    p = np.exp2(s_log2 - m)
    return m, float(p.sum()), p @ v


def fold(partials: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Combine split states in ascending split order, starting from split 0, then normalise.

    ``M' = max(M, m_j)``, ``L = L 2^(M - M') + l_j 2^(m_j - M')``,
    ``A = A 2^(M - M') + acc_j 2^(m_j - M')``; the output is ``A / L``. The order is fixed so
    that the reduction is the same however many query tokens are processed at once
    (neican.ai insight page, section 技术原理与创新点解析, batch-invariant attention item).
    """
    M, L, A = partials[0][0], partials[0][1], np.array(partials[0][2], np.float64)
    for m, l, acc in partials[1:]:
        Mn = max(M, m)
        a, b = 2.0 ** (M - Mn), 2.0 ** (m - Mn)
        L = L * a + l * b
        A = A * a + acc * b
        M = Mn
    return A / L


def split_fold_attention(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, pos: int,
                         split_size: int, scale: Optional[float] = None) -> np.ndarray:
    """One row by fixed-size splits and the ascending fold, float64 (pins the fold's algebra)."""
    D = q_row.shape[-1]
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    c = sc * math.log2(math.e)
    q64 = q_row.astype(np.float64)
    parts = []
    for k0, k1 in split_bounds(pos, split_size):
        s = (K[k0:k1].astype(np.float64) @ q64) * c
        parts.append(split_partial(s, V[k0:k1].astype(np.float64)))
    return fold(parts)
