"""Test-side glue: synthetic batches on the device, library calls, oracle comparison.

Imports both the binding (to run the HIP path) and the oracle (to check it); the two never
see each other's code. Everything here is test infrastructure.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

import invariant_attention_amd as bi
import oracle
from synth import AttnShape, Batch

TOL_MAX_ABS = 2e-3     # parity bar against the fp64 oracle (fp32 outputs, N(0,1) inputs)
TOL_MEAN_ABS = 2e-4


def cfg_for(shape: AttnShape, policy: int = bi.BI_SPLIT_FIXED, split: Optional[int] = None) -> bi.AttnConfig:
    return bi.AttnConfig(shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.page_size,
                         split or shape.split_size, bi.BI_BF16 if shape.dtype == "bf16" else bi.BI_F32,
                         0.0, policy)


def dev_tensor(x: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(dtype)


@dataclass
class DevBatch:
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    q_starts: torch.Tensor
    max_q_len: int
    max_seq_len: int


def to_device(bt: Batch, cfg: bi.AttnConfig) -> DevBatch:
    dt = cfg.torch_dtype
    return DevBatch(
        q=dev_tensor(bt.q, dt), k_new=dev_tensor(bt.k_new, dt), v_new=dev_tensor(bt.v_new, dt),
        k_cache=dev_tensor(bt.k_pool, dt), v_cache=dev_tensor(bt.v_pool, dt),
        page_table=dev_tensor(bt.page_table, torch.int32),
        seq_lens=dev_tensor(bt.seq_lens, torch.int32),
        q_starts=dev_tensor(bt.q_starts, torch.int32),
        max_q_len=bt.max_q_len, max_seq_len=bt.max_seq_len)


def page_update(cfg: bi.AttnConfig, d: DevBatch) -> None:
    bi.bi_kv_page_update(cfg, d.k_new, d.v_new, d.q_starts, d.seq_lens, d.page_table,
                         d.k_cache, d.v_cache)


def run_prefill(cfg: bi.AttnConfig, d: DevBatch, update: bool = True) -> torch.Tensor:
    if update:
        page_update(cfg, d)
    out = torch.full((d.q.shape[0], cfg.num_q_heads, cfg.head_dim), float("nan"),
                     device=d.q.device, dtype=torch.float32)
    bi.bi_attn_prefill(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.q_starts, d.seq_lens,
                       d.max_q_len, d.max_seq_len, out)
    return out


def decode_workspace(cfg: bi.AttnConfig, batch: int, max_seq_len: int) -> torch.Tensor:
    nbytes = bi.bi_attn_workspace_bytes(cfg, batch, max_seq_len)
    ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda")
    ws.fill_(float("nan"))   # poisoned: any read of an unwritten partial shows up
    return ws


def run_decode(cfg: bi.AttnConfig, d: DevBatch, update: bool = True) -> torch.Tensor:
    """All sequences must have exactly one new token."""
    if update:
        page_update(cfg, d)
    B = d.seq_lens.shape[0]
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), device=d.q.device,
                     dtype=torch.float32)
    ws = decode_workspace(cfg, B, d.max_seq_len)
    bi.bi_attn_decode(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens, d.max_seq_len,
                      out, ws)
    return out


def oracle_out(bt: Batch) -> np.ndarray:
    kc, vc = bt.k_pool.copy(), bt.v_pool.copy()
    oracle.kv_page_update(bt.k_new, bt.v_new, bt.q_starts, bt.seq_lens, bt.page_table, kc, vc)
    return oracle.paged_attention(bt.q, kc, vc, bt.page_table, bt.q_starts, bt.seq_lens,
                                  bt.shape.num_kv_heads)


def oracle_rows(bt: Batch, rows: Sequence[Tuple[int, int]]) -> np.ndarray:
    kc, vc = bt.k_pool.copy(), bt.v_pool.copy()
    oracle.kv_page_update(bt.k_new, bt.v_new, bt.q_starts, bt.seq_lens, bt.page_table, kc, vc)
    return oracle.paged_attention_rows(bt.q, kc, vc, bt.page_table, bt.q_starts, bt.seq_lens,
                                       bt.shape.num_kv_heads, rows)


def assert_parity(got: np.ndarray, ref: np.ndarray, what: str = "") -> Tuple[float, float]:
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= TOL_MAX_ABS and mean <= TOL_MEAN_ABS, f"{what}: max-abs {mx:.3e}, mean-abs {mean:.3e}"
    return mx, mean


def bits(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().contiguous().view(torch.int32).numpy()


def assert_bitwise(a: torch.Tensor, b: torch.Tensor, what: str = "") -> None:
    """Zero differing bits; on failure report the XOR popcount and the first differing index."""
    ba, bb = bits(a), bits(b)
    if np.array_equal(ba, bb):
        return
    x = np.bitwise_xor(ba, bb).view(np.uint32)
    pop = int(np.unpackbits(x.view(np.uint8)).sum())
    first = np.argwhere(x != 0)[0].tolist()
    raise AssertionError(f"{what}: {int((x != 0).sum())} words differ, {pop} bits; first at {first}")
