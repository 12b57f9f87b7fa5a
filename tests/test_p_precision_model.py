"""Accuracy of the kernels' P precision rule over the workloads' distributions (CPU only).

``kernel_arith_model.attend_rows`` reproduces the device arithmetic row by row (lazy
reference maximum, bf16 P with the second bf16 term where the rule asks for it, fp32
accumulation, ascending fold of fixed 256-key splits). Here it runs on rows drawn like the
decode, chunked-prefill, long-context (q x 4) and mixed-trace workloads, eight seeds each, plus
peaked rows at 1024-4096 keys and a sweep of softmax sharpness, against the float64
definition. The rule must keep every case within max-abs 1e-3 (half the parity bar of 2e-3) and
mean-abs 1e-4. The position-only rule that the kernels used before is shown to miss the bar on
peaked rows, which is what the per-split (peaked-split) part of the rule is for.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from kernel_arith_model import attend_rows, exact_rows
from synth import token_values

MAX_ABS = 1e-3
MEAN_ABS = 1e-4
SEEDS = range(8)


def _stream(seed: int, length: int, q_heads: int, q_scale: float, q_lo: int, q_hi: int):
    """Keys and values of KV head 0 of one request and the q rows of its first ``q_heads``
    heads at positions [q_lo, q_hi), bf16 values as the workloads generate them."""
    K = token_values(seed, 0, "k", 0, length, 1, 128, "bf16")[:, 0]
    V = token_values(seed, 0, "v", 0, length, 1, 128, "bf16")[:, 0]
    q = token_values(seed, 0, "q", q_lo, q_hi, q_heads, 128, "bf16", q_scale)
    return q, K, V


def _rows(seed: int, length: int, positions, q_heads: int, q_scale: float = 1.0):
    positions = np.asarray(sorted(set(int(p) for p in positions)), np.int64)
    lo, hi = int(positions.min()), int(positions.max()) + 1
    q, K, V = _stream(seed, length, q_heads, q_scale, lo, hi)
    qr = q[positions - lo].reshape(-1, 128)                  # [pos][head] rows
    pr = np.repeat(positions, q_heads)
    return qr, K, V, pr


def _errors(q, K, V, pos, rule):
    got = attend_rows(q, K, V, pos, rule=rule)
    err = np.abs(got.astype(np.float64) - exact_rows(q, K, V, pos))
    return float(err.max()), float(err.mean())


def _decode_case(seed):
    # decode: context U[128, 8192], one query token, a GQA group of 8 heads
    rng = np.random.default_rng([seed, 2])
    L = int(rng.integers(128, 8193))
    return _rows(3100 + seed, L, [L - 1], 8)


def _prefill_case(seed):
    # chunked prefill: prefix U[0, 16384], chunk U[1, 2048]; 4 tokens of the chunk, 16 heads
    rng = np.random.default_rng([seed, 3])
    pre, n = int(rng.integers(0, 16385)), int(rng.integers(1, 2049))
    toks = pre + rng.integers(0, n, 4)
    return _rows(3200 + seed, pre + n, toks, 16)


def _long_case(seed):
    # long-context decode: 131072 keys, q x 4; 4 heads of the group
    L = 131072
    return _rows(3300 + seed, L, [L - 1], 4, 4.0)


def _trace_case(seed):
    # mixed trace: prompt floor(exp U[ln 64, ln 32768]) plus up to U[16, 1024] outputs;
    # 6 positions across prompt and output, 8 heads
    rng = np.random.default_rng([seed, 5])
    prompt = int(math.floor(math.exp(rng.uniform(math.log(64), math.log(32768)))))
    out = int(rng.integers(16, 1025))
    toks = rng.integers(0, prompt + out, 6)
    return _rows(3400 + seed, prompt + out, toks, 8)


def _peaked_mid_case(seed):
    # q x 4 rows at positions 1024 .. 4096
    rng = np.random.default_rng([seed, 6])
    toks = rng.integers(1024, 4097, 8)
    return _rows(3500 + seed, 4097, toks, 4, 4.0)


CASES = {"decode": _decode_case, "prefill": _prefill_case, "long_q4": _long_case,
         "trace": _trace_case, "q4_1k_4k": _peaked_mid_case}


@pytest.mark.parametrize("name", list(CASES))
def test_rule_keeps_workload_rows_within_half_the_bar(name):
    worst = (0.0, 0.0)
    for seed in SEEDS:
        mx, mean = _errors(*CASES[name](seed), rule="kernel")
        assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{name} seed {seed}: max {mx:.2e} mean {mean:.2e}"
        worst = (max(worst[0], mx), max(worst[1], mean))
    print(f"{name}: worst max-abs {worst[0]:.2e}, mean-abs {worst[1]:.2e} over {len(SEEDS)} seeds")


@pytest.mark.parametrize("q_scale", [1.5, 2.0, 3.0, 8.0])
def test_rule_across_softmax_sharpness(q_scale):
    # rows between 1 and 16384 keys with scores sharper than N(0,1) by q_scale
    for seed in range(4):
        rng = np.random.default_rng([seed, 7, int(q_scale * 10)])
        toks = np.concatenate([rng.integers(0, 1024, 3), rng.integers(1024, 4096, 3),
                               rng.integers(4096, 16384, 3)])
        mx, mean = _errors(*_rows(3600 + seed, 16384, toks, 2, q_scale), rule="kernel")
        assert mx <= MAX_ABS and mean <= MEAN_ABS, f"q x {q_scale} seed {seed}: max {mx:.2e} mean {mean:.2e}"


def test_position_only_rule_misses_peaked_rows():
    # the model sees the effect the rule is there for: single bf16 P past position 1024
    worst = max(_errors(*_peaked_mid_case(seed), rule="position")[0] for seed in range(4))
    assert worst > 2e-3, worst
    # and the P_lo term everywhere is far below the bar (the model's own floor)
    assert _errors(*_peaked_mid_case(0), rule="always")[0] < 1e-4


def test_rule_adds_little_for_unpeaked_long_rows():
    # N(0,1) rows past position 1024 (the prefill and trace workloads' bulk): the second bf16
    # term is rare (a split with a score more than 7 above the first sub-tile's mean, about 4.9
    # standard deviations), so the rule costs those rows almost nothing
    st = {}
    q, K, V, pos = _rows(3700, 16384, np.arange(1024, 16384, 61), 16)
    attend_rows(q, K, V, pos, rule="kernel", stats=st)
    frac = st["lo_lanes"] / st["lanes"]
    assert frac < 0.01, frac
    print(f"N(0,1) rows past 1024: {100 * frac:.2f}% of lane sub-tiles add P_lo")


def test_peaked_rows_with_flat_first_sub_tile():
    """Rows of a q x 4 prefill (1024-token prefix, tokens 1280 .. 1535 of a 3072-token chunk,
    one KV head's 16 query heads: 4096 rows). Some of their splits start with a sub-tile whose
    scores happen to be flat; a peaked-split test on the first sub-tile alone misses those
    (the device then reached 2.4e-3 on this stretch), the test repeated on every sub-tile
    does not."""
    L, kvh = 4096, 3
    K = token_values(61, 0, "k", 0, L, 4, 128, "bf16")[:, kvh]
    V = token_values(61, 0, "v", 0, L, 4, 128, "bf16")[:, kvh]
    q = token_values(61, 0, "q", 1280, 1536, 64, 128, "bf16", 4.0)[:, 16 * kvh:16 * kvh + 16]
    qr = q.reshape(-1, 128)
    pos = np.repeat(np.arange(1280, 1536), 16)
    mx, mean = _errors(qr, K, V, pos, rule="kernel")
    assert mx <= MAX_ABS and mean <= MEAN_ABS, (mx, mean)
