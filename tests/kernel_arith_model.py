"""Numpy model of the per-row arithmetic of the GPU attention path (test infrastructure).

It reproduces, in fp32 numpy, the steps every query row takes on the device, so that the
accuracy of a choice made inside the kernels (here: when the PV product adds the second bf16
term of P) can be studied over whole workloads on the CPU:

* scores ``x = q . k`` in fp32 (the device sums the bf16 products inside an MFMA in a
  hardware-defined order; any order gives the same result to fp32 rounding, far below what
  is studied here), scaled by ``c = scale * log2(e)``;
* keys in fixed splits of S absolute positions from 0, each in 32-key sub-tiles, masked keys
  at ``-inf``; lane ``g`` of a row holds keys ``16 kb + 4 g + r`` (kb < 2, r < 4);
* a lazy reference maximum: set from the split's first sub-tile, raised (with
  ``acc *= 2^(m - m')``) only when a sub-tile's row max exceeds it by more than 8;
* ``p = 2^(fma(x, c, -m))``, ``P_hi = bf16(p)`` and, where the rule asks for it,
  ``P_lo = bf16(p - P_hi)``, both multiplied into V with fp32 accumulation (hi first, then lo);
  the lane's l is the carried part (0 at a split start, else ``l alpha``) plus its P_hi values
  two at a time in a fixed order, then its P_lo values the same way, so l sums exactly the
  weights the accumulator received;
* the split partials folded in ascending order with a lazy row reference: M is raised to the
  split's m (``a = 2^(M - m), b = 1``) only when m exceeds it by more than 8, else
  ``a = 1, b = 2^(m - M)``; ``L = fma(l, b, L a), A = fma(acc, b, A a)``.

Rules for the second bf16 term (``rule``):
  ``"kernel"``   the rule the kernels apply: rows at positions below 1024, and every key
                 of a split from the sub-tile on where some lane of the row holds a scaled
                 score more than 7 above the mean of the row's unmasked scaled scores in the
                 split's first sub-tile (the split is peaked; the flag stays set for the rest
                 of the split);
  ``"position"`` rows at positions below 1024 only;
  ``"never"`` / ``"always"``.

The model imports nothing from the HIP library and is not the oracle: the exact reference
in the tests is the float64 definition.
"""

from __future__ import annotations

import numpy as np

from synth import bf16_round

F32 = np.float32
NEG_MAX = F32(-3.4028234663852886e38)
LAZY = F32(8.0)
LO_KEYS = 1024
GAP = F32(7.0)


def _fma(a, b, c):
    """fp32 fused multiply-add (one rounding): the product of two fp32 values is exact in
    float64, so one float64 add and one rounding to fp32 match the device's fma except in
    double-rounding corner cases, which do not matter at the accuracy studied here."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(F32)


def _pair_sum(v):
    """Sum over the last axis of length 4 as the xor butterfly adds it: (v0 + v1) + (v2 + v3)."""
    return ((v[..., 0] + v[..., 1]).astype(F32) + (v[..., 2] + v[..., 3]).astype(F32)).astype(F32)


def attend_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray,
                split: int = 256, rule: str = "kernel", scale: float | None = None,
                stats: dict | None = None) -> np.ndarray:
    """fp32 outputs ``[R][D]`` of query rows ``q [R][D]`` at absolute positions ``pos [R]``
    over the keys and values ``K, V [L][D]`` of one sequence (row r sees keys 0..pos[r]).
    ``stats`` (optional dict) receives ``lanes`` (lane sub-tiles holding an unmasked key) and
    ``lo_lanes`` (those among them that add the second bf16 term)."""
    q = np.asarray(q, F32)
    K = np.asarray(K, F32)
    V = np.asarray(V, F32)
    pos = np.asarray(pos, np.int64)
    R, D = q.shape
    L = K.shape[0]
    sc = (1.0 / np.sqrt(D)) if scale is None else scale
    c = F32(sc * 1.4426950408889634)
    NS = split // 32
    J = (max(L, int(pos.max()) + 1) + split - 1) // split
    Lp = J * split
    Kp = np.zeros((Lp, D), F32)
    Vp = np.zeros((Lp, D), F32)
    Kp[:L], Vp[:L] = K, V
    X = (q @ Kp.T).astype(F32)
    X = np.where(np.arange(Lp)[None, :] <= pos[:, None], X, F32(-np.inf)).astype(F32)
    # [row][split][sub-tile][kb][g][r]: lane g holds keys 16 kb + 4 g + r of a sub-tile
    X = X.reshape(R, J, NS, 2, 4, 4)
    Vs = Vp.reshape(J, NS, 32, D)
    lo_pos = np.broadcast_to((pos < LO_KEYS)[:, None, None], (R, J, 4)) if rule != "never" else \
        np.zeros((R, J, 4), bool)
    m = np.full((R, J), NEG_MAX, F32)
    l_lane = np.zeros((R, J, 4), F32)
    acc = np.zeros((R, J, D), F32)
    lo_split = np.zeros((R, J), bool)
    with np.errstate(invalid="ignore", over="ignore"):
        for t in range(NS):
            x = X[:, :, t]                                       # [R][J][kb][g][r]
            lane_max = x.max(axis=(2, 4))                        # [R][J][g]
            rm = lane_max.max(axis=2)
            mt = (rm * c).astype(F32)
            if t == 0:
                mnew = np.maximum(mt, NEG_MAX).astype(F32)
                alpha = np.ones((R, J), F32)
                fin = np.isfinite(x)
                xs = np.where(fin, x, F32(0))
                lane_sum = np.zeros((R, J, 4), F32)
                lane_cnt = np.zeros((R, J, 4), F32)
                for kb in range(2):
                    for r in range(4):
                        lane_sum = (lane_sum + xs[:, :, kb, :, r]).astype(F32)
                        lane_cnt = (lane_cnt + fin[:, :, kb, :, r].astype(F32)).astype(F32)
                s = _pair_sum(lane_sum)
                n = _pair_sum(lane_cnt)
                # threshold: mean of the scaled scores + 7 (NaN when no score is unmasked); the
                # device multiplies by v_rcp_f32(n), within an ulp of the quotient used here
                thr = ((s * c).astype(F32) / n).astype(F32)
                thr = (thr + GAP).astype(F32)
                lo_split = np.zeros((R, J), bool)
            else:
                need = mt > (m + LAZY).astype(F32)
                mnew = np.where(need, mt, m).astype(F32)
                alpha = np.where(need, np.exp2(np.where(need, m - mt, 0).astype(F32)), F32(1)).astype(F32)
            p = np.exp2(_fma(x, c, -mnew[:, :, None, None, None])).astype(F32)
            p = np.where(np.isnan(p), F32(0), p).astype(F32)
            l_lane = np.zeros_like(l_lane) if t == 0 else (l_lane * alpha[:, :, None]).astype(F32)
            acc = np.zeros_like(acc) if t == 0 else (acc * alpha[:, :, None]).astype(F32)
            # sticky peaked flag: some lane of the row above the threshold
            lo_split = lo_split | ((lane_max * c).astype(F32) > thr[:, :, None]).any(axis=2)
            if rule == "kernel":
                lo_lane = lo_pos | lo_split[:, :, None]
            elif rule == "position":
                lo_lane = lo_pos
            elif rule == "always":
                lo_lane = np.ones((R, J, 4), bool)
            elif rule == "never":
                lo_lane = np.zeros((R, J, 4), bool)
            else:
                raise ValueError(rule)
            if stats is not None:
                live = np.isfinite(lane_max)
                stats["lanes"] = stats.get("lanes", 0) + int(live.sum())
                stats["lo_lanes"] = stats.get("lo_lanes", 0) + int((live & lo_lane).sum())
            ph = bf16_round(p)
            pl = np.where(lo_lane[:, :, None, :, None], bf16_round((p - ph).astype(F32)), F32(0)).astype(F32)
            # the lane's l: its P_hi values, then its P_lo values, two at a time in the order
            # (kb 0, r 0-1), (kb 0, r 2-3), (kb 1, r 0-1), (kb 1, r 2-3)
            for w in (ph, pl):
                wl = w.transpose(0, 1, 3, 2, 4)                  # [R][J][g][kb][r]
                for kb in range(2):
                    for r in (0, 2):
                        pair = (wl[:, :, :, kb, r] + wl[:, :, :, kb, r + 1]).astype(F32)
                        l_lane = (l_lane + pair).astype(F32)
            # back to key order 16 kb + 4 g + r
            ph_k = ph.reshape(R, J, 32)
            pl_k = pl.reshape(R, J, 32)
            acc = (acc + np.einsum("rjk,jkd->rjd", ph_k, Vs[:, t], optimize=True)).astype(F32)
            if pl_k.any():
                acc = (acc + np.einsum("rjk,jkd->rjd", pl_k, Vs[:, t], optimize=True)).astype(F32)
            m = mnew
        l_row = _pair_sum(l_lane)
        # ascending fold of the splits that start at or before the row's position
        valid = (np.arange(J)[None, :] * split) <= pos[:, None]
        M = np.full(R, -np.inf, F32)
        Lr = np.zeros(R, F32)
        A = np.zeros((R, D), F32)
        for j in range(J):
            ok = valid[:, j]
            mj = np.where(ok, m[:, j], NEG_MAX).astype(F32)
            lj = np.where(ok, l_row[:, j], F32(0)).astype(F32)
            aj = np.where(ok[:, None], acc[:, j], F32(0)).astype(F32)
            up = mj > (M + LAZY).astype(F32)
            e = np.exp2(np.where(up, M - mj, mj - M).astype(F32)).astype(F32)
            a = np.where(up, e, F32(1)).astype(F32)
            b = np.where(up, F32(1), e).astype(F32)
            Lr = _fma(lj, b, (Lr * a).astype(F32))
            A = _fma(aj, b[:, None], (A * a[:, None]).astype(F32))
            M = np.where(up, mj, M).astype(F32)
    return (A / Lr[:, None]).astype(F32)


def exact_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray,
               scale: float | None = None) -> np.ndarray:
    """float64 ``softmax(q K^T scale) V`` of each row over keys 0..pos[r] (the definition)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    sc = (1.0 / np.sqrt(q.shape[1])) if scale is None else scale
    S = (q @ K.T) * sc
    S = np.where(np.arange(K.shape[0])[None, :] <= np.asarray(pos)[:, None], S, -np.inf)
    w = np.exp(S - S.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ V
