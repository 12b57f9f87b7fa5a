"""Batch-invariant RMSNorm on the GPU: parity with the fp64 oracle and zero differing bits across
row counts, row positions and in-place use (GPU)."""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
import oracle
from synth import norm_inputs
from gpu_harness import assert_bitwise

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# Bars (fp32 accumulation of N(0,1) squares, then one division, one square root and two
# products): fp32 outputs within 5e-5 of the fp64 value relative to max(|ref|, 1); bf16 outputs
# add the final rounding to bf16 (half a unit in the 8-bit significand, 2^-9 relative), so
# |err| <= 2^-8 |ref| + 1e-6.
TOL_F32 = 5e-5


def _dt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def run(x, w, eps, out=None):
    y = torch.empty_like(x) if out is None else out
    bi.bi_rmsnorm(x, w, y, eps)
    torch.cuda.synchronize()
    return y


def check_parity(got, ref, dtype, what):
    got = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), what
    err = np.abs(got - ref)
    if dtype == "bf16":
        bad = err > 2.0 ** -8 * np.abs(ref) + 1e-6
        assert not bad.any(), f"{what}: {int(bad.sum())} elements past the bf16 bar, max {err.max():.3e}"
    else:
        rel = float((err / np.maximum(np.abs(ref), 1.0)).max())
        assert rel <= TOL_F32, f"{what}: relative error {rel:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", [(1, 8), (3, 64), (257, 4096), (17, 5120), (9, 8192),
                                         (5, 16384), (2, 20480)])
def test_rmsnorm_parity(dtype, rows, hidden):
    if dtype == "f32" and hidden % 4:
        pytest.skip("fp32 rows are whole 16-byte chunks")
    print("CASE rmsnorm", dtype, rows, hidden, flush=True)
    x, w = norm_inputs(41, rows, hidden, dtype)
    eps = 1e-6
    xd, wd = torch.from_numpy(x).cuda().to(_dt(dtype)), torch.from_numpy(w).cuda().to(_dt(dtype))
    y = run(xd, wd, eps)
    check_parity(y, oracle.rmsnorm(x, w, eps), dtype, f"rmsnorm {dtype} {rows}x{hidden}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm_rows_are_batch_invariant(dtype):
    """Each row's bits do not depend on how many rows there are, where the row sits, or whether
    the call writes in place."""
    hidden = 4096
    print("CASE rmsnorm invariance", dtype, flush=True)
    x, w = norm_inputs(42, 2048, hidden, dtype)
    xd, wd = torch.from_numpy(x).cuda().to(_dt(dtype)), torch.from_numpy(w).cuda().to(_dt(dtype))
    full = run(xd, wd, 1e-5)
    for rows in (1, 7, 64, 513):
        assert_bitwise(run(xd[:rows].contiguous(), wd, 1e-5), full[:rows], f"first {rows} rows")
    perm = torch.randperm(2048, generator=torch.Generator().manual_seed(3)).cuda()
    assert_bitwise(run(xd[perm].contiguous(), wd, 1e-5), full[perm], "permuted rows")
    for r in (0, 1000, 2047):
        assert_bitwise(run(xd[r:r + 1].contiguous(), wd, 1e-5), full[r:r + 1], f"row {r} alone")
    inplace = xd.clone()
    run(inplace, wd, 1e-5, out=inplace)
    assert_bitwise(inplace, full, "in place")


def test_rmsnorm_rejects_bad_sizes():
    x = torch.zeros((2, 12), dtype=torch.bfloat16, device="cuda")   # 24 bytes per row
    w = torch.zeros(12, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bi.BiAttnError):
        run(x, w, 1e-6)
    x = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
    w = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(bi.BiAttnError):
        run(x, w, -1.0)
