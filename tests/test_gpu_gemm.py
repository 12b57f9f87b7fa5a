"""Batch-invariant GEMM on the GPU: parity with the fp64 oracle within the fp32 summation bound,
and zero differing bits across M (GPU)."""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
import oracle
from synth import gemm_inputs
from gpu_harness import assert_bitwise

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run(a, w, out_dtype=torch.float32):
    c = torch.full((a.shape[0], w.shape[0]), float("nan"), dtype=out_dtype, device="cuda")
    bi.bi_gemm(a, w, c)
    torch.cuda.synchronize()
    return c


def check(c, a, w, what):
    """fp32 accumulation of K exact products (bf16 x bf16 fits fp32): |err| <= K 2^-24 (|A| |W|^T)
    in any summation order; a bf16 result adds its rounding, at most half a unit of an 8-bit
    significand: 2^-8 times the fp32 value."""
    ref = oracle.gemm(a, w)
    bound = a.shape[1] * 2.0 ** -24 * (np.abs(a).astype(np.float64) @ np.abs(w).astype(np.float64).T) + 1e-30
    got = c.float().cpu().numpy().astype(np.float64)
    if c.dtype == torch.bfloat16:
        bound = bound + 2.0 ** -8 * (np.abs(ref) + bound)
    assert np.isfinite(got).all(), what
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements past the bound"


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("m,n,k", [(1, 128, 64), (5, 256, 128), (32, 384, 1024), (33, 256, 576),
                                   (64, 128, 4096), (100, 128, 64), (100, 256, 192), (128, 128, 4096),
                                   (300, 384, 576), (257, 1024, 1024), (1, 128, 8192), (16, 256, 8256)])
def test_gemm_parity(out, m, n, k):
    print("CASE gemm", out, m, n, k, flush=True)
    a, w = gemm_inputs(51, m, n, k)
    ad, wd = torch.from_numpy(a).cuda().to(torch.bfloat16), torch.from_numpy(w).cuda().to(torch.bfloat16)
    c = run(ad, wd, torch.bfloat16 if out == "bf16" else torch.float32)
    check(c, a, w, f"gemm {out} {m}x{n}x{k}")


def test_gemm_rows_are_batch_invariant():
    """A row's outputs do not depend on M (the token count) or the row's position: rows computed
    by the skinny kernel (M <= 64) and by the 128 x 128 tiles are compared with each other."""
    m, n, k = 1000, 512, 2048
    print("CASE gemm invariance", flush=True)
    a, w = gemm_inputs(52, m, n, k)
    ad, wd = torch.from_numpy(a).cuda().to(torch.bfloat16), torch.from_numpy(w).cuda().to(torch.bfloat16)
    full = run(ad, wd)
    for rows in (1, 3, 32, 33, 64, 65, 127, 128, 129, 600):
        assert_bitwise(run(ad[:rows].contiguous(), wd), full[:rows], f"first {rows} rows")
    perm = torch.randperm(m, generator=torch.Generator().manual_seed(4)).cuda()
    assert_bitwise(run(ad[perm].contiguous(), wd), full[perm], "permuted rows")
    for r in (0, 500, 999):
        assert_bitwise(run(ad[r:r + 1].contiguous(), wd), full[r:r + 1], f"row {r} alone")
    fb = run(ad, wd, torch.bfloat16)
    assert_bitwise(run(ad[7:8].contiguous(), wd, torch.bfloat16), fb[7:8], "bf16 output row")


def test_gemm_skinny_rows_same_bits():
    """With K >= 8192, up to 16 rows take the skinny kernel (operands straight from memory, no
    LDS); its rows equal, bit for bit, the same rows of a 300-row product (64 x 64 tiles)."""
    m, n, k = 300, 256, 8256
    print("CASE gemm skinny invariance", flush=True)
    a, w = gemm_inputs(55, m, n, k)
    ad, wd = torch.from_numpy(a).cuda().to(torch.bfloat16), torch.from_numpy(w).cuda().to(torch.bfloat16)
    for out in (torch.float32, torch.bfloat16):
        full = run(ad, wd, out)
        for lo, hi in ((0, 16), (0, 17), (150, 151), (284, 300)):
            assert_bitwise(run(ad[lo:hi].contiguous(), wd, out), full[lo:hi], f"rows {lo}..{hi - 1} {out}")


def test_gemm_rejects_bad_sizes():
    a = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bi.BiAttnError):
        run(a, torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda"))    # N % 128
    with pytest.raises(bi.BiAttnError):
        run(torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda"),
            torch.zeros((128, 96), dtype=torch.bfloat16, device="cuda"))       # K % 64


@pytest.mark.parametrize("m,n,k", [(2048, 8192, 256), (2085, 8192, 320), (1040, 8192, 192),
                                   (1040, 4224, 192)])
def test_gemm_large_tile_parity(m, n, k):
    """Shapes with at least 160 tiles of 256 x 256 take the large tile (M = 2085: a ragged last
    tile row; K = 320 and 192: an odd number of 64-wide K steps); N = 4224 (not a multiple of 256)
    takes the 128 x 128 tile: same bound against the oracle."""
    print("CASE gemm large tile", m, flush=True)
    a, w = gemm_inputs(53, m, n, k)
    ad, wd = torch.from_numpy(a).cuda().to(torch.bfloat16), torch.from_numpy(w).cuda().to(torch.bfloat16)
    check(run(ad, wd), a, w, f"gemm f32 {m}x{n}x{k}")
    check(run(ad, wd, torch.bfloat16), a, w, f"gemm bf16 {m}x{n}x{k}")


def test_gemm_rows_same_bits_across_tile_shapes():
    """Rows of a product that takes the 256 x 256 tiles equal, bit for bit, the same rows computed
    in products that take the 128 x 128 tiles (M = 600), the 64 x 64 tiles (M = 300) and the
    64 x 64 tiles at M = 1, 7 (K = 512: below the skinny kernel's K)."""
    m, n, k = 2085, 8192, 512
    print("CASE gemm tile shapes", flush=True)
    a, w = gemm_inputs(54, m, n, k)
    ad, wd = torch.from_numpy(a).cuda().to(torch.bfloat16), torch.from_numpy(w).cuda().to(torch.bfloat16)
    for out in (torch.float32, torch.bfloat16):
        full = run(ad, wd, out)
        assert_bitwise(run(ad[:300].contiguous(), wd, out), full[:300], f"first 300 rows {out}")
        assert_bitwise(run(ad[1000:1600].contiguous(), wd, out), full[1000:1600], f"rows 1000..1599 {out}")
        assert_bitwise(run(ad[2078:].contiguous(), wd, out), full[2078:], f"last 7 rows {out}")
        for r in (0, 1041, 2084):
            assert_bitwise(run(ad[r:r + 1].contiguous(), wd, out), full[r:r + 1], f"row {r} alone {out}")
