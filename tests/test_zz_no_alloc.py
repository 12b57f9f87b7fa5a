"""The allocation-free decode entry point (GPU): the same bits as bi_attn_decode.

bi_attn_decode_noalloc keeps the split partials in the library's static device array instead
of a caller workspace. Calls in a row, each with a smaller batch or shorter sequences than the
one before (the array keeps the earlier calls' partials, which the next must not read), the first
with rows of more than 32 splits (the row-parallel combine), all bitwise equal to
bi_attn_decode with a NaN-poisoned workspace; a call needing more partials
than the array holds is refused before anything is launched.
"""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
from synth import AttnShape, SeqSpec, build_batch
from gpu_harness import assert_bitwise, cfg_for, page_update, run_decode, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _case(seed, B, lo, hi):
    shape = AttnShape(32, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(lo, hi + 1, B)]
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)], seed=seed,
                     page_seed=seed + 1, extra_pages=3)
    return cfg, bt


def test_noalloc_decode_equals_decode_on_two_calls():
    for seed, B, lo, hi in ((90, 4, 9000, 20000), (91, 48, 128, 8192), (92, 5, 1, 3000)):
        cfg, bt = _case(seed, B, lo, hi)
        d = to_device(bt, cfg)
        ref = run_decode(cfg, d)                   # NaN-poisoned workspace
        out = torch.full_like(ref, float("nan"))
        bi.bi_attn_decode_noalloc(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens,
                                  d.max_seq_len, out)
        assert torch.isfinite(out).all()
        assert_bitwise(out, ref, f"noalloc decode, batch {B}")


def test_noalloc_decode_refuses_past_its_array():
    cfg, bt = _case(93, 2, 100, 200)
    d = to_device(bt, cfg)
    page_update(cfg, d)
    out = torch.zeros((2, 32, 128), device="cuda")
    # 2 sequences claimed up to 2^22 tokens: far more partials than the array holds
    with pytest.raises(bi.BiAttnError) as e:
        bi.bi_attn_decode_noalloc(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens,
                                  1 << 22, out)
    assert e.value.status == bi._lib.BI_EWORKSPACE
    assert int(torch.count_nonzero(out)) == 0, "nothing may be launched"
