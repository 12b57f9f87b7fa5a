"""Decode with the page update folded in (bi_attn_decode_append) against the separate calls (GPU).

bi_attn_decode_append must leave the same bits as bi_kv_page_update (one token per sequence)
followed by bi_attn_decode: in the outputs, and in every byte of both caches. Checked for each
decode kernel form (bf16 and fp32, head dim 128 and 64, GQA groups 8 to 64), for lengths on
both sides of page (16), sub-tile (32) and split (256) boundaries, and for the documented
exceptions: a new token whose page is absent (row NaN, nothing written either way), a length
past max_seq_len and a length of 0 (row NaN; the folded form writes no slot for them). The
two-phase form (append partials, then combine) must give the one-call bits.
"""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
from synth import CONFIG_SHAPES, AttnShape, SeqSpec, build_batch, token_values
from gpu_harness import (assert_bitwise, assert_parity, cfg_for, decode_workspace, oracle_out,
                         page_update, to_device)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513, 4096, 4097]


def _append(cfg, d, max_seq_len, two_phase=False):
    B = d.seq_lens.shape[0]
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda")
    ws = decode_workspace(cfg, B, max_seq_len)
    if two_phase:
        bi.bi_attn_decode_append_partials(cfg, d.q, d.k_new, d.v_new, d.k_cache, d.v_cache,
                                          d.page_table, d.seq_lens, max_seq_len, ws)
        bi.bi_attn_decode_combine(cfg, d.seq_lens, max_seq_len, out, ws)
    else:
        bi.bi_attn_decode_append(cfg, d.q, d.k_new, d.v_new, d.k_cache, d.v_cache, d.page_table,
                                 d.seq_lens, max_seq_len, out, ws)
    return out


def _separate(cfg, d, max_seq_len):
    page_update(cfg, d)
    B = d.seq_lens.shape[0]
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda")
    bi.bi_attn_decode(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens, max_seq_len, out,
                      decode_workspace(cfg, B, max_seq_len))
    return out


SHAPES = [CONFIG_SHAPES["decode_bf16"],                   # bf16, D 128, group 8
          AttnShape(64, 2, 128, 16, 256, "bf16"),         # group 32
          AttnShape(64, 1, 64, 16, 256, "bf16"),          # D 64, group 64
          AttnShape(16, 2, 128, 16, 256, "f32"),          # fp32, D 128
          AttnShape(16, 4, 64, 16, 32, "f32")]            # fp32, D 64, split 32


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_append_equals_update_then_decode(si):
    shape = SHAPES[si]
    cfg = cfg_for(shape)
    rng = np.random.default_rng([91, si])
    lens = EDGE_LENS + [int(x) for x in rng.integers(1, 8193, 13)]
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)], seed=92 + si,
                     page_seed=93 + si)
    print(f"CASE append shape {si}: {shape}, batch {len(lens)}", flush=True)
    d1, d2 = to_device(bt, cfg), to_device(bt, cfg)
    mx = bt.max_seq_len
    ref = _separate(cfg, d1, mx)
    got = _append(cfg, d2, mx)
    assert_bitwise(got, ref, "append vs page update + decode: outputs")
    assert_bitwise(d2.k_cache, d1.k_cache, "append vs page update: K cache")
    assert_bitwise(d2.v_cache, d1.v_cache, "append vs page update: V cache")
    # the two-phase form, on caches that already hold the tokens (rewritten with the same bits)
    got2 = _append(cfg, d2, mx, two_phase=True)
    assert_bitwise(got2, ref, "append partials + combine vs one append call")
    assert_bitwise(d2.k_cache, d1.k_cache, "second append: K cache")
    if si == 0:
        assert_parity(got.cpu().numpy(), oracle_out(bt), "append vs oracle")


def test_append_steps_then_decode_reads_written_slots():
    """Three consecutive appends per sequence, each step's token written by the previous call
    and read from the cache by the next: outputs equal the separate calls at every step."""
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg = cfg_for(shape)
    lens0 = [1, 14, 15, 30, 254, 255, 1000, 4094]
    steps = 3
    # the batch of the last step, whose pages hold every position; earlier steps use shorter
    # lengths over the same table and NaN-poisoned slots past them
    bt = build_batch(shape, [SeqSpec(i, L + steps - 2, 1) for i, L in enumerate(lens0)],
                     seed=94, page_seed=95)
    d1, d2 = to_device(bt, cfg), to_device(bt, cfg)
    # poison the slots of the positions the steps write, so every later read of them sees what
    # an earlier call of the same form wrote
    for i, L in enumerate(lens0):
        for p in range(L - 1, L + steps - 1):
            pg = int(bt.page_table[i, p // 16])
            for d in (d1, d2):
                d.k_cache[pg, :, p % 16] = float("nan")
                d.v_cache[pg, :, p % 16] = float("nan")

    def rows(tensor, heads, k):
        return torch.stack([torch.from_numpy(token_values(94, i, tensor, L + k - 1, L + k, heads, 128,
                                                          "bf16")[0])
                            for i, L in enumerate(lens0)]).to("cuda", torch.bfloat16)

    for k in range(steps):
        sl = torch.tensor([L + k for L in lens0], dtype=torch.int32, device="cuda")
        kn, vn, q = rows("k", 4, k), rows("v", 4, k), rows("q", 32, k)
        mx = int(sl.max())
        for d in (d1, d2):
            d.seq_lens, d.k_new, d.v_new, d.q = sl, kn, vn, q
            d.q_starts = torch.arange(len(lens0) + 1, dtype=torch.int32, device="cuda")
        ref = _separate(cfg, d1, mx)
        got = _append(cfg, d2, mx)
        assert_bitwise(got, ref, f"step {k}: outputs")
        assert_bitwise(d2.k_cache, d1.k_cache, f"step {k}: K cache")
        assert_bitwise(d2.v_cache, d1.v_cache, f"step {k}: V cache")
        assert torch.isfinite(got).all()


def test_append_documented_exceptions():
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg = cfg_for(shape)
    lens = [100, 257, 3000, 33, 700, 16]
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)], seed=96, page_seed=97)
    # sequence 1: the new token's page is absent from the table
    bt.page_table[1, (lens[1] - 1) // 16] = -1
    # sequence 2 (3000 tokens): length past max_seq_len; sequence 5: length 0
    mx = 2999
    bt.seq_lens[5] = 0
    d1, d2 = to_device(bt, cfg), to_device(bt, cfg)
    k0 = d2.k_cache.clone()
    ref = _separate(cfg, d1, mx)
    got = _append(cfg, d2, mx)
    nan_rows = [1, 2, 5]
    assert torch.isnan(got[nan_rows]).all() and torch.isnan(ref[nan_rows]).all()
    ok = [0, 3, 4]
    assert_bitwise(got[ok], ref[ok], "valid rows")
    # sequence 2 (3000 > max_seq_len): the separate page update wrote its slot, the folded form
    # leaves it; every other byte of the caches is equal
    pg = int(bt.page_table[2, 2999 // 16])
    slot = (pg, slice(None), 2999 % 16)
    assert_bitwise(d2.k_cache[slot], k0[slot], "skipped slot unchanged")
    d2.k_cache[slot] = d1.k_cache[slot]
    d2.v_cache[slot] = d1.v_cache[slot]
    assert_bitwise(d2.k_cache, d1.k_cache, "K cache outside the skipped slot")
    assert_bitwise(d2.v_cache, d1.v_cache, "V cache outside the skipped slot")
