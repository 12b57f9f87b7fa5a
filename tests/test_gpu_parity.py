"""Parity of the HIP path against the fp64 oracle (GPU).

Bar: max-abs <= 2e-3 and mean-abs <= 2e-4 on fp32 outputs for N(0,1) inputs, element by
element at sizes the oracle finishes in seconds (several 32-key sub-tiles and 256-key
splits, ragged tails), and on sampled rows at full workload sizes.
"""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
from synth import CONFIG_SHAPES, AttnShape, SeqSpec, build_batch, token_values
from gpu_harness import (assert_bitwise, assert_parity, cfg_for, oracle_out, oracle_rows,
                         run_decode, run_prefill, to_device)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _print_case(*a):
    print("CASE", *a, flush=True)


def test_tiny_f32_prefill_and_decode_parity():
    shape = CONFIG_SHAPES["tiny_f32"]
    cfg = cfg_for(shape)
    rng = np.random.default_rng(2025)
    seqs = [SeqSpec(0, 128, 16)]
    for r in range(1, 4):
        L = int(rng.integers(16, 257))
        n = int(rng.integers(1, 17))
        seqs.append(SeqSpec(r, L - n, n))
    _print_case("tiny_f32 prefill", seqs)
    bt = build_batch(shape, seqs, seed=2025, page_seed=1, extra_pages=4)
    out = run_prefill(cfg, to_device(bt, cfg)).cpu().numpy()
    assert_parity(out, oracle_out(bt), "tiny_f32 prefill")
    # decode of single tokens
    dseqs = [SeqSpec(s.req, s.seq_len - 1, 1) for s in seqs]
    bt2 = build_batch(shape, dseqs, seed=2025, page_seed=2)
    outd = run_decode(cfg, to_device(bt2, cfg)).cpu().numpy()
    assert_parity(outd, oracle_out(bt2), "tiny_f32 decode")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hq,hkv,d", [(32, 4, 128), (64, 4, 128), (8, 8, 64), (16, 2, 64)])
def test_decode_parity(dtype, hq, hkv, d):
    shape = AttnShape(hq, hkv, d, 16, 256, dtype)
    cfg = cfg_for(shape)
    rng = np.random.default_rng(7)
    lens = [1, 2, 31, 32, 33, 255, 256, 257, 600] + [int(x) for x in rng.integers(128, 2500, 3)]
    seqs = [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)]
    _print_case("decode", dtype, hq, hkv, d)
    bt = build_batch(shape, seqs, seed=11, page_seed=3, extra_pages=5)
    out = run_decode(cfg, to_device(bt, cfg)).cpu().numpy()
    assert_parity(out, oracle_out(bt), f"decode {dtype} {hq}/{hkv}/{d}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hq,hkv,d", [(64, 4, 128), (32, 4, 128), (8, 8, 64), (4, 1, 64)])
def test_prefill_parity(dtype, hq, hkv, d):
    shape = AttnShape(hq, hkv, d, 16, 256, dtype)
    cfg = cfg_for(shape)
    seqs = [SeqSpec(0, 0, 300), SeqSpec(1, 517, 45), SeqSpec(2, 255, 1), SeqSpec(3, 0, 1),
            SeqSpec(4, 1000, 0), SeqSpec(5, 31, 70)]
    _print_case("prefill", dtype, hq, hkv, d)
    bt = build_batch(shape, seqs, seed=12, page_seed=4, extra_pages=3)
    out = run_prefill(cfg, to_device(bt, cfg)).cpu().numpy()
    assert_parity(out, oracle_out(bt), f"prefill {dtype} {hq}/{hkv}/{d}")


def test_q_zero_gives_prefix_mean():
    """Closed form: q = 0 makes every weight exactly 1, so the output is the mean of V."""
    shape = AttnShape(64, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    seqs = [SeqSpec(0, 700, 40), SeqSpec(1, 0, 33)]
    bt = build_batch(shape, seqs, seed=13, page_seed=5)
    bt.q[:] = 0.0
    _print_case("q zero")
    d = to_device(bt, cfg)
    out = run_prefill(cfg, d).cpu().numpy()
    for b, s in enumerate(seqs):
        V = token_values(13, s.req, "v", 0, s.seq_len, 4, 128, "bf16").astype(np.float64)
        r0 = int(bt.q_starts[b])
        for i in range(s.n_new):
            pos = s.cached + i
            mean = V[: pos + 1].mean(axis=0)           # [Hkv][D]
            ref = np.repeat(mean, 16, axis=0)
            np.testing.assert_allclose(out[r0 + i], ref, atol=2e-5, rtol=0)
    bt1 = build_batch(shape, [SeqSpec(0, 739, 1)], seed=13)
    bt1.q[:] = 0.0
    outd = run_decode(cfg, to_device(bt1, cfg)).cpu().numpy()
    V = token_values(13, 0, "v", 0, 740, 4, 128, "bf16").astype(np.float64)
    np.testing.assert_allclose(outd[0], np.repeat(V.mean(axis=0), 16, axis=0), atol=2e-5, rtol=0)


def test_split_edges_single_sequence():
    """Lengths at split and sub-tile edges, decode and prefill, against the oracle."""
    shape = AttnShape(32, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    for L in (1, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 4095, 4096, 4097, 16383,
              16384, 16385):
        bt = build_batch(shape, [SeqSpec(L, L - 1, 1)], seed=14)
        _print_case("edge", L)
        out = run_decode(cfg, to_device(bt, cfg)).cpu().numpy()
        assert_parity(out, oracle_out(bt), f"decode L={L}")
        outp = run_prefill(cfg, to_device(bt, cfg))
        assert_bitwise(outp, torch.from_numpy(out), f"decode vs prefill L={L}")


@pytest.mark.parametrize("d,dtype,hq,hkv", [(128, "bf16", 8, 2), (64, "f32", 8, 2), (64, "bf16", 2, 2)])
def test_long_rows_combine_windows(d, dtype, hq, hkv):
    """Decode with rows of 1 to 200 splits in one call (the combine for rows of more than 32
    splits hands coefficients over in 64-split windows): windows that end exactly, one split
    past a window, a single split; every row bitwise equal to the prefill of the same token,
    sampled rows against the oracle, and rows of invalid length NaN without touching the rest.
    With 2 heads the 14 rows are not a multiple of the 8 XCDs the rows are dealt out to."""
    shape = AttnShape(hq, hkv, d, 16, 256, dtype)
    cfg = cfg_for(shape)
    lens = [100, 256 * 63, 256 * 64, 256 * 64 + 1, 256 * 128, 256 * 128 + 1, 256 * 199 + 77]
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)], seed=61,
                     page_seed=62)
    dd = to_device(bt, cfg)
    _print_case("long rows combine", d, dtype, hq, hkv)
    out = run_decode(cfg, dd)
    outp = run_prefill(cfg, to_device(bt, cfg))
    assert_bitwise(outp, out, "decode (row-parallel combine) vs prefill (in-loop fold)")
    rows = [(r, h) for r in range(len(lens)) for h in (0, hq - 1)]
    ref = oracle_rows(bt, rows)
    got = np.stack([out[r, h].cpu().numpy() for r, h in rows])
    assert_parity(got, ref, "long rows, sampled")
    sl = dd.seq_lens.clone()
    sl[1], sl[4] = 0, bt.max_seq_len + 1
    o2 = torch.full_like(out, 0.0)
    ws = torch.empty(bi.bi_attn_workspace_bytes(cfg, len(lens), bt.max_seq_len) // 4 + 64, device="cuda")
    bi.bi_attn_decode(cfg, dd.q, dd.k_cache, dd.v_cache, dd.page_table, sl, bt.max_seq_len, o2, ws)
    assert torch.isnan(o2[[1, 4]]).all()
    good = [0, 2, 3, 5, 6]
    assert_bitwise(o2[good], out[good], "valid long rows next to invalid ones")


def test_decode_at_one_million_tokens():
    """The largest decode here: one sequence of 2^20 tokens (4096 splits, 64 coefficient windows
    in the long-row combine) beside one of 300001 tokens, decode_bf16 heads: sampled rows against
    the oracle, every row bitwise equal to the prefill of the same token, and the shorter
    sequence alone (other pages, a smaller max_seq_len) bitwise equal to its row of the pair."""
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg = cfg_for(shape)
    _print_case("decode at 2^20 tokens")
    specs = [SeqSpec(0, (1 << 20) - 1, 1), SeqSpec(1, 300000, 1)]
    bt = build_batch(shape, specs, seed=77, page_seed=78)
    out = run_decode(cfg, to_device(bt, cfg))
    rows = [(0, 0), (0, 31), (1, 5)]
    got = np.stack([out[r, h].cpu().numpy() for r, h in rows])
    assert_parity(got, oracle_rows(bt, rows), "decode at 2^20 tokens, sampled rows")
    outp = run_prefill(cfg, to_device(bt, cfg))
    assert_bitwise(outp, out, "decode vs prefill at 2^20 tokens")
    del outp
    alone = build_batch(shape, specs[1:], seed=77, page_seed=79)
    out1 = run_decode(cfg, to_device(alone, cfg))
    assert_bitwise(out1[0], out[1], "300001-token sequence alone vs beside the 2^20-token one")


@pytest.mark.parametrize("seed", [2028, 3028])
def test_long_decode_full_output(seed):
    """The long-context workload whole: 8 sequences of 131072 tokens, 64/4 heads, peaked softmax
    (q x 4): every one of the 8 x 64 output rows against the oracle."""
    shape = CONFIG_SHAPES["long_decode_bf16"]
    cfg = cfg_for(shape)
    L = 131072
    seqs = [SeqSpec(i, L - 1, 1) for i in range(8)]
    _print_case("long decode 8 x 131072, seed", seed)
    bt = build_batch(shape, seqs, seed=seed, page_seed=seed + 1, q_scale=4.0)
    out = run_decode(cfg, to_device(bt, cfg)).cpu().numpy()
    mx, mean = assert_parity(out, oracle_out(bt), f"long decode seed {seed}")
    print(f"long decode seed {seed}: max-abs {mx:.2e}, mean-abs {mean:.2e}")


def test_peaked_prefill_rows_1024_to_4096():
    """q x 4 (peaked softmax) prefill rows at positions 1024 .. 4095 (a 1024-token prefix and a
    3072-token chunk) and a shorter second sequence: every row against the oracle."""
    shape = AttnShape(64, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    seqs = [SeqSpec(0, 1024, 3072), SeqSpec(1, 300, 200)]
    _print_case("peaked prefill 1024..4096")
    bt = build_batch(shape, seqs, seed=61, page_seed=62, extra_pages=3, q_scale=4.0)
    out = run_prefill(cfg, to_device(bt, cfg)).cpu().numpy()
    mx, mean = assert_parity(out, oracle_out(bt), "peaked prefill")
    print(f"peaked prefill: max-abs {mx:.2e}, mean-abs {mean:.2e}")


@pytest.mark.parametrize("bad", ["negative", "past_pool"])
def test_bad_page_entry_gives_nan_rows_only_where_needed(bad):
    """A table entry outside [0, num_pages) is never dereferenced: query rows whose causal
    window reaches that page come out NaN, every other row is bit-identical to a clean run."""
    shape = AttnShape(16, 2, 128, page_size=16, split_size=64, dtype="bf16")
    cfg = cfg_for(shape)
    # sequence 1: 100 cached + 60 new tokens (positions 100..159); page 8 holds keys 128..143
    seqs = [SeqSpec(0, 70, 5), SeqSpec(1, 100, 60), SeqSpec(2, 300, 9)]
    bt = build_batch(shape, seqs, seed=31, page_seed=32, extra_pages=4)
    clean = run_prefill(cfg, to_device(bt, cfg))
    d = to_device(bt, cfg)
    n_pages = d.k_cache.shape[0]
    d.page_table[1, 8] = -7 if bad == "negative" else n_pages + 3
    _print_case("bad page prefill", bad)
    got = run_prefill(cfg, d)
    r0, r1 = bt.token_rows(1)
    pos = np.arange(100, 160)
    need = pos >= 128
    g = got[r0:r1].cpu()
    assert torch.isnan(g[torch.from_numpy(need)]).all(), "rows needing the bad page must be NaN"
    ok_rows = torch.cat([got[:r0], got[r0:r1][torch.from_numpy(~need).cuda()], got[r1:]])
    ok_ref = torch.cat([clean[:r0], clean[r0:r1][torch.from_numpy(~need).cuda()], clean[r1:]])
    assert_bitwise(ok_rows, ok_ref, f"rows not reaching the bad page ({bad})")
    # decode: the last token of each sequence; only sequence 1 reaches page 8
    dseqs = [SeqSpec(0, 74, 1), SeqSpec(1, 159, 1), SeqSpec(2, 308, 1)]
    bd = build_batch(shape, dseqs, seed=33, page_seed=34, extra_pages=4)
    clean_d = run_decode(cfg, to_device(bd, cfg))
    dd = to_device(bd, cfg)
    dd.page_table[1, 8] = -7 if bad == "negative" else dd.k_cache.shape[0] + 3
    _print_case("bad page decode", bad)
    got_d = run_decode(cfg, dd)
    assert torch.isnan(got_d[1]).all()
    assert_bitwise(got_d[[0, 2]], clean_d[[0, 2]], f"decode rows of other sequences ({bad})")


def test_decode_many_sequences_with_invalid_lengths():
    """150 sequences (the work split walks several chunks of 64 sequences); rows whose length is
    0 or above max_seq_len come out NaN, and every other row keeps its bits and its parity."""
    shape = AttnShape(32, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 1500, 150)]
    seqs = [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)]
    bt = build_batch(shape, seqs, seed=42, page_seed=43, extra_pages=8)
    d = to_device(bt, cfg)
    _print_case("decode 150 sequences")
    clean = run_decode(cfg, d)
    bad = [3, 64, 70, 128, 149]
    sl = d.seq_lens.clone()
    for i, r in enumerate(bad):
        sl[r] = 0 if i % 2 == 0 else bt.max_seq_len + 5
    out = torch.full_like(clean, float("nan"))
    ws = torch.empty(bi.bi_attn_workspace_bytes(cfg, 150, bt.max_seq_len) // 4 + 64, device="cuda")
    bi.bi_attn_decode(cfg, d.q, d.k_cache, d.v_cache, d.page_table, sl, bt.max_seq_len, out, ws)
    assert torch.isnan(out[bad]).all()
    good = [r for r in range(150) if r not in bad]
    assert_bitwise(out[good], clean[good], "valid rows next to invalid ones")
    rows = [(r, h) for r in good[::7] for h in (0, 13, 31)]
    ref = oracle_rows(bt, rows)
    got = np.stack([clean[r, h].cpu().numpy() for r, h in rows])
    assert_parity(got, ref, "decode 150 sequences, sampled rows")


@pytest.mark.parametrize("hq", [64, 32])
def test_prefill_many_sequences_with_invalid_lengths(hq):
    """90 sequences of mixed prefix and chunk lengths (some chunks empty): the longest-first
    order of the query tiles walks several chunks of 64 sequences and many equal costs. Every
    token of a valid sequence gets a finite row within parity; making some lengths invalid
    turns exactly their tokens NaN and leaves every other row's bits as they were."""
    shape = AttnShape(hq, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    rng = np.random.default_rng(51)
    seqs = [SeqSpec(i, int(rng.integers(0, 600)), int(rng.integers(0, 40))) for i in range(90)]
    bt = build_batch(shape, seqs, seed=52, page_seed=53, extra_pages=8)
    d = to_device(bt, cfg)
    _print_case("prefill 90 sequences", hq)
    clean = run_prefill(cfg, d)
    assert torch.isfinite(clean).all(), "a query tile was skipped"
    qs = bt.q_starts
    bad = [b for b in (2, 33, 64, 65, 89) if qs[b + 1] > qs[b]]
    sl = d.seq_lens.clone()
    for i, b in enumerate(bad):
        sl[b] = (qs[b + 1] - qs[b]) - 1 if i % 2 == 0 else bt.max_seq_len + 5
    out = torch.full_like(clean, float("nan"))
    bi.bi_attn_prefill(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.q_starts, sl,
                       d.max_q_len, d.max_seq_len, out)
    bad_rows = np.concatenate([np.arange(qs[b], qs[b + 1]) for b in bad])
    good_rows = np.setdiff1d(np.arange(bt.total_tokens), bad_rows)
    assert torch.isnan(out[torch.from_numpy(bad_rows)]).all()
    assert_bitwise(out[torch.from_numpy(good_rows)], clean[torch.from_numpy(good_rows)],
                   "valid rows next to invalid sequences")
    rows = [(int(r), h) for r in good_rows[::11] for h in (0, hq // 2 + 1, hq - 1)]
    ref = oracle_rows(bt, rows)
    got = np.stack([clean[r, h].cpu().numpy() for r, h in rows])
    assert_parity(got, ref, "prefill 90 sequences, sampled rows")


def test_prefill_invalid_chunks_give_nan_rows_only():
    """A sequence with more new tokens than max_q_len, or whose q_starts entry runs past
    total_tokens, is invalid: its rows that lie in q come out NaN (none is left unwritten), and
    every other sequence's rows keep the bits of a clean run."""
    shape = AttnShape(64, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    seqs = [SeqSpec(0, 300, 40), SeqSpec(1, 100, 200), SeqSpec(2, 50, 30), SeqSpec(3, 700, 60)]
    bt = build_batch(shape, seqs, seed=71, page_seed=72, extra_pages=4)
    d = to_device(bt, cfg)
    clean = run_prefill(cfg, d)
    assert torch.isfinite(clean).all()
    T, qs = bt.total_tokens, bt.q_starts
    _print_case("prefill n_new > max_q_len")
    # sequence 1 has 200 new tokens; max_q_len 60 makes it invalid (its 200 rows need
    # several strides of its capped tiles)
    out = torch.zeros_like(clean)
    bi.bi_attn_prefill(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.q_starts, d.seq_lens, 60,
                       d.max_seq_len, out)
    r0, r1 = int(qs[1]), int(qs[2])
    assert torch.isnan(out[r0:r1]).all()
    keep = torch.cat([torch.arange(0, r0), torch.arange(r1, T)]).cuda()
    assert_bitwise(out[keep], clean[keep], "rows of valid sequences next to n_new > max_q_len")
    _print_case("prefill q_starts past total_tokens")
    # the last entry of q_starts 25 past the rows of q: the last sequence is invalid, its rows
    # inside q are NaN, nothing is read or written past q and out
    qs2 = d.q_starts.clone()
    qs2[-1] = T + 25
    out = torch.zeros_like(clean)
    bi.bi_attn_prefill(cfg, d.q, d.k_cache, d.v_cache, d.page_table, qs2, d.seq_lens, d.max_q_len,
                       d.max_seq_len, out)
    r3 = int(qs[3])
    assert torch.isnan(out[r3:]).all()
    assert_bitwise(out[:r3], clean[:r3], "rows of valid sequences next to a q_starts overrun")
