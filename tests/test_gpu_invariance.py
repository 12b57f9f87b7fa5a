"""Bitwise batch invariance of the HIP path (GPU).

Zero differing bits for a token's fp32 output across batch size, position in the batch,
physical page placement, chunk size and route (prefill or decode). A failure reports the
number of differing words, the XOR popcount and the first differing (token, head, dim).
The split-count-by-batch variant is the negative control: it must change bits.
"""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
from synth import CONFIG_SHAPES, AttnShape, SeqSpec, build_batch
from gpu_harness import (assert_bitwise, assert_parity, bits, cfg_for, decode_workspace,
                         oracle_out, oracle_rows, page_update, run_decode, run_prefill,
                         to_device)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _print_case(*a):
    print("CASE", *a, flush=True)


def _decode_sub(cfg, d, idx, max_seq_len, ws=None):
    """Decode over the batch rows ``idx`` (device gathers of table, lengths and q)."""
    it = torch.tensor(idx, dtype=torch.long, device="cuda")
    pt, sl, q = d.page_table[it].contiguous(), d.seq_lens[it].contiguous(), d.q[it].contiguous()
    out = torch.full((len(idx), cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda")
    ws = decode_workspace(cfg, len(idx), max_seq_len) if ws is None else ws
    bi.bi_attn_decode(cfg, q, d.k_cache, d.v_cache, pt, sl, max_seq_len, out, ws)
    return out


# ----------------------------------------------------------------------------- tiny fp32
def test_tiny_f32_batch_and_route_invariance():
    """Probe = 128 cached + 16 new tokens; batch sizes 1-4 at every position; 16 decodes."""
    shape = CONFIG_SHAPES["tiny_f32"]
    cfg = cfg_for(shape)
    rng = np.random.default_rng(2025)
    others = []
    for r in range(1, 4):
        L = int(rng.integers(16, 257))
        n = int(rng.integers(1, 17))
        others.append(SeqSpec(r, L - n, n))
    probe = SeqSpec(0, 128, 16)
    ref = None
    for B in range(1, 5):
        for p in range(B):
            seqs = others[: B - 1]
            seqs = seqs[:p] + [probe] + seqs[p:]
            bt = build_batch(shape, seqs, seed=2025, page_seed=100 * B + p, extra_pages=2)
            _print_case("tiny batch", B, p)
            out = run_prefill(cfg, to_device(bt, cfg))
            r0, r1 = bt.token_rows(p)
            got = out[r0:r1]
            if ref is None:
                ref = got.clone()
                assert_parity(out.cpu().numpy(), oracle_out(bt), "tiny prefill")
            else:
                assert_bitwise(got, ref, f"tiny prefill B={B} pos={p}")
    # one token at a time through decode, with the other rows decoding alongside
    for i in range(16):
        seqs = [SeqSpec(0, 128 + i, 1)] + [SeqSpec(s.req, s.seq_len - 1, 1) for s in others]
        bt = build_batch(shape, seqs, seed=2025, page_seed=7 + i)
        out = run_decode(cfg, to_device(bt, cfg))
        assert_bitwise(out[0], ref[i], f"tiny decode token {i}")
        # and through prefill with 1-token chunks
        outp = run_prefill(cfg, to_device(bt, cfg))
        assert_bitwise(outp[0], ref[i], f"tiny 1-token prefill token {i}")


# ----------------------------------------------------------------------------- decode sweep
def test_decode_batch_and_position_invariance():
    """Probes at lengths {128, 255, 256, 257, 4096, 8191, 8192} across B in {1..64}."""
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg = cfg_for(shape)
    probe_lens = [128, 255, 256, 257, 4096, 8191, 8192]
    rng = np.random.default_rng(2026)
    other_lens = [int(x) for x in rng.integers(128, 8193, 63)]
    seqs = [SeqSpec(1000 + i, L - 1, 1) for i, L in enumerate(probe_lens)]
    seqs += [SeqSpec(i, L - 1, 1) for i, L in enumerate(other_lens)]
    _print_case("decode sweep build")
    bt = build_batch(shape, seqs, seed=2026, page_seed=5)
    d = to_device(bt, cfg)
    page_update(cfg, d)
    mx = 8192
    ws = decode_workspace(cfg, 64, mx)
    nP = len(probe_lens)
    others = list(range(nP, nP + 63))
    for k, L in enumerate(probe_lens):
        ref = _decode_sub(cfg, d, [k], mx, ws)[0].clone()
        if k == 0:
            full = _decode_sub(cfg, d, list(range(len(seqs))), mx)
            assert_parity(full.cpu().numpy(), oracle_out(bt), "decode sweep parity")
        for B in (1, 2, 4, 8, 16, 32, 64):
            positions = range(B) if B <= 8 else (0, B // 2, B - 1)
            for p in positions:
                idx = others[: B - 1]
                idx = idx[:p] + [k] + idx[p:]
                out = _decode_sub(cfg, d, idx, mx, ws)
                assert_bitwise(out[p], ref, f"probe L={L} B={B} pos={p}")
        _print_case("probe done", L)


def test_decode_page_placement_invariance():
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg = cfg_for(shape)
    ref = None
    for ps in range(4):
        bt = build_batch(shape, [SeqSpec(77, 3000, 1)], seed=2026, page_seed=ps, extra_pages=50 * ps)
        out = run_decode(cfg, to_device(bt, cfg))
        if ref is None:
            ref = out
        else:
            assert_bitwise(out, ref, f"page seed {ps}")


def test_run_to_run_determinism():
    shape = CONFIG_SHAPES["prefill_bf16"]
    cfg = cfg_for(shape)
    bt = build_batch(shape, [SeqSpec(0, 900, 300), SeqSpec(1, 10, 77)], seed=5)
    d = to_device(bt, cfg)
    a = run_prefill(cfg, d)
    for _ in range(3):
        assert_bitwise(run_prefill(cfg, d, update=False), a, "prefill rerun")


# ----------------------------------------------------------------------------- routes
def _chunked_route(shape, cfg, specs, chunk, seed, q_scale=1.0):
    """Process every sequence's new tokens in chunks of ``chunk`` (1 => decode calls)."""
    full = build_batch(shape, specs, seed=seed, page_seed=11, q_scale=q_scale)
    d = to_device(full, cfg)
    # fresh NaN pool holding only the prefixes; tokens arrive chunk by chunk
    outs = torch.full((full.total_tokens, cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda")
    done = [0] * len(specs)
    while True:
        rows, ks, sl, qs, tbl_rows, tok_idx = [], [], [], [0], [], []
        for b, s in enumerate(specs):
            if done[b] >= s.n_new:
                continue
            n = min(chunk, s.n_new - done[b])
            r0 = int(full.q_starts[b]) + done[b]
            tok_idx.extend(range(r0, r0 + n))
            sl.append(s.cached + done[b] + n)
            qs.append(qs[-1] + n)
            tbl_rows.append(b)
            done[b] += n
        if not tbl_rows:
            break
        ti = torch.tensor(tok_idx, dtype=torch.long, device="cuda")
        bi_rows = torch.tensor(tbl_rows, dtype=torch.long, device="cuda")
        q = d.q[ti].contiguous()
        kn, vn = d.k_new[ti].contiguous(), d.v_new[ti].contiguous()
        pt = d.page_table[bi_rows].contiguous()
        slt = torch.tensor(sl, dtype=torch.int32, device="cuda")
        qst = torch.tensor(qs, dtype=torch.int32, device="cuda")
        bi.bi_kv_page_update(cfg, kn, vn, qst, slt, pt, d.k_cache, d.v_cache)
        mx = max(sl)
        out = torch.full((len(tok_idx), cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda")
        if chunk == 1:
            ws = decode_workspace(cfg, len(tbl_rows), mx)
            bi.bi_attn_decode(cfg, q, d.k_cache, d.v_cache, pt, slt, mx, out, ws)
        else:
            bi.bi_attn_prefill(cfg, q, d.k_cache, d.v_cache, pt, qst, slt, max(np.diff(qs)), mx, out)
        outs[ti] = out
    return outs, full


@pytest.mark.parametrize("scale", ["small", "full"])
def test_prefill_route_invariance(scale):
    """Each token identical in one prefill, chunks of 512 and 128, and token-by-token decode."""
    shape = CONFIG_SHAPES["prefill_bf16"]
    cfg = cfg_for(shape)
    rng = np.random.default_rng(2027)
    if scale == "small":
        B, pre_hi, chunk_hi, chunks = 6, 1200, 300, (64, 16, 1)
    else:
        B, pre_hi, chunk_hi, chunks = 16, 16384, 2048, (512, 128, 1)
    specs = [SeqSpec(i, int(rng.integers(0, pre_hi + 1)), int(rng.integers(1, chunk_hi + 1)))
             for i in range(B)]
    _print_case("route", scale, [(s.cached, s.n_new) for s in specs])
    ref, full = _chunked_route(shape, cfg, specs, 1 << 30, seed=2027)
    if scale == "small":
        assert_parity(ref.cpu().numpy(), oracle_out(full), "route prefill parity")
    for ch in chunks:
        got, _ = _chunked_route(shape, cfg, specs, ch, seed=2027)
        assert_bitwise(got, ref, f"chunk {ch} vs one prefill")
        _print_case("route chunk ok", ch)


def test_long_decode_batch_invariance():
    """131072-token sequences at B in {1, 2, 4, 8}: every sequence's bits unchanged."""
    shape = CONFIG_SHAPES["long_decode_bf16"]
    cfg = cfg_for(shape)
    L = 131072
    seqs = [SeqSpec(i, L - 1, 1) for i in range(8)]
    _print_case("long build")
    bt = build_batch(shape, seqs, seed=2028, page_seed=13, q_scale=4.0)
    d = to_device(bt, cfg)
    page_update(cfg, d)
    ws = decode_workspace(cfg, 8, L)
    ref = _decode_sub(cfg, d, list(range(8)), L, ws)
    for B in (1, 2, 4):
        for start in range(0, 8, B):
            idx = list(range(start, start + B))
            out = _decode_sub(cfg, d, idx, L, ws)
            assert_bitwise(out, ref[start:start + B], f"long B={B} start={start}")


def test_peaked_route_invariance():
    """q x 4 rows at positions 1024 .. 4095, where the second bf16 term of P follows the scores
    (peaked splits, outliers above the lazy reference) rather than the position alone: one
    prefill, chunks of 512 and 128, and token-by-token decode give identical bits."""
    shape = AttnShape(64, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    specs = [SeqSpec(0, 1024, 3072), SeqSpec(1, 2000, 300), SeqSpec(2, 0, 700)]
    _print_case("peaked routes")
    ref, full = _chunked_route(shape, cfg, specs, 1 << 30, seed=63, q_scale=4.0)
    for ch in (512, 128, 1):
        got, _ = _chunked_route(shape, cfg, specs, ch, seed=63, q_scale=4.0)
        assert_bitwise(got, ref, f"peaked: chunk {ch} vs one prefill")
        _print_case("peaked route ok", ch)


def test_decode_two_phases_equal_one_call():
    """bi_attn_decode_partials then bi_attn_decode_combine on the same workspace give the bits
    of bi_attn_decode (the route the benchmark times), also from a NaN-poisoned workspace and
    for sequences of 1 to 64 splits."""
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg = cfg_for(shape)
    rng = np.random.default_rng(81)
    lens = [1, 255, 256, 257, 16384, 16385] + [int(x) for x in rng.integers(128, 8193, 26)]
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)], seed=82, page_seed=83)
    d = to_device(bt, cfg)
    page_update(cfg, d)
    B, mx = len(lens), bt.max_seq_len
    ref = _decode_sub(cfg, d, list(range(B)), mx)
    ws = decode_workspace(cfg, B, mx)                   # NaN-filled
    out = torch.full_like(ref, float("nan"))
    bi.bi_attn_decode_partials(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens, mx, ws)
    bi.bi_attn_decode_combine(cfg, d.seq_lens, mx, out, ws)
    assert_bitwise(out, ref, "partials + combine vs one decode call")


def test_probe_unique_bit_patterns_over_1000_compositions():
    """The kernel-level analogue of the pages' experiment (one prompt, 1000 runs, count the
    distinct completions): a decode probe in 1000 random batch compositions (batch size 1..64,
    random position, random neighbours from 200 sequences of the decode workload's lengths)
    gives exactly one bit pattern; the split-by-batch variant gives more than one."""
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg = cfg_for(shape)
    cfg_v = cfg_for(shape, policy=bi.BI_SPLIT_BY_BATCH)
    rng = np.random.default_rng(2026)
    lens = [4097] + [int(x) for x in rng.integers(128, 8193, 200)]
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)], seed=2026, page_seed=84)
    d = to_device(bt, cfg)
    page_update(cfg, d)
    mx = 8192
    ws = torch.empty(bi.bi_attn_workspace_bytes(cfg_v, 64, mx) // 4 + 64, device="cuda")
    patterns, patterns_v = set(), set()
    for trial in range(1000):
        B = int(rng.integers(1, 65))
        p = int(rng.integers(0, B))
        nb = [int(x) + 1 for x in rng.choice(200, B - 1, replace=False)]
        idx = nb[:p] + [0] + nb[p:]
        patterns.add(bits(_decode_sub(cfg, d, idx, mx, ws)[p]).tobytes())
        patterns_v.add(bits(_decode_sub(cfg_v, d, idx, mx, ws)[p]).tobytes())
        if trial % 250 == 0:
            _print_case("composition", trial, len(patterns), len(patterns_v))
    print(f"1000 compositions: {len(patterns)} bit pattern(s) with the fixed split size, "
          f"{len(patterns_v)} with the split count chosen by batch")
    assert len(patterns) == 1
    assert len(patterns_v) > 1


# ----------------------------------------------------------------------------- negative control
def test_split_by_batch_variant_changes_bits():
    """The batch-dependent split policy must show more than one bit pattern for a probe."""
    shape = CONFIG_SHAPES["decode_bf16"]
    cfg_v = cfg_for(shape, policy=bi.BI_SPLIT_BY_BATCH)
    rng = np.random.default_rng(3)
    other_lens = [int(x) for x in rng.integers(128, 8193, 63)]
    seqs = [SeqSpec(999, 4095, 1)] + [SeqSpec(i, L - 1, 1) for i, L in enumerate(other_lens)]
    bt = build_batch(shape, seqs, seed=2026, page_seed=21)
    d = to_device(bt, cfg_v)
    page_update(cfg_v, d)
    patterns = set()
    for B in (1, 2, 4, 8, 16, 32, 64):
        out = _decode_sub(cfg_v, d, list(range(B)), 8192)
        patterns.add(bits(out[0]).tobytes())
        if B == 64:
            assert_parity(out.cpu().numpy(), oracle_out(bt), "variant parity")
    assert len(patterns) > 1


@pytest.mark.parametrize("hq", [64, 32])
def test_p_precision_boundary_route_invariance(hq):
    """Rows on both sides of the position where P drops its second bf16 term (1024), also
    inside one MFMA block (G = 8: two tokens per block): one prefill, chunks of 7 and decode
    give identical bits, and the outputs are within the parity bar."""
    shape = AttnShape(hq, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    specs = [SeqSpec(0, 1000, 60), SeqSpec(1, 1020, 9), SeqSpec(2, 1023, 2), SeqSpec(3, 10, 20),
             SeqSpec(4, 1024, 3)]
    _print_case("p precision boundary", hq)
    ref, full = _chunked_route(shape, cfg, specs, 1 << 30, seed=77)
    got, want = ref.cpu().numpy(), oracle_out(full)
    assert_parity(got, want, "prefill across the P precision boundary")
    # rows below position 1024 carry the second bf16 term of P: errors near 1e-6, far inside
    # the bar that the single-term rows meet
    pos = np.concatenate([np.arange(s.cached, s.cached + s.n_new) for s in specs])
    short = pos < 1024
    assert short.any() and (~short).any()
    err_short = float(np.abs(got[short] - want[short]).max())
    assert err_short <= 2e-5, f"rows below 1024: max-abs {err_short:.2e}"
    for ch in (7, 1):
        got, _ = _chunked_route(shape, cfg, specs, ch, seed=77)
        assert_bitwise(got, ref, f"chunk {ch} vs one prefill across the P precision boundary")


@pytest.mark.parametrize("hq,dtype,d", [(64, "bf16", 128), (32, "bf16", 128), (32, "f32", 128),
                                        (16, "bf16", 64), (8, "f32", 64)])
def test_prefill_past_page_id_ring(hq, dtype, d):
    """Sequences past 32768 tokens: a 40000-token prefix with a 70-token chunk and a shorter
    neighbour. bf16 with D = 128 streams K/V straight into LDS with page ids in registers; fp32,
    and bf16 with D = 64, stage K/V through registers and read page ids from an LDS ring of 2048
    entries, which is refilled while the tile runs past 32768 tokens. One prefill, chunks of 16
    and decode give identical bits; sampled rows match the oracle."""
    shape = AttnShape(hq, 4, d, 16, 256, dtype)
    cfg = cfg_for(shape)
    specs = [SeqSpec(0, 40000, 70), SeqSpec(1, 33000, 5)]
    _print_case("ring", hq, dtype, d)
    ref, full = _chunked_route(shape, cfg, specs, 1 << 30, seed=91)
    for ch in (16, 1):
        got, _ = _chunked_route(shape, cfg, specs, ch, seed=91)
        assert_bitwise(got, ref, f"chunk {ch} vs one prefill past the page-id ring")
    rows = [(t, h) for t in (0, 37, 69, 70, 74) for h in (0, hq // 2 + 3, hq - 1)]
    want = oracle_rows(full, rows)
    got = np.stack([ref[t, h].cpu().numpy() for t, h in rows])
    assert_parity(got, want, "prefill rows past the page-id ring")
