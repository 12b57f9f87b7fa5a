"""Host-side checks of the seeded input generators (CPU only)."""

import numpy as np
import torch

from synth import (AttnShape, SeqSpec, bf16_bits, bf16_round, build_batch, from_bf16_bits,
                   mixed_trace, token_values)
from synth.workloads import PageAllocator


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38, -3.4e38, np.inf, -np.inf],
                                 np.float32)])
    # exact ties: low 16 bits == 0x8000 (round to even both ways)
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), ref)
    assert np.array_equal(bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    nan = bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(from_bf16_bits(nan))[0]


def test_token_values_regenerate_any_range():
    full = token_values(3, 17, "k", 0, 1000, 4, 16, "bf16")
    part = token_values(3, 17, "k", 250, 777, 4, 16, "bf16")
    assert np.array_equal(full[250:777], part)
    assert np.array_equal(bf16_round(full), full)
    other = token_values(3, 18, "k", 0, 1000, 4, 16, "bf16")
    assert not np.array_equal(full, other)
    q4 = token_values(3, 17, "q", 0, 10, 4, 16, "bf16", scale=4.0)
    q1 = token_values(3, 17, "q", 0, 10, 4, 16, "bf16")
    assert np.array_equal(q4, q1 * 4)          # a power-of-two scale commutes with rounding


def test_build_batch_layout():
    shape = AttnShape(8, 2, 16, page_size=16, split_size=32, dtype="bf16")
    seqs = [SeqSpec(5, 40, 3), SeqSpec(9, 0, 20), SeqSpec(2, 16, 1)]
    bt = build_batch(shape, seqs, seed=1, page_seed=4, extra_pages=5)
    assert bt.total_tokens == 24 and list(bt.q_starts) == [0, 3, 23, 24]
    assert list(bt.seq_lens) == [43, 20, 17]
    used = bt.page_table[bt.page_table >= 0]
    assert len(set(used.tolist())) == len(used) == 3 + 2 + 2
    # prefix placed, new-token slots still poisoned
    P = 16
    for b, s in enumerate(seqs):
        ref = token_values(1, s.req, "v", 0, s.cached, 2, 16, "bf16")
        for pos in range(s.seq_len):
            slot = bt.v_pool[bt.page_table[b][pos // P], :, pos % P]
            if pos < s.cached:
                assert np.array_equal(slot, ref[pos])
            else:
                assert np.isnan(slot).all()
    assert np.array_equal(bt.q[3:23], token_values(1, 9, "q", 0, 20, 8, 16, "bf16"))
    assert list(bt.positions()) == [40, 41, 42] + list(range(20)) + [16]


def test_mixed_trace_schedule():
    tr = mixed_trace(2025 + 4)
    prompts, outputs = tr.prompts, tr.outputs
    assert prompts.min() >= 64 and prompts.max() <= 32768
    assert outputs.min() >= 16 and outputs.max() <= 1024
    done = np.zeros(len(prompts), np.int64)
    dec = np.zeros(len(prompts), np.int64)
    for st in tr.steps:
        assert st.tokens <= 8192
        ids = [r for r, _ in st.decode]
        assert ids == sorted(ids)
        for r, pos in st.decode:
            assert done[r] == prompts[r] and pos == prompts[r] + dec[r]
        for r, start, n in st.prefill:
            assert start == done[r] and n >= 1 and start + n <= prompts[r]
        # FCFS: at most the last prefill chunk is cut short by the budget
        for r, start, n in st.prefill[:-1]:
            assert start + n == prompts[r]
        if st.prefill and st.tokens < 8192:
            r, start, n = st.prefill[-1]
            assert start + n == prompts[r]
        for r, _ in st.decode:
            dec[r] += 1
        for r, start, n in st.prefill:
            done[r] += n
    assert sum(len(s.decode) for s in tr.steps) > 0


def test_page_allocator_reuses_freed_pages():
    al = PageAllocator(10, seed=1)
    a = al.ensure(0, 33, 16)
    assert len(a) == 3
    b = al.ensure(1, 80, 16)
    assert len(b) == 5 and not set(a) & set(b)
    al.release(0)
    c = al.ensure(2, 40, 16)
    assert set(c) <= set(a) | set(range(10)) and not set(c) & set(b)


def test_device_generator_definition_and_moments():
    """splitmix64 against its published definition in Python integers; N(0, 1) moments."""
    from synth.device import normal_tokens, splitmix64

    def ref(x):
        m = (1 << 64) - 1
        z = (x + 0x9E3779B97F4A7C15) & m
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
        return z ^ (z >> 31)

    xs = [0, 1, 2, 12345, (1 << 63) - 1, 1 << 62, 0x0123456789ABCDEF]
    got = splitmix64(torch.tensor([x - (1 << 64) if x >= 1 << 63 else x for x in xs], dtype=torch.int64))
    assert [int(v) & ((1 << 64) - 1) for v in got] == [ref(x) for x in xs]
    req = torch.arange(64).repeat_interleave(16)
    pos = torch.arange(16).repeat(64)
    z = normal_tokens(7, req, "k", pos, 4, 128, dtype=torch.float32)
    assert abs(float(z.mean())) < 0.01 and abs(float(z.std()) - 1.0) < 0.01
    # stateless: any subset of tokens regenerates the same values
    z2 = normal_tokens(7, req[100:300], "k", pos[100:300], 4, 128, dtype=torch.float32)
    assert torch.equal(z[100:300], z2)
    assert not torch.equal(normal_tokens(7, req, "v", pos, 4, 128, dtype=torch.float32), z)
