"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped scale, a wrong GQA
index, an off-by-one causal mask, a transposed operand, a wrong page lookup, a wrong fold
coefficient) fails at least one of them; ``test_pins_catch_planted_mistakes`` plants such
slips in copies of the computation, on the CPU, and checks they are caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import AttnShape, SeqSpec, build_batch

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------- helpers
def paged_from_dense(seqs_k, seqs_v, page_size, seed, extra_pages=3):
    """Place dense per-sequence K/V ``[L][Hkv][D]`` in a shuffled NaN pool; returns pool, table."""
    rng = np.random.default_rng(seed)
    Hkv, D = seqs_k[0].shape[1], seqs_k[0].shape[2]
    npages = [(k.shape[0] + page_size - 1) // page_size for k in seqs_k]
    total = sum(npages) + extra_pages
    perm = rng.permutation(total)
    kp = np.full((total, Hkv, page_size, D), np.nan)
    vp = np.full((total, Hkv, page_size, D), np.nan)
    table = np.full((len(seqs_k), max(npages)), -1, np.int32)
    off = 0
    for b, (k, v) in enumerate(zip(seqs_k, seqs_v)):
        for pos in range(k.shape[0]):
            page = perm[off + pos // page_size]
            kp[page, :, pos % page_size] = k[pos]
            vp[page, :, pos % page_size] = v[pos]
        table[b, : npages[b]] = perm[off: off + npages[b]]
        off += npages[b]
    return kp, vp, table


def brute_force(q, seqs_k, seqs_v, n_new, scale=None, gqa=lambda h, G, Hkv: h // G):
    """Pure-Python loops with math.exp: out[t][h][d] straight from the definition."""
    T, Hq, D = q.shape
    Hkv = seqs_k[0].shape[1]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.zeros((T, Hq, D))
    t = 0
    for b, k in enumerate(seqs_k):
        L = k.shape[0]
        for i in range(n_new[b]):
            pos = L - n_new[b] + i
            for h in range(Hq):
                g = gqa(h, G, Hkv)
                s = [sum(float(q[t, h, d]) * float(k[j, g, d]) for d in range(D)) * sc
                     for j in range(pos + 1)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                for d in range(D):
                    out[t, h, d] = sum(w[j] * float(seqs_v[b][j, g, d]) for j in range(pos + 1)) / tot
            t += 1
    return out


def random_case(seed, Hq=4, Hkv=2, D=8, lens=(5, 17, 33), n_new=(5, 3, 8), page_size=4):
    rng = np.random.default_rng(seed)
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    q = rng.standard_normal((sum(n_new), Hq, D))
    kp, vp, table = paged_from_dense(ks, vs, page_size, seed + 1)
    q_starts = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    seq_lens = np.array(lens, np.int32)
    return dict(q=q, ks=ks, vs=vs, kp=kp, vp=vp, table=table, q_starts=q_starts,
                seq_lens=seq_lens, n_new=list(n_new), Hkv=Hkv)


def run_oracle(c, **kw):
    return oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["q_starts"],
                                  c["seq_lens"], c["Hkv"], **kw)


# ----------------------------------------------------------------------------- definition pins
def test_closed_forms_golden():
    spec = json.load(open(os.path.join(HERE, "golden", "closed_forms.json")))
    for case in spec["cases"]:
        D = case["head_dim"]
        K = np.array(case["keys"], np.float64)[:, None, :]
        V = np.array(case["values"], np.float64)[:, None, :]
        L = K.shape[0]
        kp, vp, table = paged_from_dense([K], [V], 2, seed=7)
        q = np.tile(np.array(case["q"], np.float64), (L, 1))[:, None, :]
        out = oracle.paged_attention(q, kp, vp, table, np.array([0, L], np.int32),
                                     np.array([L], np.int32), 1)
        for pos, exp in case["expected"].items():
            np.testing.assert_allclose(out[int(pos), 0], exp, atol=1e-12, rtol=0,
                                       err_msg=case["name"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    c = random_case(seed)
    got = run_oracle(c)
    ref = brute_force(c["q"], c["ks"], c["vs"], c["n_new"])
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


def test_torch_sdpa_float64():
    c = random_case(11, Hq=6, Hkv=3, D=16, lens=(40, 9, 64), n_new=(40, 2, 7), page_size=16)
    got = run_oracle(c)
    G = 2
    t = 0
    for b, k in enumerate(c["ks"]):
        L, n = k.shape[0], c["n_new"][b]
        pos = torch.arange(L - n, L)
        mask = torch.arange(L)[None, :] <= pos[:, None]                 # True = attend
        qb = torch.from_numpy(c["q"][t:t + n]).permute(1, 0, 2)         # [Hq][n][D]
        kb = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)
        vb = torch.from_numpy(np.repeat(c["vs"][b], G, axis=1)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask)
        np.testing.assert_allclose(got[t:t + n], ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
        t += n


@pytest.mark.parametrize("seed", [0, 3])
def test_varlen_brute_force_tiny(seed):
    """The dense (varlen) form against the pure-Python definition, sequences laid end to end."""
    c = random_case(seed, lens=(7, 20, 1, 33), n_new=(7, 4, 1, 9))
    k = np.concatenate(c["ks"]); v = np.concatenate(c["vs"])
    k_starts = np.concatenate([[0], np.cumsum([x.shape[0] for x in c["ks"]])]).astype(np.int32)
    got = oracle.varlen_attention(c["q"], k, v, c["q_starts"], k_starts, c["Hkv"])
    ref = brute_force(c["q"], c["ks"], c["vs"], c["n_new"])
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


def test_varlen_torch_sdpa_float64():
    c = random_case(12, Hq=8, Hkv=2, D=16, lens=(50, 16, 3), n_new=(50, 5, 1), page_size=16)
    k = np.concatenate(c["ks"]); v = np.concatenate(c["vs"])
    k_starts = np.array([0, 50, 66, 69], np.int32)
    got = oracle.varlen_attention(c["q"], k, v, c["q_starts"], k_starts, 2)
    G, t = 4, 0
    for b, kb_np in enumerate(c["ks"]):
        L, n = kb_np.shape[0], c["n_new"][b]
        pos = torch.arange(L - n, L)
        mask = torch.arange(L)[None, :] <= pos[:, None]
        qb = torch.from_numpy(c["q"][t:t + n]).permute(1, 0, 2)
        kb = torch.from_numpy(np.repeat(kb_np, G, axis=1)).permute(1, 0, 2)
        vb = torch.from_numpy(np.repeat(c["vs"][b], G, axis=1)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask)
        np.testing.assert_allclose(got[t:t + n], ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
        t += n


# ----------------------------------------------------------------------------- invariants
def test_weights_sum_to_one():
    c = random_case(3)
    for vp in (c["vp"],):
        ones = np.where(np.isnan(vp), np.nan, 1.0)
        out = oracle.paged_attention(c["q"], c["kp"], ones, c["table"], c["q_starts"],
                                     c["seq_lens"], c["Hkv"])
        np.testing.assert_allclose(out, 1.0, atol=1e-12, rtol=0)


def test_constant_v_returns_v():
    c = random_case(4)
    const = np.arange(c["vp"].shape[-1], dtype=np.float64) - 2.5
    vp = np.where(np.isnan(c["vp"]), np.nan, const)
    out = oracle.paged_attention(c["q"], c["kp"], vp, c["table"], c["q_starts"],
                                 c["seq_lens"], c["Hkv"])
    np.testing.assert_allclose(out, np.broadcast_to(const, out.shape), atol=1e-12, rtol=0)


def test_dominant_key_returns_its_value():
    c = random_case(5, Hq=2, Hkv=1, D=8, lens=(20,), n_new=(1,))
    k = c["ks"][0]
    j = 13
    q = np.array(k[j, 0] * 200.0)[None, None, :].repeat(2, axis=1)
    # make key j the clear winner: unit-norm keys except j scaled up
    ks = [k / np.linalg.norm(k, axis=-1, keepdims=True)]
    ks[0][j] = ks[0][j] * 3.0
    kp, vp, table = paged_from_dense(ks, c["vs"], 4, seed=9)
    out = oracle.paged_attention(q, kp, vp, table, np.array([0, 1], np.int32),
                                 np.array([20], np.int32), 1)
    np.testing.assert_allclose(out[0, 0], c["vs"][0][j, 0], atol=1e-6, rtol=0)


def test_page_permutation_is_bitwise_neutral():
    c = random_case(6)
    base = run_oracle(c)
    rng = np.random.default_rng(99)
    perm = rng.permutation(c["kp"].shape[0])          # new physical slot of every page
    kp2 = np.empty_like(c["kp"])
    vp2 = np.empty_like(c["vp"])
    kp2[perm] = c["kp"]
    vp2[perm] = c["vp"]
    table2 = np.where(c["table"] >= 0, perm[np.maximum(c["table"], 0)], -1).astype(np.int32)
    out = oracle.paged_attention(c["q"], kp2, vp2, table2, c["q_starts"], c["seq_lens"], c["Hkv"])
    assert np.array_equal(out.view(np.int64), base.view(np.int64))


def test_causality_is_bitwise():
    c = random_case(7, lens=(30,), n_new=(30,))
    base = run_oracle(c)
    # perturb every key and value after position 12; rows 0..12 must not move a bit
    ks = [c["ks"][0].copy()]
    vs = [c["vs"][0].copy()]
    ks[0][13:] += 5.0
    vs[0][13:] -= 3.0
    kp, vp, table = paged_from_dense(ks, vs, 4, seed=8)
    out = oracle.paged_attention(c["q"], kp, vp, table, c["q_starts"], c["seq_lens"], c["Hkv"])
    assert np.array_equal(out[:13].view(np.int64), base[:13].view(np.int64))
    assert not np.allclose(out[13:], base[13:])


def test_gqa_equals_mha_with_repeated_heads():
    c = random_case(8, Hq=8, Hkv=2)
    gqa = run_oracle(c)
    G = 4
    ks = [np.repeat(k, G, axis=1) for k in c["ks"]]
    vs = [np.repeat(v, G, axis=1) for v in c["vs"]]
    kp, vp, table = paged_from_dense(ks, vs, 4, seed=10)
    mha = oracle.paged_attention(c["q"], kp, vp, table, c["q_starts"], c["seq_lens"], 8)
    np.testing.assert_allclose(gqa, mha, atol=1e-13, rtol=0)


def test_q_zero_gives_prefix_mean():
    c = random_case(9)
    q0 = np.zeros_like(c["q"])
    out = oracle.paged_attention(q0, c["kp"], c["vp"], c["table"], c["q_starts"],
                                 c["seq_lens"], c["Hkv"])
    G = c["q"].shape[1] // c["Hkv"]
    t = 0
    for b, v in enumerate(c["vs"]):
        L, n = v.shape[0], c["n_new"][b]
        for i in range(n):
            pos = L - n + i
            mean = v[: pos + 1].mean(axis=0)                   # [Hkv][D]
            np.testing.assert_allclose(out[t], np.repeat(mean, G, axis=0), atol=1e-12, rtol=0)
            t += 1


def test_rows_match_full():
    c = random_case(10)
    full = run_oracle(c)
    rows = [(0, 0), (4, 3), (5, 1), (8, 2), (15, 0), (12, 3)]
    got = oracle.paged_attention_rows(c["q"], c["kp"], c["vp"], c["table"], c["q_starts"],
                                      c["seq_lens"], c["Hkv"], rows)
    for n, (t, h) in enumerate(rows):
        np.testing.assert_allclose(got[n], full[t, h], atol=1e-13, rtol=0)


# ----------------------------------------------------------------------------- split and fold
@pytest.mark.parametrize("S", [16, 32, 256])
def test_split_fold_equals_plain(S):
    rng = np.random.default_rng(S)
    D, L = 32, 700
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    for pos in (0, 1, S - 1, S, S + 1, 3 * S + 5, L - 1):
        if pos >= L:
            continue
        q = rng.standard_normal(D) * 3.0
        got = oracle.split_fold_attention(q, K, V, pos, S)
        s = K[: pos + 1] @ q / math.sqrt(D)
        w = np.exp(s - s.max())
        np.testing.assert_allclose(got, (w / w.sum()) @ V[: pos + 1], atol=1e-12, rtol=0)


def test_split_bounds_fixed_size_and_aligned():
    for S in (32, 256):
        for pos in (0, 5, S - 1, S, S + 1, 10 * S - 1, 10 * S, 12345):
            b = oracle.split_bounds(pos, S)
            assert b[0][0] == 0 and b[-1][1] == pos + 1
            assert all(b1 == a2 for (_, b1), (a2, _) in zip(b, b[1:]))
            assert all(k0 == j * S for j, (k0, _) in enumerate(b))
            assert all(k1 - k0 == S for k0, k1 in b[:-1]) and 1 <= b[-1][1] - b[-1][0] <= S
            assert len(b) == pos // S + 1


# ----------------------------------------------------------------------------- page update
def test_kv_page_update_roundtrip():
    shape = AttnShape(4, 2, 8, page_size=4, split_size=32, dtype="f32")
    seqs = [SeqSpec(0, 5, 3), SeqSpec(1, 0, 9), SeqSpec(2, 12, 1), SeqSpec(3, 7, 0)]
    bt = build_batch(shape, seqs, seed=5, page_seed=3, extra_pages=2)
    kc, vc = bt.k_pool.copy(), bt.v_pool.copy()
    before = kc.copy()
    oracle.kv_page_update(bt.k_new, bt.v_new, bt.q_starts, bt.seq_lens, bt.page_table, kc, vc)
    from synth import token_values
    written = np.zeros(kc.shape[:1] + kc.shape[2:3], bool)   # [page][slot]
    for b, s in enumerate(seqs):
        for name, cache in (("k", kc), ("v", vc)):
            ref = token_values(5, s.req, name, 0, s.seq_len, 2, 8, "f32")
            got = oracle.gather_kv(cache, bt.page_table[b], s.seq_len)
            assert np.array_equal(got, ref.astype(np.float64))
        for pos in range(s.cached, s.seq_len):
            written[bt.page_table[b][pos // 4], pos % 4] = True
    # nothing else was touched
    untouched = ~written[:, None, :, None].repeat(2, 1).repeat(8, 3)
    assert np.array_equal(np.isnan(kc[untouched]), np.isnan(before[untouched]))
    assert np.array_equal(np.nan_to_num(kc[untouched]), np.nan_to_num(before[untouched]))


# ----------------------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes():
    """Slips planted in copies of the computation (CPU only) must fail the pins above."""
    c = random_case(12)
    ref = brute_force(c["q"], c["ks"], c["vs"], c["n_new"])
    # 1. wrong scale
    assert not np.allclose(run_oracle(c, scale=1.0 / 8), ref, atol=1e-6)
    # 2. wrong GQA mapping (h % Hkv instead of h // G)
    wrong = brute_force(c["q"], c["ks"], c["vs"], c["n_new"], gqa=lambda h, G, Hkv: h % Hkv)
    assert not np.allclose(wrong, ref, atol=1e-6)
    # 3. mask off by one (a token not seeing itself): shift positions by one
    lens = [k.shape[0] for k in c["ks"]]
    short = [dict(k=k[: L - 1], v=v[: L - 1]) for k, v, L in zip(c["ks"], c["vs"], lens)]
    sub = brute_force(c["q"][1:2], [short[0]["k"]], [short[0]["v"]], [1])
    assert not np.allclose(sub[0], ref[0], atol=1e-6)
    # 4. transposed page lookup (slot-major instead of page-major) breaks the gather
    kp_t = c["kp"].transpose(0, 2, 1, 3).copy().reshape(c["kp"].shape)
    bad = oracle.paged_attention(c["q"], kp_t, c["vp"], c["table"], c["q_starts"],
                                 c["seq_lens"], c["Hkv"])
    assert not np.allclose(np.nan_to_num(bad), ref, atol=1e-6)
    # 5. a fold that forgets to rescale the running sum
    rng = np.random.default_rng(1)
    K, V, q = rng.standard_normal((100, 8)), rng.standard_normal((100, 8)), rng.standard_normal(8) * 3
    parts = [oracle.split_partial(K[a:b] @ q * math.log2(math.e) / math.sqrt(8), V[a:b])
             for a, b in oracle.split_bounds(99, 32)]
    M, L, A = parts[0]
    for m, l, acc in parts[1:]:
        Mn = max(M, m)
        L = L + l * 2.0 ** (m - Mn)            # slip: no 2^(M - M') on L
        A = A * 2.0 ** (M - Mn) + acc * 2.0 ** (m - Mn)
        M = Mn
    s = K @ q / math.sqrt(8)
    w = np.exp(s - s.max())
    good = (w / w.sum()) @ V
    assert np.allclose(oracle.fold(parts), good, atol=1e-12)
    assert not np.allclose(A / L, good, atol=1e-6)
