"""Dense varlen attention (trainer form) on the GPU: parity with the fp64 oracle, and the same
bits as the paged prefill and decode routes on the same keys and values (GPU)."""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
import oracle
from synth import AttnShape, SeqSpec, build_batch
from gpu_harness import assert_bitwise, assert_parity, cfg_for, decode_workspace, run_prefill, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _print_case(*a):
    print("CASE", *a, flush=True)


def dense_from_paged(d, seq_lens, pad_rows=0):
    """The sequences' keys and values laid end to end, [total_k][Hkv][D] (the same bits as
    the paged cache), plus pad_rows NaN rows after the last sequence; and k_starts."""
    ks, vs = [], []
    for b, L in enumerate(seq_lens):
        npg = (int(L) + 15) // 16
        pages = d.page_table[b, :npg].long()
        for cache, dst in ((d.k_cache, ks), (d.v_cache, vs)):
            blk = cache[pages]                                   # [npg][Hkv][16][D]
            dst.append(blk.permute(0, 2, 1, 3).reshape(npg * 16, blk.shape[1], blk.shape[3])[: int(L)])
    if pad_rows:
        pad = torch.full((pad_rows,) + tuple(ks[0].shape[1:]), float("nan"), dtype=ks[0].dtype,
                         device=ks[0].device)
        ks.append(pad)
        vs.append(pad.clone())
    k_starts = np.concatenate([[0], np.cumsum(np.asarray(seq_lens, np.int64))]).astype(np.int32)
    return (torch.cat(ks).contiguous(), torch.cat(vs).contiguous(),
            torch.from_numpy(k_starts).cuda())


def run_varlen(cfg, q, k, v, q_starts, k_starts, max_q_len, max_seq_len):
    out = torch.full((q.shape[0], cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda",
                     dtype=torch.float32)
    bi.bi_attn_varlen(cfg, q, k, v, q_starts, k_starts, max_q_len, max_seq_len, out)
    torch.cuda.synchronize()
    return out


CASES = [(64, 4, 128, "bf16"), (32, 4, 128, "bf16"), (8, 8, 64, "bf16"), (64, 4, 128, "f32"),
         (4, 1, 64, "f32")]


@pytest.mark.parametrize("hq,hkv,d,dtype", CASES)
def test_varlen_parity_and_same_bits_as_paged(hq, hkv, d, dtype):
    shape = AttnShape(hq, hkv, d, 16, 256, dtype)
    cfg = cfg_for(shape)
    # ragged lengths: not multiples of 16 or 32, a whole-sequence prefill, single tokens,
    # and a long prefix (several 256-key splits)
    seqs = [SeqSpec(0, 0, 37), SeqSpec(1, 300, 5), SeqSpec(2, 781, 200), SeqSpec(3, 15, 1),
            SeqSpec(4, 0, 16), SeqSpec(5, 511, 2)]
    _print_case("varlen", hq, hkv, d, dtype)
    bt = build_batch(shape, seqs, seed=31, page_seed=9, extra_pages=3)
    dv = to_device(bt, cfg)
    out_paged = run_prefill(cfg, dv)                       # also writes the new tokens
    k, v, k_starts = dense_from_paged(dv, bt.seq_lens, pad_rows=19)
    out = run_varlen(cfg, dv.q, k, v, dv.q_starts, k_starts, dv.max_q_len, dv.max_seq_len)
    assert_bitwise(out, out_paged, f"varlen vs paged prefill {hq}/{hkv}/{d} {dtype}")
    ref = oracle.varlen_attention(dv.q.float().cpu().numpy(), k.float().cpu().numpy(),
                                  v.float().cpu().numpy(), bt.q_starts, k_starts.cpu().numpy(), hkv)
    assert_parity(out.cpu().numpy(), ref, f"varlen {hq}/{hkv}/{d} {dtype}")


@pytest.mark.parametrize("hq,hkv,d,dtype", [(64, 4, 128, "bf16"), (8, 8, 64, "bf16")])
def test_varlen_last_tokens_equal_decode(hq, hkv, d, dtype):
    """The last token of each sequence: dense varlen == paged decode, bit for bit."""
    shape = AttnShape(hq, hkv, d, 16, 256, dtype)
    cfg = cfg_for(shape)
    seqs = [SeqSpec(0, 100, 30), SeqSpec(1, 1000, 3), SeqSpec(2, 0, 1), SeqSpec(3, 255, 2)]
    _print_case("varlen vs decode", hq, hkv, d, dtype)
    bt = build_batch(shape, seqs, seed=32, page_seed=10)
    dv = to_device(bt, cfg)
    run_prefill(cfg, dv)
    k, v, k_starts = dense_from_paged(dv, bt.seq_lens)
    out = run_varlen(cfg, dv.q, k, v, dv.q_starts, k_starts, dv.max_q_len, dv.max_seq_len)
    last = (dv.q_starts[1:] - 1).long()
    q_last = dv.q[last].contiguous()
    B = len(seqs)
    out_d = torch.full((B, hq, d), float("nan"), device="cuda", dtype=torch.float32)
    ws = decode_workspace(cfg, B, dv.max_seq_len)
    bi.bi_attn_decode(cfg, q_last, dv.k_cache, dv.v_cache, dv.page_table, dv.seq_lens,
                      dv.max_seq_len, out_d, ws)
    torch.cuda.synchronize()
    assert_bitwise(out[last], out_d, "varlen last tokens vs decode")


def test_varlen_batch_invariance_and_bad_ranges():
    """Each sequence alone == in the batch, bit for bit; a sequence whose rows run past the
    arrays gets NaN rows and leaves the others' bits unchanged."""
    shape = AttnShape(64, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    seqs = [SeqSpec(0, 64, 50), SeqSpec(1, 700, 9), SeqSpec(2, 5, 40)]
    _print_case("varlen invariance")
    bt = build_batch(shape, seqs, seed=33, page_seed=11)
    dv = to_device(bt, cfg)
    run_prefill(cfg, dv)
    k, v, k_starts = dense_from_paged(dv, bt.seq_lens)
    full = run_varlen(cfg, dv.q, k, v, dv.q_starts, k_starts, dv.max_q_len, dv.max_seq_len)
    qs = bt.q_starts
    for b in range(len(seqs)):
        k0, k1 = int(k_starts[b]), int(k_starts[b + 1])
        q0, q1 = int(qs[b]), int(qs[b + 1])
        one = run_varlen(cfg, dv.q[q0:q1].contiguous(), k[k0:k1].contiguous(), v[k0:k1].contiguous(),
                         torch.tensor([0, q1 - q0], dtype=torch.int32, device="cuda"),
                         torch.tensor([0, k1 - k0], dtype=torch.int32, device="cuda"),
                         q1 - q0, k1 - k0)
        assert_bitwise(one, full[q0:q1], f"varlen sequence {b} alone vs batch")
    # the last sequence claims rows past the arrays
    bad = k_starts.clone()
    bad[-1] = k.shape[0] + 5
    out = run_varlen(cfg, dv.q, k, v, dv.q_starts, bad, dv.max_q_len, dv.max_seq_len + 5)
    q_last0 = int(qs[-2])
    assert torch.isnan(out[q_last0:]).all(), "rows of the out-of-range sequence must be NaN"
    assert_bitwise(out[:q_last0], full[:q_last0], "other sequences unchanged")
