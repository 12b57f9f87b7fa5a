"""The stream argument: every entry point run on a side stream (the binding's default is the
current stream; GEMM and RMSNorm also take it explicitly) gives the same bits as on the
default stream (GPU)."""

import pytest
import torch

import invariant_attention_amd as bi
from gpu_harness import assert_bitwise, to_device
from synth import AttnShape, SeqSpec, build_batch, gemm_inputs, norm_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _attention(cfg, bt):
    d = to_device(bt, cfg)
    bi.bi_kv_page_update(cfg, d.k_new, d.v_new, d.q_starts, d.seq_lens, d.page_table, d.k_cache, d.v_cache)
    out = torch.full((d.q.shape[0], cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda")
    bi.bi_attn_prefill(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.q_starts, d.seq_lens,
                       d.max_q_len, d.max_seq_len, out)
    last = torch.tensor([int(bt.q_starts[b + 1]) - 1 for b in range(bt.batch)], device="cuda")
    ql = d.q[last].contiguous()
    outd = torch.full((bt.batch, cfg.num_q_heads, cfg.head_dim), float("nan"), device="cuda")
    ws = torch.full((bi.bi_attn_workspace_bytes(cfg, bt.batch, d.max_seq_len) // 4 + 1,), float("nan"),
                    device="cuda")
    bi.bi_attn_decode(cfg, ql, d.k_cache, d.v_cache, d.page_table, d.seq_lens, d.max_seq_len, outd, ws)
    return out, outd


def test_side_stream_same_bits():
    print("CASE streams", flush=True)
    shape = AttnShape(32, 4, 128, 16, 256, "bf16")
    cfg = bi.AttnConfig(32, 4, 128, 16, 256, bi.BI_BF16)
    bt = build_batch(shape, [SeqSpec(0, 700, 33), SeqSpec(1, 0, 5), SeqSpec(2, 256, 1)], seed=7,
                     page_seed=8, extra_pages=2)
    x, wn = norm_inputs(9, 33, 512, "bf16")
    a, w = gemm_inputs(10, 70, 256, 320)
    xd, wnd = torch.from_numpy(x).cuda().to(torch.bfloat16), torch.from_numpy(wn).cuda().to(torch.bfloat16)
    ad, wd = torch.from_numpy(a).cuda().to(torch.bfloat16), torch.from_numpy(w).cuda().to(torch.bfloat16)

    out0, outd0 = _attention(cfg, bt)
    y0 = torch.empty_like(xd)
    bi.bi_rmsnorm(xd, wnd, y0, 1e-6)
    c0 = torch.empty((70, 256), device="cuda")
    bi.bi_gemm(ad, wd, c0)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()            # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):         # attention: the binding takes the current stream
        out1, outd1 = _attention(cfg, bt)
    y1 = torch.empty_like(xd)
    c1 = torch.empty((70, 256), device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    bi.bi_rmsnorm(xd, wnd, y1, 1e-6, stream=side)   # explicit stream argument
    bi.bi_gemm(ad, wd, c1, stream=side)
    side.synchronize()
    assert_bitwise(out1, out0, "prefill on a side stream")
    assert_bitwise(outd1, outd0, "decode on a side stream")
    assert_bitwise(y1.view(torch.int16).to(torch.int32), y0.view(torch.int16).to(torch.int32), "rmsnorm")
    assert_bitwise(c1, c0, "gemm")
