"""Graph replay (GPU): the calls of a serving step captured once into a HIP graph and replayed.

The graph holds the decode step with the page update folded in (bi_attn_decode_append, writing
into its own copy of the caches), bi_attn_decode with a workspace, the allocation-free decode
and a chunked prefill. Between replays the host writes new query values, new sequence lengths
and new K/V rows into the captured buffers (eager work, then a synchronization); every replay's
outputs, and the cache slots the step wrote, are bitwise equal to the same calls made eagerly on
the same inputs. The library records no memset and no allocation, so capture needs nothing but
the buffers the caller passes.
"""

import numpy as np
import pytest
import torch

import invariant_attention_amd as bi
from synth import AttnShape, SeqSpec, build_batch
from gpu_harness import assert_bitwise, cfg_for, decode_workspace, page_update, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _nan(shape):
    return torch.full(shape, float("nan"), device="cuda", dtype=torch.float32)


def test_graph_replays_equal_eager_calls():
    print("CASE graph replay: decode_append, decode, decode_noalloc, prefill", flush=True)
    shape = AttnShape(32, 4, 128, 16, 256, "bf16")
    cfg = cfg_for(shape)
    dt = cfg.torch_dtype
    rng = np.random.default_rng(310)
    B = 12
    lens = [int(x) for x in rng.integers(300, 9000, B)]
    lens[0], lens[1] = 256, 8193   # a split edge and a row of 33 splits (the long-row combine)
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)], seed=310,
                     page_seed=311, extra_pages=3)
    d = to_device(bt, cfg)
    page_update(cfg, d)   # the new tokens in the cache: the plain decodes read them
    Lmax = d.max_seq_len
    Hq, D = cfg.num_q_heads, cfg.head_dim

    # prefill batch: chunks on top of cached prefixes, one sequence with no new tokens
    bp = build_batch(shape, [SeqSpec(0, 700, 40), SeqSpec(1, 0, 17), SeqSpec(2, 3000, 0),
                             SeqSpec(3, 255, 300)], seed=312, page_seed=313, extra_pages=2)
    p = to_device(bp, cfg)
    page_update(cfg, p)
    Tp = p.q.shape[0]

    # captured buffers
    kc_a, vc_a = d.k_cache.clone(), d.v_cache.clone()   # the append step's own caches
    out_a, out_d, out_n, out_p = _nan((B, Hq, D)), _nan((B, Hq, D)), _nan((B, Hq, D)), _nan((Tp, Hq, D))
    ws_a = decode_workspace(cfg, B, Lmax)
    ws_d = decode_workspace(cfg, B, Lmax)

    def step(kc, vc, oa, od, on, op, wa, wd):
        bi.bi_attn_decode_append(cfg, d.q, d.k_new, d.v_new, kc, vc, d.page_table, d.seq_lens,
                                 Lmax, oa, wa)
        bi.bi_attn_decode(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens, Lmax, od, wd)
        bi.bi_attn_decode_noalloc(cfg, d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens,
                                  Lmax, on)
        bi.bi_attn_prefill(cfg, p.q, p.k_cache, p.v_cache, p.page_table, p.q_starts, p.seq_lens,
                           p.max_q_len, p.max_seq_len, op)

    # eager warm-up on the capture's own buffers (the library's per-device set-up runs here)
    step(kc_a, vc_a, out_a, out_d, out_n, out_p, ws_a, ws_d)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(kc_a, vc_a, out_a, out_d, out_n, out_p, ws_a, ws_d)
    torch.cuda.synchronize()

    for rep in range(3):
        print(f"CASE graph replay {rep}", flush=True)
        if rep > 0:
            # new inputs in the captured buffers: query values, K/V rows of the new tokens and
            # lengths (every length stays within the captured max_seq_len)
            r = np.random.default_rng(320 + rep)
            d.q.copy_(torch.from_numpy(r.standard_normal((B, Hq, D), dtype=np.float32)).to(dt))
            kv_shape = tuple(d.k_new.shape)
            d.k_new.copy_(torch.from_numpy(r.standard_normal(kv_shape, dtype=np.float32)).to(dt))
            d.v_new.copy_(torch.from_numpy(r.standard_normal(kv_shape, dtype=np.float32)).to(dt))
            new_lens = [int(r.integers(1, L + 1)) for L in lens]
            new_lens[1] = lens[1] if rep == 1 else 4097   # 33 splits, then 17
            d.seq_lens.copy_(torch.tensor(new_lens, dtype=torch.int32))
            p.q.copy_(torch.from_numpy(r.standard_normal((Tp, Hq, D), dtype=np.float32)).to(dt))
        # the append step's cache state before the replay, for its eager twin
        kc_e, vc_e = kc_a.clone(), vc_a.clone()
        for o in (out_a, out_d, out_n, out_p):
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        oa, od, on, op = _nan((B, Hq, D)), _nan((B, Hq, D)), _nan((B, Hq, D)), _nan((Tp, Hq, D))
        step(kc_e, vc_e, oa, od, on, op, decode_workspace(cfg, B, Lmax), decode_workspace(cfg, B, Lmax))
        torch.cuda.synchronize()
        assert torch.isfinite(out_a).all() and torch.isfinite(out_d).all()
        assert_bitwise(out_a, oa, f"replay {rep}: decode_append")
        assert_bitwise(out_d, od, f"replay {rep}: decode")
        assert_bitwise(out_n, on, f"replay {rep}: decode_noalloc")
        assert_bitwise(out_p, op, f"replay {rep}: prefill")
        assert_bitwise(kc_a, kc_e, f"replay {rep}: K slots written by the step")
        assert_bitwise(vc_a, vc_e, f"replay {rep}: V slots written by the step")
        # decode_append after the page update equals decode on the same cache only when the
        # step's K/V rows are the ones already in the cache (the first replay)
        if rep == 0:
            assert_bitwise(out_a, out_d, "replay 0: decode_append vs decode")
