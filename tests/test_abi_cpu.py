"""The C-ABI library loads, exports what include/*.h declare, and validates arguments.

CPU only: every call below fails validation, so nothing is ever launched.
"""

import ctypes
import glob
import os
import re

import pytest

import invariant_attention_amd as bi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(bi_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = bi.load()
    names = declared_functions()
    assert set(names) == set(bi.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings():
    assert bi.bi_status_string(0) == "ok"
    for s in range(1, 5):
        assert bi.bi_status_string(s) not in ("ok", "unknown status")
    assert bi.bi_status_string(99) == "unknown status"


BASE = dict(num_q_heads=64, num_kv_heads=4, head_dim=128, page_size=16, split_size=256,
            dtype=bi.BI_BF16, softmax_scale=0.0, split_policy=bi.BI_SPLIT_FIXED)


@pytest.mark.parametrize("override,status", [
    (dict(num_q_heads=63), bi._lib.BI_EINVAL),                 # Hq % Hkv != 0
    (dict(num_kv_heads=0), bi._lib.BI_EINVAL),
    (dict(head_dim=96), bi._lib.BI_EUNSUPPORTED),
    (dict(head_dim=256), bi._lib.BI_EUNSUPPORTED),
    (dict(page_size=32), bi._lib.BI_EUNSUPPORTED),
    (dict(split_size=48), bi._lib.BI_EUNSUPPORTED),            # not a multiple of 32
    (dict(split_size=0), bi._lib.BI_EINVAL),
    (dict(dtype=7), bi._lib.BI_EINVAL),
    (dict(split_policy=3), bi._lib.BI_EINVAL),
    (dict(softmax_scale=-1.0), bi._lib.BI_EINVAL),
    (dict(softmax_scale=float("nan")), bi._lib.BI_EINVAL),
    (dict(num_q_heads=12, num_kv_heads=4), bi._lib.BI_EUNSUPPORTED),   # group 3
    (dict(num_q_heads=128, num_kv_heads=1), bi._lib.BI_EUNSUPPORTED),  # group 128
])
def test_config_validation(override, status):
    cfg = bi.AttnConfig(**{**BASE, **override})
    lib = bi.load()
    c = cfg.c()
    fake = ctypes.c_void_p(0x1000)
    st = lib.bi_attn_decode(ctypes.byref(c), fake, fake, fake, fake, 4, 4, fake, 1, 16, fake,
                            fake, 1 << 30, None)
    assert st == status
    st = lib.bi_attn_prefill(ctypes.byref(c), fake, fake, fake, fake, 4, 4, fake, fake, 1, 1, 1,
                             16, fake, None, 0, None)
    assert st == status
    st = lib.bi_kv_page_update(ctypes.byref(c), fake, fake, fake, fake, fake, 4, 4, 1, 1, fake,
                               fake, None)
    assert st == status
    assert lib.bi_attn_workspace_bytes(ctypes.byref(c), 4, 100) == 0


def test_argument_validation_launches_nothing():
    lib = bi.load()
    c = bi.AttnConfig(**BASE).c()
    f = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    E = bi._lib
    # null pointers
    assert lib.bi_attn_decode(ctypes.byref(c), None, f, f, f, 4, 4, f, 1, 16, f, f, 1 << 30, None) == E.BI_EINVAL
    assert lib.bi_attn_prefill(ctypes.byref(c), f, f, f, f, 4, 4, None, f, 1, 1, 1, 16, f, None, 0, None) == E.BI_EINVAL
    assert lib.bi_kv_page_update(ctypes.byref(c), f, f, f, f, None, 4, 4, 1, 1, f, f, None) == E.BI_EINVAL
    assert lib.bi_attn_decode(None, f, f, f, f, 4, 4, f, 1, 16, f, f, 1 << 30, None) == E.BI_EINVAL
    # negative sizes
    assert lib.bi_attn_decode(ctypes.byref(c), f, f, f, f, 4, 4, f, -1, 16, f, f, 1 << 30, None) == E.BI_EINVAL
    assert lib.bi_attn_prefill(ctypes.byref(c), f, f, f, f, 4, 4, f, f, 1, -2, 1, 16, f, None, 0, None) == E.BI_EINVAL
    # misaligned
    assert lib.bi_attn_decode(ctypes.byref(c), odd, f, f, f, 4, 4, f, 1, 16, f, f, 1 << 30, None) == E.BI_EINVAL
    # workspace missing or too small
    need = lib.bi_attn_workspace_bytes(ctypes.byref(c), 1, 16)
    assert need > 0
    assert lib.bi_attn_decode(ctypes.byref(c), f, f, f, f, 4, 4, f, 1, 16, f, None, 0, None) == E.BI_EWORKSPACE
    assert lib.bi_attn_decode(ctypes.byref(c), f, f, f, f, 4, 4, f, 1, 16, f, f, need - 1, None) == E.BI_EWORKSPACE
    # partials of one (sequence, KV head) reaching 2 GiB: refused before the workspace check
    G, D = BASE["num_q_heads"] // BASE["num_kv_heads"], BASE["head_dim"]
    lim = (1 << 31) // (G * D * 4) * BASE["split_size"]   # first max_seq_len refused
    assert lib.bi_attn_decode(ctypes.byref(c), f, f, f, f, 4, 4, f, 1, lim, f, None, 0, None) == E.BI_EUNSUPPORTED
    assert lib.bi_attn_decode_combine(ctypes.byref(c), f, 1, lim, f, None, 0, None) == E.BI_EUNSUPPORTED
    assert lib.bi_attn_decode(ctypes.byref(c), f, f, f, f, 4, 4, f, 1, lim - BASE["split_size"], f, None, 0,
                              None) == E.BI_EWORKSPACE
    # empty work is a no-op success
    assert lib.bi_attn_decode(ctypes.byref(c), None, None, None, None, 0, 0, None, 0, 0, None, None, 0, None) == E.BI_OK
    assert lib.bi_attn_prefill(ctypes.byref(c), None, None, None, None, 0, 0, None, None, 0, 0, 0, 0, None, None, 0, None) == E.BI_OK


def test_workspace_bytes_formula():
    lib = bi.load()
    c = bi.AttnConfig(**BASE).c()
    # fixed policy: rows * ceil(len / S) * (8 + 4 D), with the (m, l) block padded to 256 B
    for rows, L in ((1, 1), (3, 256), (64, 8192), (8, 131072)):
        J = (L + 255) // 256
        ml = (rows * 64 * J * 8 + 255) // 256 * 256
        assert lib.bi_attn_workspace_bytes(ctypes.byref(c), rows, L) == ml + rows * 64 * J * 128 * 4


def test_bindings_refuse_host_and_strided_tensors():
    """The binding hands the kernels raw row-major addresses, so it refuses host tensors and
    strided views (with an error, before any GPU call) instead of letting them be misread."""
    import torch

    import invariant_attention_amd as bi

    a = torch.zeros((4, 64), dtype=torch.bfloat16)
    w = torch.zeros((128, 64), dtype=torch.bfloat16)
    c = torch.zeros((4, 128), dtype=torch.float32)
    with pytest.raises(bi.BiAttnError):
        bi.bi_gemm(a, w, c)
    x = torch.zeros((3, 512))[:, :256]
    assert not x.is_contiguous()
    with pytest.raises(bi.BiAttnError):
        bi.bi_rmsnorm(x, torch.ones(256), torch.zeros((3, 256)), 1e-6)
    with pytest.raises(bi.BiAttnError):    # weight of the wrong length: refused before any call
        bi.bi_rmsnorm(torch.zeros((3, 256)), torch.ones(255), torch.zeros((3, 256)), 1e-6)


def test_bindings_refuse_wrong_dtypes_and_shapes():
    """Every attention entry point checks each tensor's dtype against cfg.dtype (index arrays
    int32, out fp32) and its shape against the configured heads, head_dim and page size, before
    any GPU call: a mismatch would otherwise be read or written past the tensor."""
    import torch

    cfg = bi.AttnConfig(**BASE)           # bf16, Hq 64, Hkv 4, D 128, page 16
    B, T, P = 2, 5, 6
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32

    def good():
        return dict(q=torch.zeros((T, 64, 128), dtype=bf), kc=torch.zeros((P, 4, 16, 128), dtype=bf),
                    vc=torch.zeros((P, 4, 16, 128), dtype=bf), pt=torch.zeros((B, 3), dtype=i32),
                    qs=torch.zeros(B + 1, dtype=i32), sl=torch.zeros(B, dtype=i32),
                    out=torch.zeros((T, 64, 128), dtype=f32), kn=torch.zeros((T, 4, 128), dtype=bf))

    def prefill(**kw):
        a = {**good(), **kw}
        bi.bi_attn_prefill(cfg, a["q"], a["kc"], a["vc"], a["pt"], a["qs"], a["sl"], 4, 64, a["out"])

    def decode(**kw):
        a = {**good(), **kw}
        q = a["q"][:B] if "q" not in kw else a["q"]
        out = a["out"][:B] if "out" not in kw else a["out"]
        bi.bi_attn_decode(cfg, q, a["kc"], a["vc"], a["pt"], a["sl"], 64, out, torch.zeros(8))

    def update(**kw):
        a = {**good(), **kw}
        bi.bi_kv_page_update(cfg, a["kn"], a["kn"] if "kn" in kw else a["kn"].clone(), a["qs"],
                             a["sl"], a["pt"], a["kc"], a["vc"])

    def append(**kw):
        a = {**good(), **kw}
        q = a["q"][:B] if "q" not in kw else a["q"]
        out = a["out"][:B] if "out" not in kw else a["out"]
        kn = a["kn"][:B] if "kn" not in kw else a["kn"]
        bi.bi_attn_decode_append(cfg, q, kn, kn.clone(), a["kc"], a["vc"], a["pt"], a["sl"], 64, out,
                                 torch.zeros(8))

    bad_cases = [
        (prefill, dict(q=torch.zeros((T, 64, 128), dtype=f32)), "q must be"),           # fp32 q, bf16 cfg
        (prefill, dict(out=torch.zeros((T, 64, 128), dtype=bf)), "out must be"),         # bf16 out
        (prefill, dict(kc=torch.zeros((P, 4, 16, 128), dtype=f32)), "k_cache must be"),
        (prefill, dict(kc=torch.zeros((P * 64, 128), dtype=bf)), "k_cache must have"),   # flattened
        (prefill, dict(vc=torch.zeros((P, 4, 16, 64), dtype=bf)), "v_cache must have"),
        (prefill, dict(q=torch.zeros((T, 32, 128), dtype=bf)), "q must have"),           # wrong Hq
        (prefill, dict(qs=torch.zeros(B, dtype=i32)), "q_starts must have"),             # B, not B+1
        (prefill, dict(qs=torch.zeros(B + 1, dtype=torch.int64)), "q_starts must be"),
        (prefill, dict(pt=torch.zeros((B + 1, 3), dtype=i32)), "page_table must have"),
        (prefill, dict(out=torch.zeros((T + 1, 64, 128), dtype=f32)), "out must have"),
        (decode, dict(q=torch.zeros((B + 1, 64, 128), dtype=bf)), "q must have"),        # q rows != batch
        (decode, dict(out=torch.zeros((B, 64, 128), dtype=bf)), "out must be"),
        (decode, dict(sl=torch.zeros(B, dtype=torch.int64)), "seq_lens must be"),
        (update, dict(kn=torch.zeros((T, 4, 128), dtype=f32)), "k_new must be"),
        (update, dict(pt=torch.zeros((B, 3), dtype=torch.int16)), "page_table must be"),
        (append, dict(kn=torch.zeros((B + 1, 4, 128), dtype=bf)), "k_new must have"),    # one row per sequence
        (append, dict(kn=torch.zeros((B, 4, 128), dtype=f32)), "k_new must be"),
        (append, dict(out=torch.zeros((B, 64, 128), dtype=bf)), "out must be"),
    ]
    for fn, kw, msg in bad_cases:
        with pytest.raises(bi.BiAttnError, match=msg):
            fn(**kw)
    # well-formed host tensors pass the checks and are then refused as host tensors
    with pytest.raises(bi.BiAttnError, match="contiguous GPU tensors"):
        prefill()
