"""Parity of the HIP path with the CPU oracle at sizes the oracle finishes in
seconds: several tiles, ragged tails, every head grouping, both dtypes.

The attention stages are fed the GPU's own inputs (stage-wise parity); the
projection stage compares the GPU GEMM with the fp64 product of the same
values."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mqa_qkv_proj_amd
    return mqa_qkv_proj_amd


def torch():
    import torch as t
    return t


# ----------------------------------------------------------------------------- projection

PROJ = [  # M, hidden, H_q, H_kv, d, dtype
    (1, 256, 4, 2, 64, "bf16"), (7, 512, 8, 1, 128, "bf16"), (33, 256, 4, 4, 64, "bf16"),
    (130, 384, 8, 2, 64, "bf16"), (300, 1024, 16, 2, 128, "bf16"), (1029, 264, 4, 2, 64, "bf16"),
    (1000, 192, 5, 1, 64, "bf16"), (4100, 256, 13, 1, 64, "bf16"),
    # more tiles than CUs: 128 x 128 tiles one per CU (M = 4133), 128 x 160 two per CU with a
    # ragged last column tile (N = 6144)
    (4133, 256, 32, 4, 64, "bf16"), (2100, 256, 32, 8, 128, "bf16"),
    # the copy ring past the last k tile: one k tile (hidden 64) and two (hidden 128), tile path
    (300, 64, 4, 2, 64, "bf16"), (517, 128, 8, 2, 64, "bf16"),
    (128, 512, 4, 2, 64, "bf16"), (100, 1024, 8, 1, 128, "bf16"), (8, 256, 64, 2, 128, "bf16"),
    (24, 384, 4, 2, 64, "bf16"), (32, 128, 12, 2, 128, "bf16"),
    (128, 256, 4, 2, 64, "f32"), (45, 100, 2, 1, 128, "f32"),
    # 8-wave workgroups over all of K (hidden % 256 == 0): 16-row tiles (M <= 64, small
    # grids), 32-row tiles, and M <= 32 on a 12288-column weight; ragged row tiles
    (33, 512, 4, 2, 64, "bf16"), (97, 2048, 8, 2, 128, "bf16"), (64, 1024, 16, 2, 128, "bf16"),
    (20, 512, 32, 32, 128, "bf16"),
    # M <= 32 on decode-width weights (5120-10240 columns, K = 1024..4096): the register-
    # transpose kernel (one and two 16-row blocks; 1, 2 and 4 k steps per wave; one k range
    # at K = 256) and the reduce kernel, ragged M down to one row
    (32, 4096, 32, 8, 128, "bf16"), (17, 3072, 24, 8, 128, "bf16"), (1, 1024, 40, 4, 128, "bf16"),
    (9, 2048, 40, 4, 128, "bf16"), (32, 1024, 64, 8, 128, "bf16"), (8, 256, 64, 2, 128, "bf16"),
    # the skinny split-K kernel: hidden not a multiple of 256 (M <= 32 on a wide weight; M > 32)
    (20, 640, 64, 2, 128, "bf16"), (40, 384, 4, 2, 64, "bf16"),
]


@pytest.mark.parametrize("M,hidden,H_q,H_kv,d,dtype", PROJ)
def test_qkv_proj_matches_oracle(m, M, hidden, H_q, H_kv, d, dtype):
    say("qkv_proj", M, hidden, H_q, H_kv, d, dtype)
    N = (H_q + 2 * H_kv) * d
    enc = W.round_bf16 if dtype == "bf16" else (lambda a: a)
    x = enc(W.normal(11, M, (M, hidden)))
    w = enc(W.normal(12, hidden, (hidden, N), std=1.0 / math.sqrt(hidden)))
    got = m.qkv_proj(dev(x, dtype), dev(w, dtype), H_q, H_kv, d)
    ref = oracle.qkv_proj(x, w)
    assert_close(host(got), ref, dtype, f"qkv_proj M={M}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qkv_proj_bias(m, dtype):
    M, hidden, H_q, H_kv, d = 70, 256, 4, 2, 64
    N = (H_q + 2 * H_kv) * d
    enc = W.round_bf16 if dtype == "bf16" else (lambda a: a)
    x, w = enc(W.normal(1, 1, (M, hidden))), enc(W.normal(1, 2, (hidden, N), std=0.0625))
    bias = enc(W.normal(1, 3, (1, N))[0])
    got = m.qkv_proj(dev(x, dtype), dev(w, dtype), H_q, H_kv, d, bias=dev(bias, dtype))
    assert_close(host(got), oracle.qkv_proj(x, w, bias), dtype, "qkv_proj+bias")


@pytest.mark.parametrize("M", [5, 64, 700])
def test_qkv_proj_exact_on_integers(m, M):
    """Small-integer x and sparse {-1,0,1} W: every sum is an integer <= 256, exact in bf16."""
    rng = np.random.default_rng(M)
    hidden, H_q, H_kv, d = 512, 4, 2, 64
    N = (H_q + 2 * H_kv) * d
    x = rng.integers(-2, 3, size=(M, hidden)).astype(np.float32)
    w = (rng.integers(-1, 2, size=(hidden, N)) * (rng.random((hidden, N)) < 0.2)).astype(np.float32)
    for dtype in ("bf16", "f32"):
        got = host(m.qkv_proj(dev(x, dtype), dev(w, dtype), H_q, H_kv, d))
        assert np.array_equal(got, oracle.qkv_proj(x, w)), dtype


def test_qkv_proj_one_hot_column_selection(m):
    M, hidden, H_q, H_kv, d = 96, 256, 4, 2, 64
    N = (H_q + 2 * H_kv) * d
    x = W.round_bf16(W.normal(5, 5, (M, hidden)))
    w = np.zeros((hidden, N), np.float32)
    w[np.arange(N) % hidden, np.arange(N)] = 1.0
    got = host(m.qkv_proj(dev(x, "bf16"), dev(w, "bf16"), H_q, H_kv, d))
    assert np.array_equal(got, x[:, np.arange(N) % hidden].astype(np.float64))


def test_fused_equals_three_separate_projections(m):
    """One fused call vs three calls on the column blocks of W (the pages' claim).

    Each block W_q, W_k, W_v is run as its own projection (zero-padded to a width
    the call accepts, the padding columns dropped afterwards)."""
    M, hidden, H_q, H_kv, d = 200, 512, 8, 2, 64
    N = (H_q + 2 * H_kv) * d
    x = W.round_bf16(W.normal(9, 9, (M, hidden)))
    w = W.round_bf16(W.normal(9, 10, (hidden, N), std=0.04))
    xd = dev(x, "bf16")
    fused = host(m.qkv_proj(xd, dev(w, "bf16"), H_q, H_kv, d))
    parts = []
    for lo, hi in ((0, H_q * d), (H_q * d, (H_q + H_kv) * d), ((H_q + H_kv) * d, N)):
        n = hi - lo
        pad = max(0, 3 * d - n)
        wb = np.concatenate([w[:, lo:hi], np.zeros((hidden, pad), np.float32)], axis=1)
        heads = wb.shape[1] // d
        parts.append(host(m.qkv_proj(xd, dev(wb, "bf16"), heads - 2, 1, d))[:, :n])
    sep = np.concatenate(parts, axis=1)
    assert_close(fused, sep, "bf16", "fused vs separate", max_abs=1e-2, rel_l2=1e-3)


# ----------------------------------------------------------------------------- prefill

PREFILL = [  # B, L_q, L_kv, H_q, H_kv, d, causal
    (2, 200, 200, 8, 2, 64, True),
    (2, 200, 200, 8, 2, 128, False),
    (1, 130, 130, 4, 4, 128, True),     # MHA
    (1, 257, 257, 16, 1, 64, True),     # MQA, G=16
    (1, 97, 97, 8, 1, 128, False),      # MQA G=8
    (2, 65, 65, 6, 2, 64, True),        # G=3 (not a power of two)
    (1, 77, 300, 4, 2, 128, True),      # L_q < L_kv: bottom-right causal
    (1, 1, 1, 2, 1, 64, True),          # single token
    (3, 1, 129, 4, 2, 128, False),      # one query row
    (1, 64, 64, 64, 2, 64, True),       # G=32
    (1, 640, 640, 8, 2, 128, False),    # ten full tiles: every LDS stage reused several times
    (1, 700, 900, 4, 1, 64, True),      # long pipelined run, L_q < L_kv, ragged last tile
]


@pytest.mark.parametrize("B,L_q,L_kv,H_q,H_kv,d,causal", PREFILL)
@pytest.mark.parametrize("odt", ["bf16", "f32"])
def test_prefill_bf16_matches_oracle(m, B, L_q, L_kv, H_q, H_kv, d, causal, odt):
    t = torch()
    say("prefill", B, L_q, L_kv, H_q, H_kv, d, causal, odt)
    inp = W.small("bf16", 100 + L_q + H_q, B, L_q, L_kv, H_q, H_kv, d)
    q, k, v = (dev(inp[n], "bf16") for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = m.gqa_attn_prefill(q, k, v, causal=causal, scale=scale, return_lse=True,
                                out_dtype=t.float32 if odt == "f32" else t.bfloat16)
    ref_o, ref_l = oracle.attention(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_close(host(o), ref_o, "bf16", "O")
    assert_close(host(lse), ref_l, "bf16", "LSE", max_abs=1e-3, rel_l2=1e-4)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_f32_matches_oracle(m, causal, d):
    B, L, H_q, H_kv = 2, 150, 4, 2
    inp = W.small("f32", 3, B, L, L, H_q, H_kv, d)
    q, k, v = (dev(inp[n], "f32") for n in ("q", "k", "v"))
    o, lse = m.gqa_attn_prefill(q, k, v, causal=causal, return_lse=True)
    ref_o, ref_l = oracle.attention(inp["q"], inp["k"], inp["v"], causal, 1.0 / math.sqrt(d))
    assert_close(host(o), ref_o, "f32", "O f32")
    assert_close(host(lse), ref_l, "f32", "LSE f32")


def test_prefill_workspace_reuse(m):
    """One caller-owned workspace serves calls of different sizes in a row; each
    call rewrites every V^T image it reads, so results equal fresh-workspace ones
    bit for bit.  A workspace that is too small is rejected on the host."""
    t = torch()
    say("prefill workspace reuse")
    cases = [(2, 300, 300, 8, 2, 128, True), (1, 70, 130, 4, 4, 64, False), (2, 65, 65, 8, 1, 128, True)]
    need = max(m.prefill_workspace_bytes(B, Lkv, Hkv, d) for B, _, Lkv, _, Hkv, d, _ in cases)
    ws = t.full((need,), 0xFF, dtype=t.uint8, device="cuda")  # NaN-pattern garbage to start from
    for i, (B, L_q, L_kv, H_q, H_kv, d, causal) in enumerate(cases):
        inp = W.small("bf16", 40 + i, B, L_q, L_kv, H_q, H_kv, d)
        q, k, v = (dev(inp[n], "bf16") for n in ("q", "k", "v"))
        o1 = m.gqa_attn_prefill(q, k, v, causal=causal, out_dtype=t.float32, workspace=ws)
        o2 = m.gqa_attn_prefill(q, k, v, causal=causal, out_dtype=t.float32)
        assert t.equal(o1, o2), f"case {i}"
        assert t.isfinite(o1).all()
    small = t.empty(m.prefill_workspace_bytes(2, 300, 2, 128) - 16, dtype=t.uint8, device="cuda")
    inp = W.small("bf16", 40, 2, 300, 300, 8, 2, 128)
    q, k, v = (dev(inp[n], "bf16") for n in ("q", "k", "v"))
    with pytest.raises(m.MqkvInvalid):
        m.gqa_attn_prefill(q, k, v, workspace=small)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_d64_workgroup_shapes_agree(m, causal):
    """d=64 grids under two 8-wave workgroups per CU split each row block's
    key tiles between two waves (even and odd tiles) and merge the two partial
    softmax results at the end.  A batch of 8 sequences (an 8-wave grid of
    8 x 4 x 64 = 2048 blocks, one wave per row block) and each sequence on its
    own (256 blocks: the key-split grid) sum in different orders, so they are
    compared with the oracle's bar rather than bit for bit: every sequence run
    alone against the batch, on all rows of three heads, and both against the
    oracle on sampled rows, LSE included."""
    t = torch()
    B, L, H_q, H_kv, d = 8, 2048, 32, 4, 64
    say("prefill d=64 workgroup shapes", causal)
    g = t.Generator().manual_seed(77)
    q = t.randn(B, L, H_q, d, generator=g).to(t.bfloat16).cuda()
    k = t.randn(B, L, H_kv, d, generator=g).to(t.bfloat16).cuda()
    v = t.randn(B, L, H_kv, d, generator=g).to(t.bfloat16).cuda()
    scale = 1.0 / math.sqrt(d)
    o, lse = m.gqa_attn_prefill(q, k, v, causal=causal, return_lse=True, out_dtype=t.float32)
    rows = np.array([0, 1, 31, 32, 63, 64, 127, 128, 1000, 2047])
    for b in (0, 3, 7):
        ob, lb = m.gqa_attn_prefill(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=causal, return_lse=True,
                                    out_dtype=t.float32)
        for h in (0, 9, 31):
            assert_close(host(ob[0, :, h]), host(o[b, :, h]), "bf16", f"sequence {b} head {h}: alone vs batch")
        assert np.abs(host(lb[0]) - host(lse[b])).max() < 1e-3, f"sequence {b}: LSE differs"
        for h in (0, 31):
            ref, lref = oracle.attention_rows(host(q), host(k), host(v), b, h, rows, causal, scale)
            assert_close(host(ob[0, rows, h]), ref, "bf16", f"alone b={b} h={h} vs oracle")
            assert np.abs(host(lb[0, h, rows]) - lref).max() < 1e-3
    for b, h in ((0, 0), (7, 31)):
        ref, _ = oracle.attention_rows(host(q), host(k), host(v), b, h, rows, causal, scale)
        assert_close(host(o[b, rows, h]), ref, "bf16", f"batch rows b={b} h={h}")


def test_prefill_on_qkv_views_equals_contiguous_copies(m):
    """The split is zero-copy: strided views of qkv give the same bits as packed copies."""
    t = torch()
    B, L, H_q, H_kv, d = 2, 150, 8, 2, 64
    N = (H_q + 2 * H_kv) * d
    qkv = dev(W.round_bf16(W.normal(4, 4, (B, L, N))), "bf16")
    q, k, v = m.split_qkv(qkv, H_q, H_kv, d)
    assert q.data_ptr() == qkv.data_ptr()
    o1 = m.gqa_attn_prefill(q, k, v, causal=True)
    o2 = m.gqa_attn_prefill(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
    assert t.equal(o1, o2)


# ----------------------------------------------------------------------------- decode

DECODE = [  # B, H_q, H_kv, d, L_max, lens, split
    (3, 8, 2, 128, 300, [1, 77, 300], 0),
    (3, 8, 2, 128, 300, [1, 77, 300], 64),
    (3, 8, 2, 128, 300, [1, 77, 300], 128),
    (3, 8, 2, 128, 300, [1, 33, 300], 32),
    (2, 16, 1, 128, 1040, [17, 1040], 0),
    (4, 4, 4, 64, 200, [200, 5, 64, 65], 64),
    (2, 6, 3, 64, 130, [129, 130], 0),
    (1, 64, 1, 128, 100, [100], 64),     # G = 64 > 32: two query blocks
    # the library's choice on short caches: one workgroup per segment that
    # merges its waves' partials in LDS (no workspace, no second kernel)
    (1, 64, 1, 128, 200, [200], 0),      # four 16-head query blocks
    (64, 32, 8, 128, 600, [600, 1, 31, 32, 33] + [(i * 97) % 600 + 1 for i in range(59)], 0),
    (40, 32, 4, 64, 1000, [1000, 999, 1, 2] + [(i * 211) % 1000 + 1 for i in range(36)], 0),
]


@pytest.mark.parametrize("B,H_q,H_kv,d,L_max,lens,split", DECODE)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_matches_oracle(m, B, H_q, H_kv, d, L_max, lens, split, dtype):
    t = torch()
    say("decode", B, H_q, H_kv, d, L_max, lens, split, dtype)
    enc = W.round_bf16 if dtype == "bf16" else (lambda a: a)
    kc = enc(W.normal(21, L_max, (B, L_max, H_kv, d)))
    vc = enc(W.normal(22, L_max, (B, L_max, H_kv, d)))
    q = enc(W.normal(23, L_max, (B, H_q, d)))
    seq = np.array(lens, np.int32)
    scale = 1.0 / math.sqrt(d)
    o, lse = m.gqa_attn_decode(dev(q, dtype), dev(kc, dtype), dev(vc, dtype),
                               t.from_numpy(seq).cuda(), scale=scale, kv_split=split,
                               return_lse=True, out_dtype=t.float32)
    ref_o, ref_l = oracle.decode(q, kc, vc, seq, scale)
    assert_close(host(o), ref_o, dtype, "decode O")
    assert_close(host(lse), ref_l, dtype, "decode LSE", max_abs=1e-3 if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("B,H_q,H_kv,d,L_max", [(6, 8, 2, 128, 256), (64, 32, 8, 128, 600), (40, 32, 4, 64, 1000),
                                                 (3, 8, 2, 128, 300)])
def test_decode_bf16_output_is_rounded_f32_output(m, B, H_q, H_kv, d, L_max):
    """The bf16 output is the fp32 output rounded to nearest even, bit for bit
    (short caches through the in-LDS merge, the last case through the split
    kernels and their combine)."""
    t = torch()
    say("decode bf16 output", B, H_q, H_kv, d, L_max)
    rng = np.random.default_rng([41, B, d])
    lens = rng.integers(1, L_max + 1, size=B).astype(np.int32)
    lens[0] = L_max
    kd = dev(W.round_bf16(W.normal(41, 1, (B, L_max, H_kv, d))), "bf16")
    vd = dev(W.round_bf16(W.normal(41, 2, (B, L_max, H_kv, d))), "bf16")
    qd = dev(W.round_bf16(W.normal(41, 3, (B, H_q, d))), "bf16")
    ld = t.from_numpy(lens).cuda()
    o32, l32 = m.gqa_attn_decode(qd, kd, vd, ld, return_lse=True, out_dtype=t.float32)
    o16, l16 = m.gqa_attn_decode(qd, kd, vd, ld, return_lse=True, out_dtype=t.bfloat16)
    assert t.equal(o16, o32.to(t.bfloat16)), "bf16 output must be the rounded fp32 output"
    assert t.equal(l16, l32), "LSE must not depend on the output type"


@pytest.mark.parametrize("B,H_q,H_kv,L_max", [(64, 16, 8, 1024), (64, 64, 2, 4096)])
def test_decode_balanced_split_and_workspace_reuse(m, B, H_q, H_kv, L_max):
    """Caches large enough (>= 16384 tiles of 32 keys at capacity) for the
    library's balanced work split, where one workgroup's keys cross sequence
    and head boundaries, with ragged lengths including 1, 31-33 and L_max.
    Three calls share one workspace (filled with NaN bit patterns first, so a
    stale or unwritten partial would show): every call must match the oracle."""
    t = torch()
    d = 128
    say("decode balanced", B, H_q, H_kv, L_max)
    rng = np.random.default_rng([31, B, H_q])
    kc = W.round_bf16(W.normal(31, L_max, (B, L_max, H_kv, d)))
    vc = W.round_bf16(W.normal(32, L_max, (B, L_max, H_kv, d)))
    qd, kd, vd = None, dev(kc, "bf16"), dev(vc, "bf16")
    ws = m.decode_workspace(B, H_q, H_kv, d, L_max)
    ws.fill_(0xFF)
    for call in range(3):
        lens = rng.integers(1, L_max + 1, size=B).astype(np.int32)
        lens[:6] = [1, 31, 32, 33, L_max, L_max - 1]
        q = W.round_bf16(W.normal(33 + call, L_max, (B, H_q, d)))
        scale = 1.0 / math.sqrt(d)
        o, lse = m.gqa_attn_decode(dev(q, "bf16"), kd, vd, t.from_numpy(lens).cuda(), scale=scale,
                                   return_lse=True, out_dtype=t.float32, workspace=ws)
        ref_o, ref_l = oracle.decode(q, kc, vc, lens, scale)
        assert_close(host(o), ref_o, "bf16", f"decode O (call {call})")
        assert_close(host(lse), ref_l, "bf16", f"decode LSE (call {call})", max_abs=1e-3)


def test_decode_q_as_view_of_qkv_rows(m):
    t = torch()
    B, H_q, H_kv, d, L_max = 4, 8, 2, 64, 150
    N = (H_q + 2 * H_kv) * d
    qkv = W.round_bf16(W.normal(31, 1, (B, N)))
    kc = W.round_bf16(W.normal(31, 2, (B, L_max, H_kv, d)))
    vc = W.round_bf16(W.normal(31, 3, (B, L_max, H_kv, d)))
    seq = np.array([150, 1, 64, 100], np.int32)
    qkv_d = dev(qkv, "bf16")
    q_view = qkv_d[:, :H_q * d].unflatten(-1, (H_q, d))
    o = m.gqa_attn_decode(q_view, dev(kc, "bf16"), dev(vc, "bf16"), t.from_numpy(seq).cuda(),
                          out_dtype=t.float32)
    ref, _ = oracle.decode(qkv[:, :H_q * d].reshape(B, H_q, d), kc, vc, seq, 1 / math.sqrt(d))
    assert_close(host(o), ref, "bf16", "decode q view")
