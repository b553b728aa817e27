"""Prefill with FP8 (e4m3) scores after the incoherent map (FlashAttention-3
page, FP8 section), against the oracle's fp64 emulation of the same method:
the same random signs, the same per-row Q scales and per-64-key-tile K scales,
the same round-to-nearest-even saturating e4m3 codes.

The bar is the bf16 path's: the oracle takes the quantisation decisions in
fp64 and the kernel in fp32, so a code may differ where a value sits on a
rounding boundary; such flips are rare and far inside the bar, while a wrong
scale, sign or fragment shows up at the size of the FP8 error itself, which
each case checks is well above the bar."""
import math

import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
import workloads as W
from gpu_util import assert_close, dev, errors, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mqa_qkv_proj_amd
    return mqa_qkv_proj_amd


# B, L_q, L_kv, H_q, H_kv, causal, incoherent map on?, outliers
FP8 = [
    (1, 256, 256, 8, 2, True, True, False),
    (2, 200, 200, 8, 2, False, True, True),     # ragged tail of Q and K
    (1, 129, 300, 16, 1, True, True, True),     # MQA, L_q < L_kv, bottom-right causal
    (2, 64, 64, 4, 4, False, False, False),     # plain FP8 (no map), G = 1
    (1, 1, 77, 32, 8, True, False, True),       # one query row
    (1, 333, 333, 12, 4, True, True, False),    # G = 3
]


@pytest.mark.parametrize("B,L_q,L_kv,H_q,H_kv,causal,inc,outl", FP8)
def test_fp8_prefill_matches_oracle(m, B, L_q, L_kv, H_q, H_kv, causal, inc, outl):
    import torch
    d = 128
    say("prefill fp8", B, L_q, L_kv, H_q, H_kv, causal, inc, outl)
    seed = 200 + L_q + L_kv
    q = W.normal(seed, 1, (B, L_q, H_q, d))
    k = W.normal(seed, 2, (B, L_kv, H_kv, d))
    v = W.normal(seed, 3, (B, L_kv, H_kv, d))
    if outl:
        q, k = W.outlier_entries(q, seed, 4), W.outlier_entries(k, seed, 5)
    q, k, v = W.round_bf16(q), W.round_bf16(k), W.round_bf16(v)
    signs = W.random_signs(seed, 6, d) if inc else None
    scale = 1.0 / math.sqrt(d)
    o, lse = m.gqa_attn_prefill_fp8(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"),
                                    signs=dev(signs, "f32") if inc else None, causal=causal, scale=scale,
                                    return_lse=True, out_dtype=torch.float32)
    ref, ref_lse = ofp8.attention_fp8(q, k, v, causal, scale, signs)
    got = host(o)
    assert_close(got, ref, "bf16", "fp8 O (fp32 out)")
    assert_close(host(lse), ref_lse, "bf16", "fp8 LSE", max_abs=1e-3, rel_l2=1e-4)
    # the FP8 error itself (vs exact attention) must be far above the bar, so
    # that the comparison above tests the quantisation and not just attention
    exact, _ = oracle.attention(q, k, v, causal, scale)
    _, fp8_err = errors(ref, exact)
    _, got_err = errors(got, exact)
    say(f"FP8 error vs exact: oracle {fp8_err:.3e}, kernel {got_err:.3e}")
    assert fp8_err > 2 * 5e-3
    assert abs(got_err - fp8_err) < 0.1 * fp8_err


def test_fp8_bf16_output_on_qkv_views(m):
    """Q, K, V consumed in place from projected qkv rows (token stride N), bf16 out."""
    import torch
    B, L, H_q, H_kv, d = 2, 150, 8, 2, 128
    N = (H_q + 2 * H_kv) * d
    qkv = dev(W.round_bf16(W.normal(301, 1, (B, L, N))), "bf16")
    q = qkv[..., :H_q * d].unflatten(-1, (H_q, d))
    k = qkv[..., H_q * d:(H_q + H_kv) * d].unflatten(-1, (H_kv, d))
    v = qkv[..., (H_q + H_kv) * d:].unflatten(-1, (H_kv, d))
    signs = W.random_signs(301, 2, d)
    o = m.gqa_attn_prefill_fp8(q, k, v, signs=dev(signs, "f32"), causal=True)
    assert o.dtype == torch.bfloat16
    ref, _ = ofp8.attention_fp8(host(q), host(k), host(v), True, 1.0 / math.sqrt(d), signs)
    assert_close(host(o), ref, "bf16", "fp8 on qkv views")


def test_fp8_incoherent_processing_cuts_the_error_on_gpu(m):
    """The page's experiment on the kernel: N(0,1) Q, K, V with 0.1% of the Q
    and K entries made 10x larger; against exact fp64 attention, the FP8 error
    with the random-sign Hadamard map must be lower than without it (the same
    margin, 1.1x over four draws, as the oracle's own pin)."""
    import torch
    B, L, H, d = 1, 512, 2, 128
    scale = 1.0 / math.sqrt(d)
    e_plain = e_inc = 0.0
    for s in range(4):
        seed = 400 + s
        q = W.round_bf16(W.outlier_entries(W.normal(seed, 1, (B, L, H, d)), seed, 4))
        k = W.round_bf16(W.outlier_entries(W.normal(seed, 2, (B, L, H, d)), seed, 5))
        v = W.round_bf16(W.normal(seed, 3, (B, L, H, d)))
        exact, _ = oracle.attention(q, k, v, False, scale)
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        plain = m.gqa_attn_prefill_fp8(qd, kd, vd, causal=False, out_dtype=torch.float32)
        inc = m.gqa_attn_prefill_fp8(qd, kd, vd, signs=dev(W.random_signs(seed, 6, d), "f32"), causal=False,
                                     out_dtype=torch.float32)
        e_plain += np.linalg.norm(host(plain) - exact)
        e_inc += np.linalg.norm(host(inc) - exact)
    say(f"FP8 error without / with the incoherent map: {e_plain:.4e} / {e_inc:.4e} "
        f"({e_plain / e_inc:.2f}x)")
    assert e_inc * 1.1 < e_plain


def test_fp8_full_size_sampled_rows(m):
    """A wide-group shape (B=2, L=4096, H_q=32, H_kv=4, causal: G = 8, so the
    8-head workgroups); rows of two heads checked against the oracle, which
    computes those rows only."""
    import torch
    B, L, H_q, H_kv, d = 2, 4096, 32, 4, 128
    say("prefill fp8 full size", B, L, H_q, H_kv)
    g = torch.Generator(device="cpu").manual_seed(11)
    q = torch.randn(B, L, H_q, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, L, H_kv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, L, H_kv, d, generator=g).to(torch.bfloat16)
    signs = W.random_signs(11, 6, d)
    o = m.gqa_attn_prefill_fp8(q.cuda(), k.cuda(), v.cuda(), signs=dev(signs, "f32"), causal=True,
                               out_dtype=torch.float32)
    got = host(o)
    qh, kh, vh = host(q), host(k), host(v)
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 4095])
    for b, h in ((0, 5), (1, 31)):
        ref, _ = ofp8.attention_fp8_rows(qh, kh, vh, b, h, rows, True, 1.0 / math.sqrt(d), signs)
        assert_close(got[b, rows, h], ref, "bf16", f"fp8 full-size rows b={b} h={h}")



def test_fp8_long_context_bench_shape(m):
    """The long-context GQA prefill exactly as the benchmark times its FP8
    variant: B=2, L=8192, H_q=16, H_kv=4, d=128, causal, the workload's own
    inputs (0.1% of feature channels x20) and random signs; sampled rows of
    two (batch, head) pairs in different KV groups against the oracle."""
    import torch
    wl = W.WORKLOADS["long_kv4_causal"]
    say("prefill fp8 at the benchmark shape", wl.name)
    pin = W.prefill_inputs(wl)
    signs = W.random_signs(wl.seed, 6, wl.d)
    q, k, v = (dev(pin[n], "bf16") for n in ("q", "k", "v"))
    o = m.gqa_attn_prefill_fp8(q, k, v, signs=dev(signs, "f32"), causal=True, out_dtype=torch.float32)
    got = host(o)
    rows = np.array([0, 1, 63, 64, 65, 511, 1000, 4095, 4096, 6000, 8127, 8128, 8191])
    for b, h in ((0, 3), (1, 12)):
        ref, _ = ofp8.attention_fp8_rows(pin["q"], pin["k"], pin["v"], b, h, rows, True,
                                         1.0 / math.sqrt(wl.d), signs)
        assert_close(got[b, rows, h], ref, "bf16", f"fp8 bench-shape rows b={b} h={h}")

def test_fp8_scale_zero_gives_prefix_means(m):
    """scale = 0: every visible score is 0 whatever the FP8 codes, so each row's
    output is the mean of V over its visible keys (causal: a prefix mean)."""
    import torch
    B, L, H_q, H_kv, d = 1, 200, 4, 2, 128
    say("prefill fp8 scale 0", B, L, H_q, H_kv)
    q = W.round_bf16(W.normal(501, 1, (B, L, H_q, d)))
    k = W.round_bf16(W.normal(501, 2, (B, L, H_kv, d)))
    v = W.round_bf16(W.normal(501, 3, (B, L, H_kv, d)))
    o = m.gqa_attn_prefill_fp8(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"),
                               signs=dev(W.random_signs(501, 6, d), "f32"), causal=True, scale=0.0,
                               out_dtype=torch.float32)
    prefix = np.cumsum(v.astype(np.float64), axis=1) / np.arange(1, L + 1)[None, :, None, None]
    ref = np.repeat(prefix, H_q // H_kv, axis=2)
    assert_close(host(o), ref, "bf16", "fp8 scale 0 = prefix means")


def test_fp8_zero_rows_and_tiles(m):
    """All-zero Q rows and an all-zero 64-key K tile take the unit scale (no
    division by zero) and match the oracle."""
    import torch
    B, L, H_q, H_kv, d = 1, 256, 8, 2, 128
    say("prefill fp8 zero rows/tiles", B, L, H_q, H_kv)
    q = W.round_bf16(W.normal(502, 1, (B, L, H_q, d)))
    k = W.round_bf16(W.normal(502, 2, (B, L, H_kv, d)))
    v = W.round_bf16(W.normal(502, 3, (B, L, H_kv, d)))
    q[:, 10:20] = 0.0
    q[:, :, 3] = 0.0
    k[:, 64:128] = 0.0
    signs = W.random_signs(502, 6, d)
    for causal in (True, False):
        o, lse = m.gqa_attn_prefill_fp8(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), signs=dev(signs, "f32"),
                                        causal=causal, return_lse=True, out_dtype=torch.float32)
        ref, ref_lse = ofp8.attention_fp8(q, k, v, causal, 1.0 / math.sqrt(d), signs)
        assert_close(host(o), ref, "bf16", f"fp8 zero rows/tiles causal={causal}")
        assert_close(host(lse), ref_lse, "bf16", "fp8 zero rows/tiles LSE", max_abs=1e-3, rel_l2=1e-4)
