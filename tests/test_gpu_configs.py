"""Parity at the full workload sizes (sampled rows where the oracle would be slow)
and the invariants the pages fix, checked on the GPU path.

Stage-wise: the projection against the oracle's fp64 product of the same x, W;
attention against the oracle fed the GPU's own Q/K/V.  End-to-end (x -> O) is
also gated for the tiny fp32 layer and the TinyLlama-shaped prefill."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_close, dev, errors, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mqa_qkv_proj_amd
    return mqa_qkv_proj_amd


def T():
    import torch
    return torch


# ----------------------------------------------------------------------------- tiny fp32 layer

def test_tiny_fp32_layer_end_to_end(m):
    wl = W.WORKLOADS["tiny_f32"]
    say("tiny_f32 end-to-end")
    pj = W.proj_inputs(wl)
    qkv = m.qkv_proj(dev(pj["x"], "f32").view(wl.B, wl.L, wl.hidden), dev(pj["w"], "f32"), wl.H_q, wl.H_kv, wl.d)
    q, k, v = m.split_qkv(qkv, wl.H_q, wl.H_kv, wl.d)
    o, lse = m.gqa_attn_prefill(q, k, v, causal=True, return_lse=True)
    ref_qkv = oracle.qkv_proj(pj["x"], pj["w"]).reshape(wl.B, wl.L, -1)
    assert_close(host(qkv), ref_qkv, "f32", "tiny qkv")
    rq, rk, rv = oracle.split_qkv(ref_qkv, wl.H_q, wl.H_kv, wl.d)
    ro, rl = oracle.attention(rq, rk, rv, True, 1.0 / math.sqrt(wl.d))
    assert_close(host(o), ro, "f32", "tiny O end-to-end")
    assert_close(host(lse), rl, "f32", "tiny LSE end-to-end")


# ----------------------------------------------------------------------------- TinyLlama prefill

@pytest.mark.parametrize("L", [128, 512, 2048])
def test_tinyllama_prefill_layer(m, L):
    wl = W.WORKLOADS[f"tinyllama_L{L}"]
    say("tinyllama prefill", L)
    pj = W.proj_inputs(wl)
    qkv = m.qkv_proj(dev(pj["x"], "bf16").view(wl.B, wl.L, wl.hidden), dev(pj["w"], "bf16"), wl.H_q, wl.H_kv, wl.d)
    ref_qkv = oracle.qkv_proj(pj["x"], pj["w"]).reshape(wl.B, wl.L, -1)
    assert_close(host(qkv), ref_qkv, "bf16", f"L={L} qkv_proj")
    q, k, v = m.split_qkv(qkv, wl.H_q, wl.H_kv, wl.d)  # zero-copy views
    o = m.gqa_attn_prefill(q, k, v, causal=True)
    gq, gk, gv = oracle.split_qkv(host(qkv), wl.H_q, wl.H_kv, wl.d)
    scale = 1.0 / math.sqrt(wl.d)
    ro, _ = oracle.attention(gq, gk, gv, True, scale)
    assert_close(host(o), ro, "bf16", f"L={L} attention (stage-wise)")
    rq, rk, rv = oracle.split_qkv(ref_qkv, wl.H_q, wl.H_kv, wl.d)
    re2e, _ = oracle.attention(rq, rk, rv, True, scale)
    assert_close(host(o), re2e, "bf16", f"L={L} x -> O end-to-end")


# ----------------------------------------------------------------------------- MQA decode

@pytest.mark.parametrize("step", [0, 511, 1023])
def test_mqa_decode_steps(m, step):
    t = T()
    wl = W.WORKLOADS["mqa_decode"]
    say("mqa decode step", step)
    din = W.decode_inputs(wl)
    q = W.decode_step_q(wl, step)
    lens = W.decode_lengths(wl, step)
    o, lse = m.gqa_attn_decode(dev(q, "bf16"), dev(din["k_cache"], "bf16"), dev(din["v_cache"], "bf16"),
                               t.from_numpy(lens).cuda(), return_lse=True)
    ro, rl = oracle.decode(q, din["k_cache"], din["v_cache"], lens, 1.0 / math.sqrt(wl.d))
    assert_close(host(o), ro, "bf16", f"mqa step {step} O")
    assert_close(host(lse), rl, "bf16", f"mqa step {step} LSE", max_abs=1e-3, rel_l2=1e-4)


def test_mqa_decode_chained_on_projection(m):
    """qkv_proj of the 8 new tokens -> q as a strided view of the packed rows -> decode."""
    t = T()
    wl = W.WORKLOADS["mqa_decode"]
    pj = W.proj_inputs(wl, step=3)
    qkv = m.qkv_proj(dev(pj["x"], "bf16"), dev(pj["w"], "bf16"), wl.H_q, wl.H_kv, wl.d)
    assert_close(host(qkv), oracle.qkv_proj(pj["x"], pj["w"]), "bf16", "mqa qkv_proj")
    din = W.decode_inputs(wl)
    lens = W.decode_lengths(wl, 3)
    qv = qkv[:, :wl.H_q * wl.d].unflatten(-1, (wl.H_q, wl.d))
    o = m.gqa_attn_decode(qv, dev(din["k_cache"], "bf16"), dev(din["v_cache"], "bf16"), t.from_numpy(lens).cuda())
    gq = host(qkv)[:, :wl.H_q * wl.d].reshape(wl.B, wl.H_q, wl.d)
    ro, _ = oracle.decode(gq, din["k_cache"], din["v_cache"], lens, 1.0 / math.sqrt(wl.d))
    assert_close(host(o), ro, "bf16", "mqa chained decode")


# ----------------------------------------------------------------------------- Llama-2-7B decode sweep

@pytest.mark.parametrize("hkv", [32, 8, 4])
def test_llama7b_decode(m, hkv):
    t = T()
    wl = W.WORKLOADS[f"llama7b_decode_kv{hkv}"]
    say("llama7b decode", hkv)
    din = W.decode_inputs(wl)
    lens = din["seq_lens"]
    kc, vc = dev(din["k_cache"], "bf16"), dev(din["v_cache"], "bf16")
    o, lse = m.gqa_attn_decode(dev(din["q"], "bf16"), kc, vc, t.from_numpy(lens).cuda(), return_lse=True)
    ro, rl = oracle.decode(din["q"], din["k_cache"], din["v_cache"], lens, 1.0 / math.sqrt(wl.d))
    assert_close(host(o), ro, "bf16", f"kv{hkv} O")
    assert_close(host(lse), rl, "bf16", f"kv{hkv} LSE", max_abs=1e-3, rel_l2=1e-4)
    pj = W.proj_inputs(wl)
    qkv = m.qkv_proj(dev(pj["x"], "bf16"), dev(pj["w"], "bf16"), wl.H_q, wl.H_kv, wl.d)
    assert_close(host(qkv), oracle.qkv_proj(pj["x"], pj["w"]), "bf16", f"kv{hkv} qkv_proj")


# ----------------------------------------------------------------------------- long-context prefill

SAMPLE_FIXED = [0, 1, 2, 3, 31, 32, 63, 64, 65, 127, 128, 255, 256, 1000, 4095, 4096, 8063, 8190, 8191]


@pytest.mark.parametrize("name", ["long_kv16_causal", "long_kv16_full", "long_kv4_causal", "long_kv4_full"])
def test_long_context_prefill_sampled(m, name):
    t = T()
    wl = W.WORKLOADS[name]
    say("long prefill", name)
    pin = W.prefill_inputs(wl)
    q, k, v = (dev(pin[n], "bf16") for n in ("q", "k", "v"))
    o32, lse = m.gqa_attn_prefill(q, k, v, causal=wl.causal, return_lse=True, out_dtype=t.float32)
    o16 = m.gqa_attn_prefill(q, k, v, causal=wl.causal)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([SAMPLE_FIXED, rng.integers(0, wl.L, 24)]))
    scale = 1.0 / math.sqrt(wl.d)
    got32, got16, gotl, ref, refl = [], [], [], [], []
    o32h, o16h, lseh = host(o32), host(o16), host(lse)
    for b in range(wl.B):
        for h in range(wl.H_q):
            ro, rl = oracle.attention_rows(pin["q"], pin["k"], pin["v"], b, h, rows, wl.causal, scale)
            ref.append(ro); refl.append(rl)
            got32.append(o32h[b, rows, h]); got16.append(o16h[b, rows, h]); gotl.append(lseh[b, h, rows])
    ref, got32, got16 = np.concatenate(ref), np.concatenate(got32), np.concatenate(got16)
    assert_close(got32, ref, "bf16", f"{name} O (fp32 output, gated)")
    assert_close(np.concatenate(gotl), np.concatenate(refl), "bf16", f"{name} LSE", max_abs=2e-3, rel_l2=1e-4)
    ma, rl16 = errors(got16, ref)
    say(f"{name} O bf16 output: max-abs {ma:.3e} (bf16 half-ulp at |O|~60 is 0.125), rel-L2 {rl16:.3e}")
    assert rl16 <= 5e-3
    # every row of two (batch, head) pairs: the first head of the first
    # sequence and the last head of the last (the other KV group)
    for b, h in ((0, 0), (wl.B - 1, wl.H_q - 1)):
        ro, rl = [], []
        for r0 in range(0, wl.L, 1024):
            o_blk, l_blk = oracle.attention_rows(pin["q"], pin["k"], pin["v"], b, h, np.arange(r0, r0 + 1024),
                                                 wl.causal, scale)
            ro.append(o_blk); rl.append(l_blk)
        assert_close(o32h[b, :, h], np.concatenate(ro), "bf16", f"{name} O, all {wl.L} rows of b={b} h={h}")
        assert_close(lseh[b, h], np.concatenate(rl), "bf16", f"{name} LSE, all rows of b={b} h={h}",
                     max_abs=2e-3, rel_l2=1e-4)


# ----------------------------------------------------------------------------- invariants

def _small_prefill(seed, B=1, L=300, H_q=8, H_kv=2, d=128):
    inp = W.small("bf16", seed, B, L, L, H_q, H_kv, d)
    return inp, [dev(inp[n], "bf16") for n in ("q", "k", "v")]


def test_prefill_and_decode_are_deterministic(m):
    t = T()
    inp, (q, k, v) = _small_prefill(41)
    a = m.gqa_attn_prefill(q, k, v, causal=True, out_dtype=t.float32)
    b = m.gqa_attn_prefill(q, k, v, causal=True, out_dtype=t.float32)
    assert t.equal(a, b)
    kc, vc = k.contiguous(), v.contiguous()
    lens = t.tensor([300], dtype=t.int32, device="cuda")
    d1 = m.gqa_attn_decode(q[:, -1], kc, vc, lens, out_dtype=t.float32, kv_split=64)
    d2 = m.gqa_attn_decode(q[:, -1], kc, vc, lens, out_dtype=t.float32, kv_split=64)
    assert t.equal(d1, d2)


def test_causal_rows_ignore_future_keys_bitwise(m):
    t = T()
    inp, (q, k, v) = _small_prefill(42)
    o = m.gqa_attn_prefill(q, k, v, causal=True, out_dtype=t.float32)
    i0 = 150
    k2, v2 = k.clone(), v.clone()
    k2[:, i0 + 1:] = 30.0
    v2[:, i0 + 1:] = -7.0
    o2 = m.gqa_attn_prefill(q, k2, v2, causal=True, out_dtype=t.float32)
    assert t.equal(o[:, :i0 + 1], o2[:, :i0 + 1])
    assert not t.equal(o[:, i0 + 1:], o2[:, i0 + 1:])


def test_first_row_and_single_key_return_v0_bitwise(m):
    t = T()
    inp, (q, k, v) = _small_prefill(43)
    o = m.gqa_attn_prefill(q, k, v, causal=True, out_dtype=t.float32)
    G = 8 // 2
    # V enters the PV product as fp16 (exact in fp16's normal range, rounded below it)
    v0 = v[0, 0].to(t.float16).float()
    for h in range(8):
        assert t.equal(o[0, 0, h], v0[h // G])
    # the decode multiplies on bf16 matrix cores, where V is an exact operand:
    # one key gives P = 1 (P_hi = 1, P_lo = 0) and O = V itself
    lens = t.tensor([1], dtype=t.int32, device="cuda")
    od = m.gqa_attn_decode(q[:, 5], k.contiguous(), v.contiguous(), lens, out_dtype=t.float32)
    for h in range(8):
        assert t.equal(od[0, h], v[0, 0, h // G].float())


def test_decode_equals_prefill_last_row_and_is_split_independent(m):
    t = T()
    inp, (q, k, v) = _small_prefill(44, B=2, L=257)
    kc, vc = k.contiguous(), v.contiguous()
    lens = t.tensor([257, 257], dtype=t.int32, device="cuda")
    outs = [host(m.gqa_attn_decode(q[:, -1].contiguous(), kc, vc, lens, out_dtype=t.float32, kv_split=sp))
            for sp in (0, 32, 64, 96, 256, 1024)]
    for o in outs[1:]:
        assert_close(o, outs[0], "bf16", "split independence", max_abs=1e-3, rel_l2=1e-3)
    pre = m.gqa_attn_prefill(q[:, -1:].contiguous(), k, v, causal=True, out_dtype=t.float32)
    assert_close(host(pre[:, 0]), outs[0], "bf16", "decode vs prefill last row", max_abs=1e-3, rel_l2=1e-3)


def test_head_mapping_closed_form_on_gpu(m):
    t = T()
    B, L, H_q, H_kv, d = 1, 200, 8, 4, 64
    inp = W.small("bf16", 45, B, L, L, H_q, H_kv, d)
    v = np.zeros((B, L, H_kv, d), np.float32)
    for g in range(H_kv):
        v[:, :, g] = g + 1
    o = host(m.gqa_attn_prefill(dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(v, "bf16"), causal=True,
                                out_dtype=t.float32))
    for h in range(H_q):
        np.testing.assert_allclose(o[:, :, h], h // (H_q // H_kv) + 1, rtol=0, atol=2e-5)


def test_gqa_equals_mha_on_repeated_kv_gpu(m):
    t = T()
    inp, (q, k, v) = _small_prefill(46, L=200)
    o = host(m.gqa_attn_prefill(q, k, v, causal=True, out_dtype=t.float32))
    kr, vr = k.repeat_interleave(4, dim=2).contiguous(), v.repeat_interleave(4, dim=2).contiguous()
    o2 = host(m.gqa_attn_prefill(q, kr, vr, causal=True, out_dtype=t.float32))
    assert_close(o, o2, "bf16", "GQA vs MHA on repeated KV", max_abs=1e-3, rel_l2=1e-4)


def test_lse_normalises_softmax_rows(m):
    t = T()
    inp, (q, k, v) = _small_prefill(47, L=180)
    _, lse = m.gqa_attn_prefill(q, k, v, causal=True, return_lse=True)
    lse = host(lse)
    scale = 1.0 / math.sqrt(128)
    for h in (0, 5):
        g = h // 4
        S = scale * (inp["q"][0, :, h].astype(np.float64) @ inp["k"][0, :, g].astype(np.float64).T)
        S = np.where(np.tril(np.ones_like(S, dtype=bool)), S, -np.inf)
        sums = np.exp(S - lse[0, h][:, None]).sum(axis=1)
        np.testing.assert_allclose(sums, 1.0, rtol=0, atol=1e-3)
