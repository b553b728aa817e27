"""Parity of the rotary embedding fused into the projection epilogues
(qkv_proj_rope, qkv_proj_append_rope) with the CPU oracle.

The cases reach every projection kernel: the 16-column streaming kernel, the
skinny kernel with its direct epilogue and with a k split (rotation in the
reduce kernel), the LDS-DMA tiles, the register-prefetched tiles and the fp32
kernel.  One fp32 case isolates the device's sine and cosine: with x holding
1 at every even component and W the identity per head, the rotated Q and K
columns are exactly cos and sin of each plane's angle."""
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


def _t(a, dtype="int32"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


ROPE = [  # M, hidden, H_q, H_kv, d, dtype, bias: the kernel each case reaches
    (7, 512, 8, 1, 128, "bf16", False),      # streaming, one 16-row block
    (24, 384, 4, 2, 64, "bf16", True),       # streaming, two 16-row blocks
    (33, 256, 4, 4, 64, "bf16", True),       # 8-wave workgroups over all of K, M just above 32
    (100, 1024, 8, 1, 128, "bf16", False),   # the same, 32-row tiles
    (100, 128, 8, 2, 64, "bf16", True),      # skinny, one k range (rotation in its own epilogue)
    (40, 640, 8, 2, 64, "bf16", False),      # skinny, k split (rotation in the reduce kernel)
    (32, 4096, 32, 8, 128, "bf16", True),    # register transpose + reduce at the Llama-2-7B decode width
    (17, 3072, 24, 8, 128, "bf16", True),    # the same, N = 5120, ragged M
    (97, 2048, 8, 2, 128, "bf16", True),     # 8-wave workgroups over all of K, ragged row tile
    (128, 2048, 32, 4, 64, "bf16", False),   # the same at the TinyLlama L=128 width
    (130, 384, 8, 2, 64, "bf16", False),     # LDS-DMA tiles
    (1029, 2048, 32, 4, 64, "bf16", True),   # LDS-DMA tiles, TinyLlama width, ragged M
    (4133, 256, 32, 4, 64, "bf16", True),    # more tiles than CUs: 128 x 128 tiles, ragged M
    (2100, 192, 16, 2, 128, "bf16", True),   # more tiles than CUs: 128 x 160 tiles two per CU, d = 128
    (2100, 128, 32, 8, 128, "bf16", True),   # the same with a ragged last column tile (N = 6144)
    (300, 64, 4, 2, 128, "bf16", True),      # LDS-DMA tiles, one k tile (hidden 64)
    (300, 264, 4, 2, 64, "bf16", False),     # register-prefetched tiles (hidden % 64 != 0)
    (128, 256, 4, 2, 64, "f32", True),       # fp32
    (45, 100, 2, 1, 128, "f32", False),      # fp32, ragged
]


def _inputs(M, hidden, H_q, H_kv, d, dtype, bias, seed):
    N = (H_q + 2 * H_kv) * d
    enc = W.round_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    x = enc(W.normal(seed, 1, (M, hidden)))
    w = enc(W.normal(seed, 2, (hidden, N), std=1.0 / math.sqrt(hidden)))
    b = enc(W.normal(seed, 3, (1, N))[0]) if bias else None
    return x, w, b


@pytest.mark.parametrize("M,hidden,H_q,H_kv,d,dtype,bias", ROPE)
def test_qkv_proj_rope_matches_oracle(m, M, hidden, H_q, H_kv, d, dtype, bias):
    say("qkv_proj_rope", M, hidden, H_q, H_kv, d, dtype, bias)
    x, w, b = _inputs(M, hidden, H_q, H_kv, d, dtype, bias, 700 + M)
    rng = np.random.default_rng(M)
    pos = rng.integers(0, 8192, size=M).astype(np.int32)
    pos[:3] = (0, 1, 100000)                       # identity row, first step, a long position
    th = W.rope_inv_freq(d)
    got = host(m.qkv_proj_rope(dev(x, dtype), dev(w, dtype), _t(pos), _t(th, "float32"), H_q, H_kv, d,
                               bias=dev(b, dtype) if bias else None))
    ref = oracle.qkv_proj_rope(x, w, pos, th, H_q, H_kv, d, b)
    assert_close(got, ref, dtype, f"qkv_proj_rope M={M}")
    # V columns: those of the plain projection, bit for bit
    plain = host(m.qkv_proj(dev(x, dtype), dev(w, dtype), H_q, H_kv, d, bias=dev(b, dtype) if bias else None))
    vcol = (H_q + H_kv) * d
    assert np.array_equal(got[:, vcol:], plain[:, vcol:])


def test_device_sin_cos_of_every_plane(m):
    """fp32 path, x = (1, 0, 1, 0, ...) and W = [I | I | I] per head: rotated
    column 2i is cos a_i and column 2i+1 is sin a_i exactly as the device
    computes them.  Angles up to 2^20 rad, both signs, random frequencies."""
    M, d = 4096, 64
    H_q = H_kv = 1
    x = np.zeros((M, d), np.float32)
    x[:, 0::2] = 1.0
    w = np.concatenate([np.eye(d, dtype=np.float32)] * 3, axis=1)
    rng = np.random.default_rng(5)
    pos = rng.integers(-(1 << 20), (1 << 20) + 1, size=M).astype(np.int32)
    pos[:8] = (0, 1, -1, 2, 3, 7, 1 << 20, -(1 << 20))
    th = rng.uniform(0.0, 1.0, d // 2).astype(np.float32)
    th[:2] = (1.0, 0.5)
    got = host(m.qkv_proj_rope(dev(x, "f32"), dev(w, "f32"), _t(pos), _t(th, "float32"), H_q, H_kv, d))
    a = oracle.rope_angles(pos, th)                   # [M, d/2] fp32 angles
    for blk in (0, d):                                # the Q head, then the K head
        err_c = np.abs(got[:, blk + 0:blk + d:2] - np.cos(a)).max()
        err_s = np.abs(got[:, blk + 1:blk + d:2] - np.sin(a)).max()
        say(f"device cos/sin, block {blk}: max-abs {err_c:.3e} / {err_s:.3e} (<= 1.5e-7)")
        assert err_c <= 1.5e-7 and err_s <= 1.5e-7
    assert np.array_equal(got[:, 2 * d:], x)          # V: not rotated
    assert np.array_equal(got[0, :d], x[0])           # position 0: identity


@pytest.mark.parametrize("M,hidden,d", [(8, 256, 64), (100, 1024, 128), (300, 512, 64)])
def test_zero_frequencies_give_qkv_proj(m, M, hidden, d):
    """theta = 0: cos 0 = 1 and sin 0 = 0 exactly, so every kernel returns the
    plain projection bit for bit."""
    H_q, H_kv = 4, 2
    x, w, b = _inputs(M, hidden, H_q, H_kv, d, "bf16", True, 900 + M)
    pos = np.arange(M, dtype=np.int32) * 37
    th = np.zeros(d // 2, np.float32)
    xd, wd, bd = dev(x, "bf16"), dev(w, "bf16"), dev(b, "bf16")
    a = m.qkv_proj_rope(xd, wd, _t(pos), _t(th, "float32"), H_q, H_kv, d, bias=bd)
    import torch
    assert torch.equal(a, m.qkv_proj(xd, wd, H_q, H_kv, d, bias=bd))


APPEND = [  # B, hidden, H_q, H_kv, d, L_max, dtype
    (8, 2048, 16, 1, 128, 40, "bf16"),    # the MQA decode shape: streaming kernel
    (32, 4096, 32, 8, 128, 50, "bf16"),   # Llama-2-7B GQA-8 decode: skinny + reduce
    (16, 1024, 64, 8, 128, 30, "bf16"),   # the same at N = 10240, half the rows
    (100, 128, 8, 2, 64, 20, "bf16"),     # skinny, one k range
    (64, 1024, 8, 2, 64, 20, "bf16"),     # 8-wave workgroups over all of K
    (300, 256, 8, 2, 64, 9, "bf16"),      # LDS-DMA tiles
    (2100, 256, 32, 4, 64, 9, "bf16"),    # LDS-DMA tiles, more tiles than CUs
    (200, 264, 4, 2, 64, 17, "bf16"),     # register-prefetched tiles
    (20, 128, 4, 2, 64, 12, "f32"),       # fp32
]


@pytest.mark.parametrize("B,hidden,H_q,H_kv,d,L_max,dtype", APPEND)
def test_qkv_proj_append_rope_matches_oracle(m, B, hidden, H_q, H_kv, d, L_max, dtype):
    """Rows are rotated at their own cache slot seq_lens[b] - 1 (clamped where
    not appended); the caches receive the rotated K and the plain V, with the
    bits of qkv's columns, and nothing else of them changes."""
    say("qkv_proj_append_rope", B, hidden, H_q, H_kv, d, L_max, dtype)
    x, w, _ = _inputs(B, hidden, H_q, H_kv, d, dtype, False, 950 + B)
    enc = W.round_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    kc0 = enc(W.normal(951, B, (B, L_max, H_kv, d)))
    vc0 = enc(W.normal(952, B, (B, L_max, H_kv, d)))
    rng = np.random.default_rng(B)
    lens = rng.integers(1, L_max + 1, size=B).astype(np.int32)
    lens[1], lens[-1] = 0, L_max + 3                  # rows that are not appended
    th = W.rope_inv_freq(d)
    kc, vc = dev(kc0, dtype), dev(vc0, dtype)
    qkv = m.qkv_proj_append_rope(dev(x, dtype), dev(w, dtype), kc, vc, _t(lens), _t(th, "float32"), H_q, H_kv, d)
    got = host(qkv)
    ref = oracle.qkv_proj_rope(x, w, oracle.append_positions(lens, L_max), th, H_q, H_kv, d)
    assert_close(got, ref, dtype, f"qkv_proj_append_rope B={B}")
    _, k_new, v_new = oracle.split_qkv(got[:, None, :], H_q, H_kv, d)
    kc_ref, vc_ref = oracle.kv_append(kc0, vc0, k_new[:, 0], v_new[:, 0], lens)
    assert np.array_equal(host(kc), kc_ref) and np.array_equal(host(vc), vc_ref)


def test_rope_decode_steps_match_prefill_rows(m):
    """Prefill of T tokens rotated at positions 0..T-1 (qkv_proj_rope, then causal
    attention), against decode steps that rotate, append and attend one token at
    a time (qkv_proj_append_rope, then decode): the appended keys are the
    prefill's rotated keys, and step s's output is within the bar of prefill
    row s."""
    import torch
    B, T, hidden, H_q, H_kv, d = 4, 40, 512, 8, 2, 64
    L_max = 48
    N = (H_q + 2 * H_kv) * d
    say("rope prefill vs decode steps", B, T, hidden, H_q, H_kv, d)
    xs = W.round_bf16(W.normal(61, 1, (B, T, hidden)))
    w = W.round_bf16(W.normal(62, 1, (hidden, N), std=1.0 / math.sqrt(hidden)))
    th = W.rope_inv_freq(d)
    wd, thd = dev(w, "bf16"), _t(th, "float32")
    scale = 1.0 / math.sqrt(d)
    qkv_p = m.qkv_proj_rope(dev(xs.reshape(B * T, hidden), "bf16"), wd, _t(W.prefill_positions(B, T)), thd,
                            H_q, H_kv, d).view(B, T, N)
    q, k, v = m.split_qkv(qkv_p, H_q, H_kv, d)
    o_p = host(m.gqa_attn_prefill(q, k, v, causal=True, scale=scale))
    ref = oracle.qkv_proj_rope(xs.reshape(B * T, hidden), w, W.prefill_positions(B, T), th, H_q, H_kv, d)
    assert_close(host(qkv_p).reshape(B * T, N), ref, "bf16", "prefill projection vs oracle")
    ref = ref.reshape(B, T, N)
    kc = torch.zeros(B, L_max, H_kv, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for s in range(T):
        lens = _t(np.full(B, s + 1, np.int32))
        qkv = m.qkv_proj_append_rope(dev(xs[:, s], "bf16"), wd, kc, vc, lens, thd, H_q, H_kv, d)
        assert_close(host(qkv), ref[:, s], "bf16", f"step {s} projection vs oracle row {s}")
        o = m.gqa_attn_decode(qkv[:, :H_q * d].unflatten(-1, (H_q, d)), kc, vc, lens, scale=scale)
        if s in (0, 1, T // 2, T - 1):
            assert_close(host(o), o_p[:, s], "bf16", f"decode step {s} vs prefill row")
    qo, ko, vo = oracle.split_qkv(ref.reshape(B, T, N), H_q, H_kv, d)
    O_ref, _ = oracle.attention(qo, ko, vo, True, scale)
    assert_close(o_p, O_ref, "bf16", "prefill attention vs oracle")
