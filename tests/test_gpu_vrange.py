"""V beyond the 16-bit operand range, and decode of empty sequences.

The bf16 prefill paths multiply P by V on fp16 matrix cores: each V tile is
converted as V * 2^-s with its own power-of-two exponent s (0 inside fp16's
range), and the accumulator follows with exact power-of-two rescales.  The
bf16 decode multiplies on bf16 matrix cores, where V needs no conversion.
Either way any finite bf16 V gives a finite, exact-to-rounding result:

* O is linear in V (the oracle's own pin), so scaling V by 2^e must scale the
  kernel's fp32 output by exactly 2^e and leave the LSE bit-identical: the same
  significands, the same sums, only the exponent moves.  Checked for e = 20
  (|v| up to ~4e6, beyond fp16's 65504) and e = -40 (tiny values that fp16
  would flush), on every entry point;
* V mixing magnitudes from 1e-12 to 3e30 within one head matches the fp64
  oracle within the bf16 bar scaled to the data's magnitude.  In the prefill
  one exponent serves a whole tile, so a value far below its tile's largest
  |v| is held to that largest value: each output row must be within 5e-3 (the bar's 2e-2
  at the O(4) magnitude of N(0,1) data) of the largest |v| in the V tiles the
  row reads -- for a prefill row the whole 64-key tiles up to its last
  visible key, masked keys of the diagonal tile included; for decode the
  sequence's keys (the tile loads stop at its length) -- and the whole output
  within rel-L2 5e-3.

A decode sequence with no keys gets O = 0 and LSE = -inf (the oracle's
reading, shared with the packed prefill's blind rows)."""
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


def _mixed(v, seed):
    """V [B, L, H, d] with some keys' rows huge, one key tiny, and the first key
    tile entirely far below fp16's normal range."""
    v = v.copy()
    rng = np.random.default_rng(seed)
    n = v.shape[1]
    for mag in (3e5, -7e5, 3e30, 1e-12):
        v[:, rng.integers(0, n)] *= mag
    v[:, : min(n, 64)] *= 1e-9
    return W.round_bf16(v)


def _lift(v):
    """|v| >= 2^-10 everywhere, so every value converts to fp16 exactly both at
    scale 1 (exponent 0) and under the tile exponent of a scaled tile: the
    bitwise scaling identity below then holds exactly."""
    return np.where(np.abs(v) < 2.0 ** -10, np.copysign(2.0 ** -10, v), v).astype(np.float32)


def _scaled_bits_equal(fn, v, what):
    import torch
    v = _lift(v)
    o0, l0 = fn(v)
    assert torch.isfinite(o0).all(), f"{what}: non-finite output at scale 1"
    for e in (20, -40):
        o1, l1 = fn(v * 2.0 ** e)
        ref = o0 * 2.0 ** e
        assert torch.isfinite(o1).all(), f"{what}: non-finite output at scale 2^{e}"
        assert torch.equal(o1, ref), f"{what}: O(V*2^{e}) != 2^{e} * O(V), max diff " \
                                     f"{(o1 - ref).abs().max().item():.3e}"
        assert torch.equal(l1, l0), f"{what}: LSE changed with V's scale"
        say(f"{what}: V*2^{e} scales O exactly")
    return o0


def _bar_scaled(got, ref, vis, what):
    """Each output row within 5e-3 * (the largest |v| that row sees), and the
    whole output within rel-L2 5e-3."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref) / vis[..., None]
    worst = float(err.max())
    say(f"{what}: max |O - ref| / (row's max|V|) = {worst:.3e} (<= 5e-3)")
    assert worst <= 5e-3, f"{what}: {worst:.3e}"
    assert_close(got, ref, "bf16", what, max_abs=np.inf)


def _vis_prefill(v, L_q, H_q, causal, tile=64):
    """[B, L_q, H_q]: the largest |v| over the key tiles each query row reads
    (whole tiles of `tile` keys from the sequence start, up to the tile of its
    last visible key)."""
    a = np.abs(v).max(axis=3)  # [B, L_kv, H_kv]
    B, L_kv, H_kv = a.shape
    if causal:
        cm = np.maximum.accumulate(a, axis=1)
        last = np.minimum(np.arange(L_q) + L_kv - L_q, L_kv - 1)
        vis = cm[:, np.minimum((last // tile + 1) * tile, L_kv) - 1]
    else:
        vis = np.broadcast_to(a.max(axis=1, keepdims=True), (B, L_q, H_kv))
    return np.repeat(vis, H_q // H_kv, axis=2)


def _vis_decode(v, lens, H_q):
    """[B, H_q]: the largest |v| over each sequence's keys."""
    a = np.abs(v).max(axis=3)  # [B, L_max, H_kv]
    vis = np.stack([a[b, :max(int(n), 1)].max(axis=0) for b, n in enumerate(lens)])
    return np.repeat(vis, H_q // v.shape[2], axis=1)


PREFILL = [  # B, L_q, L_kv, H_q, H_kv, d, causal
    (1, 200, 200, 8, 2, 128, True),
    (2, 130, 300, 4, 4, 64, False),
    (1, 257, 257, 16, 1, 64, True),
]


@pytest.mark.parametrize("B,L_q,L_kv,H_q,H_kv,d,causal", PREFILL)
def test_prefill_large_and_tiny_v(m, B, L_q, L_kv, H_q, H_kv, d, causal):
    import torch
    say("prefill V range", B, L_q, L_kv, H_q, H_kv, d, causal)
    q = W.round_bf16(W.normal(301, 1, (B, L_q, H_q, d)))
    k = W.round_bf16(W.normal(301, 2, (B, L_kv, H_kv, d)))
    v = W.round_bf16(W.normal(301, 3, (B, L_kv, H_kv, d)))
    qd, kd = dev(q, "bf16"), dev(k, "bf16")
    scale = 1.0 / math.sqrt(d)

    def run(vv):
        return m.gqa_attn_prefill(qd, kd, dev(vv, "bf16"), causal=causal, scale=scale, return_lse=True,
                                  out_dtype=torch.float32)
    v = _lift(v)
    o0 = _scaled_bits_equal(run, v, f"prefill d={d}")
    ref, _ = oracle.attention(q, k, v, causal, scale)
    assert_close(host(o0), ref, "bf16", "prefill O at scale 1")
    vm = _mixed(v, 302)
    om, _ = run(vm)
    refm, _ = oracle.attention(q, k, vm, causal, scale)
    _bar_scaled(host(om), refm, _vis_prefill(vm, L_q, H_q, causal), "prefill mixed magnitudes")


def test_varlen_and_fp8_large_and_tiny_v(m):
    import torch
    H_q, H_kv, d = 8, 2, 128
    lens = [150, 1, 77]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tot = int(cu[-1])
    say("varlen / fp8 V range", lens)
    q = W.round_bf16(W.normal(311, 1, (tot, H_q, d)))
    k = W.round_bf16(W.normal(311, 2, (tot, H_kv, d)))
    v = W.round_bf16(W.normal(311, 3, (tot, H_kv, d)))
    cud = torch.from_numpy(cu).cuda()
    qd, kd = dev(q, "bf16"), dev(k, "bf16")

    def run_varlen(vv):
        return m.gqa_attn_prefill_varlen(qd, kd, dev(vv, "bf16"), cud, cud, max(lens), max(lens), causal=True,
                                         return_lse=True, out_dtype=torch.float32)
    v = _lift(v)
    o0 = _scaled_bits_equal(run_varlen, v, "varlen")
    ref, _ = oracle.attention_varlen(q, k, v, cu, cu, True, 1.0 / math.sqrt(d))
    assert_close(host(o0), ref, "bf16", "varlen O at scale 1")
    vm = _mixed(v[None], 312)[0]
    om, _ = run_varlen(vm)
    refm, _ = oracle.attention_varlen(q, k, vm, cu, cu, True, 1.0 / math.sqrt(d))
    vis = np.concatenate([_vis_prefill(vm[None, cu[b]:cu[b + 1]], lens[b], H_q, True)[0]
                          for b in range(len(lens))])
    _bar_scaled(host(om), refm, vis, "varlen mixed magnitudes")

    B, L = 1, 200
    q8 = dev(W.round_bf16(W.normal(313, 1, (B, L, H_q, d))), "bf16")
    k8 = dev(W.round_bf16(W.normal(313, 2, (B, L, H_kv, d))), "bf16")
    v8 = W.round_bf16(W.normal(313, 3, (B, L, H_kv, d)))
    signs = dev(W.random_signs(313, 6, d), "f32")

    def run_fp8(vv):
        return m.gqa_attn_prefill_fp8(q8, k8, dev(vv, "bf16"), signs=signs, causal=True, return_lse=True,
                                      out_dtype=torch.float32)
    _scaled_bits_equal(run_fp8, v8, "prefill fp8")


DECODE = [  # B, H_q, H_kv, d, L_max, kv_split (0: the library's choice)
    (3, 8, 2, 128, 300, 32),
    (4, 4, 4, 64, 200, 0),
    (64, 16, 8, 128, 1024, 0),   # balanced work split (>= 16384 tiles at capacity)
]


@pytest.mark.parametrize("B,H_q,H_kv,d,L_max,split", DECODE)
def test_decode_large_and_tiny_v(m, B, H_q, H_kv, d, L_max, split):
    import torch
    say("decode V range", B, H_q, H_kv, d, L_max, split)
    rng = np.random.default_rng(321 + B)
    kc = W.round_bf16(W.normal(321, 1, (B, L_max, H_kv, d)))
    vc = W.round_bf16(W.normal(321, 2, (B, L_max, H_kv, d)))
    q = W.round_bf16(W.normal(321, 3, (B, H_q, d)))
    lens = rng.integers(1, L_max + 1, size=B).astype(np.int32)
    lens[0] = L_max
    lens_d = torch.from_numpy(lens).cuda()
    qd, kd = dev(q, "bf16"), dev(kc, "bf16")
    scale = 1.0 / math.sqrt(d)

    def run(vv):
        return m.gqa_attn_decode(qd, kd, dev(vv, "bf16"), lens_d, scale=scale, kv_split=split, return_lse=True,
                                 out_dtype=torch.float32)
    vc = _lift(vc)
    o0 = _scaled_bits_equal(run, vc, "decode")
    ref, _ = oracle.decode(q, kc, vc, lens, scale)
    assert_close(host(o0), ref, "bf16", "decode O at scale 1")
    vm = _mixed(vc, 322)
    om, _ = run(vm)
    refm, _ = oracle.decode(q, kc, vm, lens, scale)
    _bar_scaled(host(om), refm, _vis_decode(vm, lens, H_q), "decode mixed magnitudes")
    if B <= 8:  # the same rows in a paged pool give the same bits
        P = 16 if L_max % 16 == 0 else None
        if P is not None:
            pps = L_max // P
            table = np.arange(B * pps, dtype=np.int32).reshape(B, pps)[:, ::-1].copy()
            kp = np.zeros((B * pps, P, H_kv, d), np.float32)
            vp = np.zeros_like(kp)
            for b in range(B):
                for i in range(pps):
                    kp[table[b, i]] = kc[b, i * P:(i + 1) * P]
                    vp[table[b, i]] = vm[b, i * P:(i + 1) * P]
            op = m.gqa_attn_decode_paged(qd, dev(kp, "bf16"), dev(vp, "bf16"), torch.from_numpy(table).cuda(),
                                         lens_d, scale=scale, kv_split=split, out_dtype=torch.float32)
            assert torch.equal(op, om), "paged decode must give the contiguous decode's bits"


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("big", [False, True])
def test_decode_empty_sequences(m, split, big):
    """seq_lens[b] = 0: O = 0 and LSE = -inf; the other sequences are unaffected
    (contiguous and paged caches, fixed and balanced splits, bf16 and fp32)."""
    import torch
    B, H_q, H_kv, d, L_max = (64, 16, 8, 128, 1024) if big else (5, 8, 2, 64, 96)
    say("decode empty sequences", B, H_q, H_kv, d, L_max, split)
    rng = np.random.default_rng(331 + B)
    lens = rng.integers(1, L_max + 1, size=B).astype(np.int32)
    lens[[1, B - 1]] = 0
    lens[0] = L_max
    for dtype in (("bf16",) if big else ("bf16", "f32")):
        enc = W.round_bf16 if dtype == "bf16" else (lambda a: a)
        kc = enc(W.normal(331, 1, (B, L_max, H_kv, d)))
        vc = enc(W.normal(331, 2, (B, L_max, H_kv, d)))
        q = enc(W.normal(331, 3, (B, H_q, d)))
        lens_d = torch.from_numpy(lens).cuda()
        ws = m.decode_workspace(B, H_q, H_kv, d, L_max, split)
        ws.fill_(0xFF)  # stale partials would show as NaN
        o, lse = m.gqa_attn_decode(dev(q, dtype), dev(kc, dtype), dev(vc, dtype), lens_d, kv_split=split,
                                   return_lse=True, out_dtype=torch.float32, workspace=ws)
        ref, ref_l = oracle.decode(q, kc, vc, lens, 1.0 / math.sqrt(d))
        got, got_l = host(o), host(lse)
        assert np.array_equal(got[lens == 0], np.zeros_like(got[lens == 0])), "empty sequence: O must be 0"
        assert np.all(got_l[lens == 0] == -np.inf), "empty sequence: LSE must be -inf"
        keep = lens > 0
        assert_close(got[keep], ref[keep], dtype, f"decode {dtype} around empty sequences")
        assert_close(got_l[keep], ref_l[keep], dtype, "LSE", max_abs=1e-3 if dtype == "bf16" else 1e-4)
        if dtype == "bf16" and not big:
            P = 16
            pps = L_max // P
            table = np.arange(B * pps, dtype=np.int32).reshape(B, pps)
            op = m.gqa_attn_decode_paged(dev(q, dtype), dev(kc.reshape(B * pps, P, H_kv, d), dtype),
                                         dev(vc.reshape(B * pps, P, H_kv, d), dtype),
                                         torch.from_numpy(table).cuda(), lens_d, kv_split=split,
                                         out_dtype=torch.float32)
            assert torch.equal(op, o), "paged decode with empty sequences must give the contiguous bits"
