"""Prefill over a packed batch of variable-length sequences: parity with the
oracle, agreement with one gqa_attn_prefill call per sequence, the LSE
layout, and the blind rows (no key visible) giving O = 0, LSE = -inf."""
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


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


# H_q, H_kv, d, causal, L_q lengths, L_kv lengths (None: the same)
VARLEN = [
    (8, 2, 128, True, [300, 1, 64, 129, 700], None),
    (8, 2, 128, False, [200, 77, 513], [90, 300, 513]),
    (32, 4, 64, True, [1, 255, 256, 257, 1000], None),
    (4, 4, 64, True, [40, 100], [90, 100]),           # L_q < L_kv, bottom-right alignment
    (16, 1, 128, False, [65, 3], None),
]


@pytest.mark.parametrize("H_q,H_kv,d,causal,lq,lk", VARLEN)
def test_varlen_matches_oracle_and_per_sequence_calls(m, H_q, H_kv, d, causal, lq, lk):
    import torch
    lk = lq if lk is None else lk
    say("prefill varlen", H_q, H_kv, d, causal, lq, lk)
    cq, ck = _cu(lq), _cu(lk)
    tq, tk = int(cq[-1]), int(ck[-1])
    q = W.round_bf16(W.normal(91, 1, (tq, H_q, d)))
    k = W.round_bf16(W.normal(92, 1, (tk, H_kv, d)))
    v = W.round_bf16(W.normal(93, 1, (tk, H_kv, d)))
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    scale = 1.0 / math.sqrt(d)
    o, lse = m.gqa_attn_prefill_varlen(qd, kd, vd, torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(),
                                       max(lq), max(lk), causal=causal, scale=scale, return_lse=True,
                                       out_dtype=torch.float32)
    ref, ref_lse = oracle.attention_varlen(q, k, v, cq, ck, causal, scale)
    assert_close(host(o), ref, "bf16", "varlen O (fp32 out)")
    # LSE bar as for the fixed-length call: the row sums come from fp16-rounded P
    assert_close(host(lse), ref_lse, "bf16", "varlen LSE", max_abs=1e-3, rel_l2=1e-4)
    # one fixed-length call per sequence: the same result.  The packed grid and
    # a lone short sequence may pick different workgroup shapes (a small d=64
    # grid splits each row block's keys between two waves), which sum in a
    # different order, so the comparison is at the oracle's bar.
    for b in range(len(lq)):
        if lq[b] == 0:
            continue
        ob, lb = m.gqa_attn_prefill(qd[None, cq[b]:cq[b + 1]], kd[None, ck[b]:ck[b + 1]], vd[None, ck[b]:ck[b + 1]],
                                    causal=causal, scale=scale, return_lse=True, out_dtype=torch.float32)
        assert_close(host(ob[0]), host(o[cq[b]:cq[b + 1]]), "bf16", f"sequence {b}: its own call vs the batch")
        assert np.abs(host(lb[0]) - host(lse[:, cq[b]:cq[b + 1]])).max() < 1e-3, f"sequence {b}: LSE"


def test_varlen_blind_rows_and_empty_sequences(m):
    """Sequences with no keys, no queries, or (causal) more queries than keys."""
    import torch
    H_q, H_kv, d = 4, 2, 64
    lq, lk = [5, 0, 70, 3], [0, 4, 10, 3]
    cq, ck = _cu(lq), _cu(lk)
    tq, tk = int(cq[-1]), int(ck[-1])
    q = W.round_bf16(W.normal(94, 1, (tq, H_q, d)))
    k = W.round_bf16(W.normal(95, 1, (tk, H_kv, d)))
    v = W.round_bf16(W.normal(96, 1, (tk, H_kv, d)))
    for causal in (False, True):
        o, lse = m.gqa_attn_prefill_varlen(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"),
                                           torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), max(lq), max(lk),
                                           causal=causal, scale=0.3, return_lse=True, out_dtype=torch.float32)
        ref, ref_lse = oracle.attention_varlen(q, k, v, cq, ck, causal, 0.3)
        got = host(o)
        assert np.isfinite(got).all()
        assert_close(got, ref, "bf16", f"blind rows causal={causal}")
        gl = host(lse)
        assert np.array_equal(np.isinf(gl), np.isinf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert_close(gl[fin], ref_lse[fin], "bf16", "blind rows LSE", max_abs=1e-3, rel_l2=1e-4)


def test_varlen_bf16_output_on_qkv_views(m):
    """The packed layout consumed in place from projected qkv rows (token stride N)."""
    import torch
    H_q, H_kv, d = 8, 2, 64
    N = (H_q + 2 * H_kv) * d
    lens = [17, 300, 64]
    cu = _cu(lens)
    qkv = dev(W.round_bf16(W.normal(97, 1, (int(cu[-1]), N))), "bf16")
    q = qkv[:, :H_q * d].unflatten(-1, (H_q, d))
    k = qkv[:, H_q * d:(H_q + H_kv) * d].unflatten(-1, (H_kv, d))
    v = qkv[:, (H_q + H_kv) * d:].unflatten(-1, (H_kv, d))
    cu_d = torch.from_numpy(cu).cuda()
    o = m.gqa_attn_prefill_varlen(q, k, v, cu_d, cu_d, max(lens), max(lens), causal=True)
    ref, _ = oracle.attention_varlen(host(q), host(k), host(v), cu, cu, True, 1.0 / math.sqrt(d))
    assert_close(host(o), ref, "bf16", "varlen on qkv views")
