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


# H_q, H_kv, d, causal, L_q lengths, L_kv lengths (None: the same), seed
SCHEDULED = [
    # 300 sequences (some empty): the planning scans run over more sequences than threads, and the
    # list holds more row blocks than there are persistent workers, so each worker claims several
    (8, 2, 128, True, "many", None, 101),
    (8, 2, 128, False, [200, 77, 0, 513, 64], [90, 300, 5, 513, 1], 102),
    # the TinyLlama-shaped batch: 8 sequences of 128..2048 tokens, four KV heads of 8 query heads
    (32, 4, 64, True, "tinyllama8", None, 103),
    # a long and a short causal sequence
    (32, 4, 64, True, [2048, 1000], None, 104),
    # d = 64, not causal, key lengths unlike the query lengths (one sequence without keys)
    (16, 2, 64, False, [700, 33, 129, 0, 257], [64, 900, 129, 5, 0], 108),
]


def _lengths(spec, seed):
    rng = np.random.default_rng(seed)
    if spec == "many":
        lens = rng.integers(0, 300, size=300, endpoint=True)
        lens[[0, 17, 299]] = 0
        return lens.tolist()
    if spec == "tinyllama8":
        return rng.integers(128, 2048, size=8, endpoint=True).tolist()
    return spec


@pytest.mark.parametrize("H_q,H_kv,d,causal,lq,lk,seed", SCHEDULED)
def test_varlen_schedule_matches_grid_path_and_oracle(m, H_q, H_kv, d, causal, lq, lk, seed):
    """The persistent heaviest-first workers (workspace with a schedule) against
    the grid of one workgroup per row block (workspace of V images only): the
    same per-row arithmetic, so bit-identical outputs and LSE; sampled
    sequences against the oracle."""
    import torch
    lq = _lengths(lq, seed)
    lk = lq if lk is None else lk
    say("prefill varlen schedule", H_q, H_kv, d, causal, len(lq), "sequences", sum(lq), "queries")
    cq, ck = _cu(lq), _cu(lk)
    tq, tk = int(cq[-1]), int(ck[-1])
    q = W.round_bf16(W.normal(seed, 1, (tq, H_q, d)))
    k = W.round_bf16(W.normal(seed, 2, (tk, H_kv, d)))
    v = W.round_bf16(W.normal(seed, 3, (tk, H_kv, d)))
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    scale = 1.0 / math.sqrt(d)
    B = len(lq)
    need = m.prefill_varlen_workspace_bytes(B, max(lk), tq, H_q, H_kv, d)
    assert need > m.prefill_workspace_bytes(B, max(lk), H_kv, d)
    # stale bytes everywhere, the schedule's header included: the plan rewrites all it reads
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    kw = dict(causal=causal, scale=scale, return_lse=True, out_dtype=torch.float32)
    o_s, l_s = m.gqa_attn_prefill_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), workspace=ws, **kw)
    o_s2, l_s2 = m.gqa_attn_prefill_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), workspace=ws, **kw)
    o_g, l_g = m.gqa_attn_prefill_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), schedule=False, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_s2) and torch.equal(l_s, l_s2), "a second call on the same workspace differs"
    assert torch.equal(o_s, o_g), "scheduled and grid outputs differ"
    assert torch.equal(l_s, l_g), "scheduled and grid LSE differ"
    # oracle on the longest sequence and a few others
    order = np.argsort(lq)[::-1]
    pick = [int(b) for b in order[:2]] + [int(b) for b in np.random.default_rng(seed).choice(B, min(B, 3), False)]
    got, gl = host(o_s), host(l_s)
    for b in sorted(set(pick)):
        if lq[b] == 0:
            continue
        sl_q, sl_k = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        ref, ref_lse = oracle.attention_varlen(q[sl_q], k[sl_k], v[sl_k], _cu([lq[b]]), _cu([lk[b]]), causal, scale)
        assert_close(got[sl_q], ref, "bf16", f"scheduled sequence {b} ({lq[b]} x {lk[b]})")
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isinf(gl[:, sl_q]), ~fin)
        assert_close(gl[:, sl_q][fin], ref_lse[fin], "bf16", f"scheduled sequence {b} LSE", max_abs=1e-3, rel_l2=1e-4)


@pytest.mark.parametrize("B,L", [(1, 2048), (2, 1024)])
def test_varlen_equal_lengths_equal_fixed_length_call(m, B, L):
    """Packed sequences all at the maximum length (TinyLlama-shaped heads) take
    the grid even with a schedule-sized workspace, and equal the fixed-length
    call on the same rows bit for bit."""
    import torch
    H_q, H_kv, d = 32, 4, 64
    say("prefill varlen equal lengths vs fixed length", B, L, H_q, H_kv, d)
    q = dev(W.round_bf16(W.normal(105, 1, (B * L, H_q, d))), "bf16")
    k = dev(W.round_bf16(W.normal(105, 2, (B * L, H_kv, d))), "bf16")
    v = dev(W.round_bf16(W.normal(105, 3, (B * L, H_kv, d))), "bf16")
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device="cuda")
    o_p, l_p = m.gqa_attn_prefill_varlen(q, k, v, cu, cu, L, L, causal=True, return_lse=True)
    o_f, l_f = m.gqa_attn_prefill(q.view(B, L, H_q, d), k.view(B, L, H_kv, d), v.view(B, L, H_kv, d),
                                  causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_f.view(B * L, H_q, d))
    # LSE [H_q, total_q] against [B, H_q, L]
    assert torch.equal(l_p, l_f.permute(1, 0, 2).reshape(H_q, B * L))


@pytest.mark.parametrize("B", [1024, 1025])
def test_varlen_schedule_at_the_sequence_limit(m, B):
    """1024 sequences: the largest batch the schedule is planned for (its LDS
    scans and binary search at full size); 1025: no schedule size exists, and
    the call runs the grid.  Short causal prompts of 0..48 tokens, d = 128,
    two KV heads of four query heads; the schedule against the grid bit for
    bit, and sampled sequences against the oracle."""
    import torch
    H_q, H_kv, d = 8, 2, 128
    lens = np.random.default_rng(B).integers(0, 48, size=B, endpoint=True)
    lens[[0, B // 2]] = 0
    lq = lens.tolist()
    say("prefill varlen at the sequence limit", B, "sequences", sum(lq), "tokens")
    cq = _cu(lq)
    tq = int(cq[-1])
    q = W.round_bf16(W.normal(106, 1, (tq, H_q, d)))
    k = W.round_bf16(W.normal(106, 2, (tq, H_kv, d)))
    v = W.round_bf16(W.normal(106, 3, (tq, H_kv, d)))
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    cqd = torch.from_numpy(cq).cuda()
    need = m.prefill_varlen_workspace_bytes(B, max(lq), tq, H_q, H_kv, d)
    assert (need > 0) == (B <= 1024)
    o_s = m.gqa_attn_prefill_varlen(qd, kd, vd, cqd, cqd, max(lq), max(lq), out_dtype=torch.float32)
    o_g = m.gqa_attn_prefill_varlen(qd, kd, vd, cqd, cqd, max(lq), max(lq), out_dtype=torch.float32,
                                    schedule=False)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_g)
    got = host(o_s)
    scale = 1.0 / math.sqrt(d)
    for b in (1, 2, B // 2 + 1, B - 1):
        if lq[b] == 0:
            continue
        sl = slice(cq[b], cq[b + 1])
        ref, _ = oracle.attention_varlen(q[sl], k[sl], v[sl], _cu([lq[b]]), _cu([lq[b]]), True, scale)
        assert_close(got[sl], ref, "bf16", f"sequence {b} of {B} ({lq[b]} tokens)")


def test_varlen_schedule_replays_from_a_captured_graph(m):
    """The scheduled packed prefill captured in a HIP graph: the plan rewrites
    the list and zeroes the claim counter with kernel stores on every call (no
    memset node), so each replay, with other work and synchronisations
    between them, equals the eager call bit for bit."""
    import torch
    H_q, H_kv, d = 32, 4, 64
    lq = np.random.default_rng(107).integers(16, 700, size=6, endpoint=True).tolist()
    say("prefill varlen schedule in a graph", lq)
    cq = _cu(lq)
    tq = int(cq[-1])
    q = dev(W.round_bf16(W.normal(107, 1, (tq, H_q, d))), "bf16")
    k = dev(W.round_bf16(W.normal(107, 2, (tq, H_kv, d))), "bf16")
    v = dev(W.round_bf16(W.normal(107, 3, (tq, H_kv, d))), "bf16")
    cqd = torch.from_numpy(cq).cuda()
    ws = torch.empty(m.prefill_varlen_workspace_bytes(len(lq), max(lq), tq, H_q, H_kv, d), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty(tq, H_q, d, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    call = lambda: m.gqa_attn_prefill_varlen(q, k, v, cqd, cqd, max(lq), max(lq), out=o, workspace=ws)
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    ref = o.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for i in range(3):
        o.zero_()
        ws.fill_(0xFF)  # stale schedule and counter bytes
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"replay {i}"
