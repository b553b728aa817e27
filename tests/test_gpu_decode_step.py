"""The decode step as one unit: the projection with the KV-cache append fused
into its epilogue (qkv_proj_append), chained with decode, and the whole step
captured as a HIP graph and replayed.

Parity is against the oracle's plain definition (project, split, write the new
token's K/V at position seq_lens[b] - 1, attend); the cache rows are checked
bit for bit: the appended rows must equal the qkv output's K/V columns, every
other row must keep its previous contents."""
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


def _lens(rng, B, L_max, skip=True):
    lens = rng.integers(1, L_max + 1, size=B).astype(np.int32)
    if skip and B >= 3:
        lens[1] = 0           # not appended: length 0
        lens[-1] = L_max + 1  # not appended: beyond the cache
    return lens


# B, hidden, H_q, H_kv, d, L_max, dtype: the cases reach every projection kernel
# (16-column streaming; register transpose + reduce; skinny with and without a
# k split; 8-wave workgroups over all of K; LDS-DMA tiles; register-prefetched
# tiles; fp32).  With a k split the append sits in the reduce kernel.
APPEND = [
    (8, 512, 16, 1, 128, 40, "bf16"),     # streaming kernel, one 16-row block
    (24, 256, 4, 2, 64, 33, "bf16"),      # streaming kernel, two 16-row blocks
    (32, 1024, 32, 8, 128, 50, "bf16"),   # register transpose, k split + reduce kernel
    (20, 640, 64, 2, 128, 24, "bf16"),    # skinny, k split + reduce kernel (hidden % 256 != 0)
    (100, 128, 8, 2, 64, 20, "bf16"),     # skinny, one k range
    (48, 512, 8, 2, 64, 20, "bf16"),      # 8-wave workgroups over all of K
    (300, 256, 8, 2, 64, 9, "bf16"),      # LDS-DMA tiles
    (200, 264, 4, 2, 64, 17, "bf16"),     # register-prefetched tiles (hidden % 64 != 0)
    (20, 128, 4, 2, 64, 12, "f32"),       # fp32 path
]


@pytest.mark.parametrize("B,hidden,H_q,H_kv,d,L_max,dtype", APPEND)
def test_qkv_proj_append_matches_oracle_and_touches_one_row(m, B, hidden, H_q, H_kv, d, L_max, dtype):
    import torch
    say("qkv_proj_append", B, hidden, H_q, H_kv, d, L_max, dtype)
    rng = np.random.default_rng(B * 7 + hidden)
    N = (H_q + 2 * H_kv) * d
    enc = W.round_bf16 if dtype == "bf16" else (lambda a: a)
    x = enc(W.normal(31, B, (B, hidden)))
    w = enc(W.normal(32, hidden, (hidden, N), std=1.0 / math.sqrt(hidden)))
    kc0 = enc(W.normal(33, B, (B, L_max, H_kv, d)))
    vc0 = enc(W.normal(34, B, (B, L_max, H_kv, d)))
    lens = _lens(rng, B, L_max)
    kc, vc = dev(kc0, dtype), dev(vc0, dtype)
    lens_d = torch.from_numpy(lens).cuda()
    qkv = m.qkv_proj_append(dev(x, dtype), dev(w, dtype), kc, vc, lens_d, H_q, H_kv, d)
    got = host(qkv)
    assert_close(got, oracle.qkv_proj(x, w), dtype, f"qkv_proj_append B={B}")
    # the caches: exactly the appended rows changed, to the bits of qkv's K/V columns
    _, k_new, v_new = oracle.split_qkv(got[:, None, :], H_q, H_kv, d)
    kc_ref, vc_ref = oracle.kv_append(kc0, vc0, k_new[:, 0], v_new[:, 0], lens)
    assert np.array_equal(host(kc), kc_ref), "k_cache differs from qkv's K columns / its old contents"
    assert np.array_equal(host(vc), vc_ref), "v_cache differs from qkv's V columns / its old contents"


def test_qkv_proj_append_equals_qkv_proj(m):
    """The append changes nothing of the projection itself: same bits as qkv_proj."""
    import torch
    B, hidden, H_q, H_kv, d, L_max = 32, 1024, 32, 8, 128, 16
    N = (H_q + 2 * H_kv) * d
    x = dev(W.round_bf16(W.normal(41, 1, (B, hidden))), "bf16")
    w = dev(W.round_bf16(W.normal(42, 1, (hidden, N), std=0.03)), "bf16")
    kc = torch.zeros(B, L_max, H_kv, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    lens = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    a = m.qkv_proj_append(x, w, kc, vc, lens, H_q, H_kv, d)
    b = m.qkv_proj(x, w, H_q, H_kv, d)
    assert torch.equal(a, b)


def _decode_step_inputs(B, hidden, H_q, H_kv, d, L_max, steps, seed):
    N = (H_q + 2 * H_kv) * d
    xs = W.round_bf16(W.normal(seed, 1, (steps, B, hidden)))
    w = W.round_bf16(W.normal(seed + 1, 1, (hidden, N), std=1.0 / math.sqrt(hidden)))
    kc = W.round_bf16(W.normal(seed + 2, 1, (B, L_max, H_kv, d)))
    vc = W.round_bf16(W.normal(seed + 3, 1, (B, L_max, H_kv, d)))
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, L_max - steps + 1, size=B).astype(np.int32)
    return xs, w, kc, vc, lens


@pytest.mark.parametrize("B,hidden,H_q,H_kv,d,L_max", [
    (8, 2048, 16, 1, 128, 64),    # the MQA decode shape (16 query heads on one KV head)
    (32, 1024, 32, 8, 128, 80),   # GQA-8, projection with a k split
])
def test_decode_steps_match_oracle(m, B, hidden, H_q, H_kv, d, L_max):
    """Project + append, then decode, for a few steps; each step against the oracle."""
    import torch
    say("decode steps", B, hidden, H_q, H_kv, d, L_max)
    steps = 3
    xs, w, kc0, vc0, lens0 = _decode_step_inputs(B, hidden, H_q, H_kv, d, L_max, steps, 51)
    wd = dev(w, "bf16")
    kc, vc = dev(kc0, "bf16"), dev(vc0, "bf16")
    kc_ref, vc_ref = kc0.astype(np.float64), vc0.astype(np.float64)
    lens = lens0.copy()
    scale = 1.0 / math.sqrt(d)
    for s in range(steps):
        lens_d = torch.from_numpy(lens).cuda()
        qkv = m.qkv_proj_append(dev(xs[s], "bf16"), wd, kc, vc, lens_d, H_q, H_kv, d)
        q = qkv[:, :H_q * d].unflatten(-1, (H_q, d))
        o = m.gqa_attn_decode(q, kc, vc, lens_d, scale=scale)
        # oracle step on the GPU's own projection (stage-wise parity)
        qkv_h = host(qkv)
        qo, ko, vo = oracle.split_qkv(qkv_h[:, None, :], H_q, H_kv, d)
        kc_ref, vc_ref = oracle.kv_append(kc_ref, vc_ref, ko[:, 0], vo[:, 0], lens)
        O_ref, _ = oracle.decode(qo[:, 0], kc_ref, vc_ref, lens, scale)
        assert_close(host(o), O_ref, "bf16", f"decode step {s}")
        assert np.array_equal(host(kc), kc_ref) and np.array_equal(host(vc), vc_ref)
        lens = lens + 1


@pytest.mark.parametrize("B,hidden,H_q,H_kv,d,L_max,steps", [
    (8, 2048, 16, 1, 128, 48, 5),     # MQA: 16-column streaming projection
    (32, 4096, 32, 8, 128, 96, 4),    # Llama-2-7B GQA-8 width: register transpose + reduce kernel
])
def test_decode_step_graph_replays_match_eager(m, B, hidden, H_q, H_kv, d, L_max, steps):
    """The whole step (project + append, decode, lengths + 1) captured once as a
    HIP graph and replayed: every replay equals the same step run eagerly, with
    eager work and synchronisations between the replays."""
    import torch
    N = (H_q + 2 * H_kv) * d
    say("decode step graph", B, hidden, H_q, H_kv, d, L_max, steps)
    xs, w, kc0, vc0, lens0 = _decode_step_inputs(B, hidden, H_q, H_kv, d, L_max, steps, 61)
    wd = dev(w, "bf16")
    xs_d = [dev(xs[s], "bf16") for s in range(steps)]
    scale = 1.0 / math.sqrt(d)

    def buffers():
        return dict(kc=dev(kc0, "bf16"), vc=dev(vc0, "bf16"), lens=torch.from_numpy(lens0.copy()).cuda(),
                    qkv=torch.empty(B, N, dtype=torch.bfloat16, device="cuda"),
                    o=torch.empty(B, H_q, d, dtype=torch.bfloat16, device="cuda"),
                    ws_p=torch.empty(max(16, m.qkv_proj_workspace_bytes(B, hidden, H_q, H_kv, d)),
                                     dtype=torch.uint8, device="cuda"),
                    ws_d=torch.empty(m.decode_workspace_bytes(B, H_q, H_kv, d, L_max), dtype=torch.uint8,
                                     device="cuda"),
                    x=torch.empty(B, hidden, dtype=torch.bfloat16, device="cuda"))

    def step(bf):
        m.qkv_proj_append(bf["x"], wd, bf["kc"], bf["vc"], bf["lens"], H_q, H_kv, d, out=bf["qkv"],
                          workspace=bf["ws_p"])
        q = bf["qkv"][:, :H_q * d].unflatten(-1, (H_q, d))
        m.gqa_attn_decode(q, bf["kc"], bf["vc"], bf["lens"], scale=scale, workspace=bf["ws_d"], out=bf["o"])
        bf["lens"].add_(1)

    # eager reference, step by step
    ref = buffers()
    eager_o = []
    for s in range(steps):
        ref["x"].copy_(xs_d[s])
        step(ref)
        eager_o.append(ref["o"].clone())
    torch.cuda.synchronize()

    g_bf = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (on copies, state restored below)
        warm = buffers()
        warm["x"].copy_(xs_d[0])
        step(warm)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    g_bf["x"].copy_(xs_d[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(g_bf)
    # capture records without running: the state is still the initial one
    torch.cuda.synchronize()
    assert torch.equal(g_bf["lens"].cpu(), torch.from_numpy(lens0))
    for s in range(steps):
        g_bf["x"].copy_(xs_d[s])          # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_bf["o"], eager_o[s]), f"replay {s}: output differs from the eager step"
        assert torch.equal(g_bf["lens"].cpu(), torch.from_numpy(lens0 + s + 1))
    assert torch.equal(g_bf["kc"], ref["kc"]) and torch.equal(g_bf["vc"], ref["vc"])
    say("graph replays equal the eager steps")
