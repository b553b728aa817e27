"""A prefill layer (the projection on the LDS-DMA tile path, the split views,
the causal prefill with its V-image pre-pass) captured once as a HIP graph and
replayed with new inputs: every replay must equal the same layer run eagerly,
bit for bit, with eager work and synchronisations between the replays.  The
oracle parity of each call is covered by the other tests; this one checks that
nothing in the calls depends on host-side state at launch time (the tile
kernel's LDS is static, its scratch is the caller's)."""
import math

import pytest

import workloads as W
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mqa_qkv_proj_amd
    return mqa_qkv_proj_amd


# B, L, hidden, H_q, H_kv, d, rope + bias
LAYERS = [
    (1, 512, 512, 8, 2, 64, False),    # 64-row tiles, d = 64
    (2, 300, 256, 8, 2, 128, True),    # ragged rows, d = 128, rotation and bias in the epilogue
]


@pytest.mark.parametrize("B,L,hidden,H_q,H_kv,d,rope", LAYERS)
def test_layer_graph_replays_match_eager(m, B, L, hidden, H_q, H_kv, d, rope):
    import torch
    say("layer graph", B, L, hidden, H_q, H_kv, d, rope)
    N = (H_q + 2 * H_kv) * d
    M = B * L
    steps = 4
    xs = [dev(W.round_bf16(W.normal(300 + s, 1, (B, L, hidden))), "bf16") for s in range(steps)]
    w = dev(W.round_bf16(W.normal(301, 2, (hidden, N), std=1.0 / math.sqrt(hidden))), "bf16")
    bias = dev(W.round_bf16(W.normal(302, 3, (1, N))[0]), "bf16") if rope else None
    pos = torch.from_numpy(W.prefill_positions(B, L)).cuda()
    th = torch.from_numpy(W.rope_inv_freq(d)).cuda()
    x = torch.empty(B, L, hidden, dtype=torch.bfloat16, device="cuda")
    qkv = torch.empty(B, L, N, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(B, L, H_q, d, dtype=torch.bfloat16, device="cuda")
    wsg = torch.empty(max(16, m.qkv_proj_workspace_bytes(M, hidden, H_q, H_kv, d)), dtype=torch.uint8, device="cuda")
    wsp = torch.empty(m.prefill_workspace_bytes(B, L, H_kv, d), dtype=torch.uint8, device="cuda")
    q, k, v = m.split_qkv(qkv, H_q, H_kv, d)

    def layer():
        if rope:
            m.qkv_proj_rope(x.view(M, hidden), w, pos, th, H_q, H_kv, d, bias=bias, out=qkv.view(M, N),
                            workspace=wsg)
        else:
            m.qkv_proj(x.view(M, hidden), w, H_q, H_kv, d, out=qkv.view(M, N), workspace=wsg)
        m.gqa_attn_prefill(q, k, v, causal=True, out=o, workspace=wsp)

    eager = []
    for s in range(steps):
        x.copy_(xs[s])
        layer()
        eager.append((qkv.clone(), o.clone()))
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    x.copy_(xs[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()
    for s in range(steps):
        x.copy_(xs[s])  # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(qkv, eager[s][0]), f"replay {s}: qkv differs from the eager layer"
        assert torch.equal(o, eager[s][1]), f"replay {s}: attention output differs from the eager layer"
    say("graph replays equal the eager layers")
