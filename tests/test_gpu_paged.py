"""Decode over a paged KV cache: parity with the oracle (which gathers the pages
into the contiguous cache they describe), bit-identity with the contiguous
kernel on the same rows, and pages outside the pool reading as zeros."""
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


def _paged(rng, kc, vc, P, extra_pages=3):
    """Scatter contiguous caches [B, L, H, d] into a shuffled page pool; the
    table's entries past each sequence's pages hold ids that must never be read."""
    B, L = kc.shape[:2]
    pps = L // P
    n = B * pps + extra_pages
    slots = rng.permutation(n)[:B * pps].reshape(B, pps).astype(np.int32)
    kp = np.zeros((n, P) + kc.shape[2:], dtype=kc.dtype)
    vp = np.zeros_like(kp)
    for b in range(B):
        for i in range(pps):
            kp[slots[b, i]] = kc[b, i * P:(i + 1) * P]
            vp[slots[b, i]] = vc[b, i * P:(i + 1) * P]
    return kp, vp, slots


# B, H_q, H_kv, d, page size, pages per sequence, kv_split
PAGED = [
    (4, 8, 2, 128, 16, 12, 0),
    (3, 16, 1, 128, 32, 5, 0),
    (5, 4, 4, 64, 48, 4, 64),
    (2, 32, 8, 128, 64, 3, 32),
]


@pytest.mark.parametrize("B,H_q,H_kv,d,P,pps,split", PAGED)
def test_paged_decode_matches_oracle_and_contiguous_bits(m, B, H_q, H_kv, d, P, pps, split):
    import torch
    say("paged decode", B, H_q, H_kv, d, P, pps, split)
    rng = np.random.default_rng(B * 100 + P)
    L = pps * P
    kc = W.round_bf16(W.normal(71, B, (B, L, H_kv, d)))
    vc = W.round_bf16(W.normal(72, B, (B, L, H_kv, d)))
    q = W.round_bf16(W.normal(73, B, (B, H_q, d)))
    lens = rng.integers(1, L + 1, size=B).astype(np.int32)
    lens[0] = L
    kp, vp, table = _paged(rng, kc, vc, P)
    # entries past each sequence's used pages: never read, so any value is harmless
    for b in range(B):
        used = -(-int(lens[b]) // P)
        table[b, used:] = [-1, 1 << 30][b % 2]
    scale = 1.0 / math.sqrt(d)
    lens_d = torch.from_numpy(lens).cuda()
    got = m.gqa_attn_decode_paged(dev(q, "bf16"), dev(kp, "bf16"), dev(vp, "bf16"),
                                  torch.from_numpy(table).cuda(), lens_d, scale=scale, kv_split=split)
    ref, _ = oracle.decode(q, kc, vc, lens, scale)
    assert_close(host(got), ref, "bf16", f"paged decode P={P}")
    cont = m.gqa_attn_decode(dev(q, "bf16"), dev(kc, "bf16"), dev(vc, "bf16"), lens_d, scale=scale,
                             kv_split=split)
    assert torch.equal(got, cont), "paged and contiguous caches with the same rows must give the same bits"


def test_paged_balanced_split_equals_contiguous_bits(m):
    """A cache large enough for the balanced work split (32 sequences x 8 KV
    heads x 2048 keys), ragged lengths, 16-key pages."""
    import torch
    B, H_q, H_kv, d, P, L = 32, 32, 8, 128, 16, 2048
    say("paged balanced", B, H_q, H_kv, d, P, L)
    g = torch.Generator(device="cpu").manual_seed(5)
    kc = torch.randn(B, L, H_kv, d, generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn(B, L, H_kv, d, generator=g).to(torch.bfloat16).cuda()
    q = torch.randn(B, H_q, d, generator=g).to(torch.bfloat16).cuda()
    lens = torch.randint(1, L + 1, (B,), generator=g, dtype=torch.int32).cuda()
    pps = L // P
    perm = torch.randperm(B * pps, generator=g).to(torch.int32)
    table = perm.reshape(B, pps).cuda()
    kp = torch.empty(B * pps, P, H_kv, d, dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    kp[table.flatten().long()] = kc.reshape(B * pps, P, H_kv, d)
    vp[table.flatten().long()] = vc.reshape(B * pps, P, H_kv, d)
    got = m.gqa_attn_decode_paged(q, kp, vp, table, lens)
    cont = m.gqa_attn_decode(q, kc, vc, lens)
    assert torch.equal(got, cont)
    # and a sampled check of two sequences against the oracle
    for b in (0, B - 1):
        n = int(lens[b])
        ref, _ = oracle.decode(host(q[b:b + 1]), host(kc[b:b + 1]), host(vc[b:b + 1]), np.array([n]),
                               1.0 / math.sqrt(d))
        assert_close(host(got[b:b + 1]), ref, "bf16", f"paged balanced seq {b}")


def test_pages_outside_the_pool_read_as_zeros(m):
    import torch
    B, H_q, H_kv, d, P, pps = 2, 8, 2, 64, 16, 4
    rng = np.random.default_rng(9)
    kp = W.round_bf16(W.normal(81, 1, (B * pps, P, H_kv, d)))
    vp = W.round_bf16(W.normal(82, 1, (B * pps, P, H_kv, d)))
    q = W.round_bf16(W.normal(83, 1, (B, H_q, d)))
    table = np.arange(B * pps, dtype=np.int32).reshape(B, pps)
    table[0, 1] = -5           # a hole inside sequence 0's keys
    table[1, 2] = B * pps + 7  # an id past the pool inside sequence 1's keys
    lens = np.array([pps * P, pps * P - 3], dtype=np.int32)
    got = m.gqa_attn_decode_paged(dev(q, "bf16"), dev(kp, "bf16"), dev(vp, "bf16"),
                                  torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), scale=0.2)
    ref, _ = oracle.decode_paged(q, kp, vp, table, lens, 0.2)
    assert_close(host(got), ref, "bf16", "holes in the page table")
