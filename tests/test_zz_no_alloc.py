"""gqa_attn_decode_noalloc: the decode call without a workspace argument, whose
split partials live in the library's static per-GPU scratch buffer.

Called through the C ABI (ctypes, device pointers), it must give the bits of
gqa_attn_decode with a caller workspace on the same inputs, and so the oracle's
result within the bf16 bar.  Two bf16 calls in a row, the second smaller, so
the second reuses a buffer that still holds the first call's partials; then an
fp32 call (the other split kernel) and a batch with an empty sequence."""
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


def _noalloc(m, q, kc, vc, lens, out_dtype, lse=True, split=0):
    """One call of the C entry point on torch device tensors; returns (o, lse)."""
    import torch
    B, H_q, d = q.shape
    _, L_max, H_kv, _ = kc.shape
    o = torch.empty(B, H_q, d, dtype=out_dtype, device=q.device)
    ls = torch.empty(B, H_q, dtype=torch.float32, device=q.device) if lse else None
    code = {torch.bfloat16: m.MQKV_BF16, torch.float32: m.MQKV_F32}
    st = m.lib.gqa_attn_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), lens.data_ptr(), o.data_ptr(),
                                       ls.data_ptr() if ls is not None else None, B, H_q, H_kv, d, L_max,
                                       q.stride(0), 1.0 / math.sqrt(d), split, code[q.dtype], code[out_dtype],
                                       torch.cuda.current_stream().cuda_stream)
    m.check(st, "gqa_attn_decode_noalloc")
    return o, ls


CASES = [  # B, H_q, H_kv, d, L_max, dtype, lengths (None: U{L_max/4 .. L_max}), kv_split
    (32, 32, 8, 128, 4096, "bf16", None, 0),     # Llama-2-7B-shaped GQA decode, balanced split
    (3, 8, 2, 64, 200, "bf16", [200, 1, 77], 0),  # smaller: reuses the buffer the first call filled
    (4, 8, 2, 128, 300, "f32", [300, 33, 1, 64], 0),
    (5, 16, 1, 128, 1040, "bf16", [1040, 0, 17, 513, 0], 64),
]


def test_noalloc_decode_matches_the_workspace_call(m):
    import torch
    for i, (B, H_q, H_kv, d, L_max, dtype, lens, split) in enumerate(CASES):
        say("decode noalloc call", i, B, H_q, H_kv, d, L_max, dtype, lens, split)
        enc = W.round_bf16 if dtype == "bf16" else (lambda a: a)
        kc = enc(W.normal(341 + i, 1, (B, L_max, H_kv, d)))
        vc = enc(W.normal(341 + i, 2, (B, L_max, H_kv, d)))
        q = enc(W.normal(341 + i, 3, (B, H_q, d)))
        if lens is None:
            lens = np.random.default_rng(341).integers(L_max // 4, L_max + 1, size=B)
        lens = np.asarray(lens, np.int32)
        qd, kd, vd = dev(q, dtype), dev(kc, dtype), dev(vc, dtype)
        lens_d = torch.from_numpy(lens).cuda()
        o, lse = _noalloc(m, qd, kd, vd, lens_d, torch.float32, split=split)
        ref_o, ref_l = m.gqa_attn_decode(qd, kd, vd, lens_d, kv_split=split, return_lse=True,
                                         out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), f"call {i}: O differs from gqa_attn_decode's"
        assert torch.equal(lse, ref_l), f"call {i}: LSE differs from gqa_attn_decode's"
        oo, ol = oracle.decode(q, kc, vc, lens, 1.0 / math.sqrt(d))
        keep = lens > 0
        assert_close(host(o)[keep], oo[keep], dtype, f"noalloc call {i} O vs oracle")
        assert np.all(host(o)[~keep] == 0) and np.all(host(lse)[~keep] == -np.inf)
        if dtype == "bf16":  # bf16 output, no LSE
            ob, _ = _noalloc(m, qd, kd, vd, lens_d, torch.bfloat16, lse=False, split=split)
            rb = m.gqa_attn_decode(qd, kd, vd, lens_d, kv_split=split)
            torch.cuda.synchronize()
            assert torch.equal(ob, rb), f"call {i}: bf16 O differs from gqa_attn_decode's"
        del kd, vd
        torch.cuda.empty_cache()
