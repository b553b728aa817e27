"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects malformed arguments on the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa_qkv.h")

INV, UNS = 1, 2
F32, BF16 = 0, 1
A = 0x1000  # a 16-byte aligned fake device address; never dereferenced on rejection


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)) - {"if"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("qkv_proj", "qkv_proj_workspace_bytes", "qkv_proj_append", "qkv_proj_rope", "qkv_proj_append_rope",
              "gqa_attn_prefill",
              "gqa_attn_prefill_workspace_bytes",
              "gqa_attn_decode", "gqa_attn_decode_workspace_bytes", "gqa_attn_decode_paged",
              "gqa_attn_prefill_varlen", "gqa_attn_prefill_varlen_workspace_bytes",
              "gqa_attn_prefill_fp8", "gqa_attn_prefill_fp8_workspace_bytes",
              "mqkv_status_string", "mqkv_last_error", "mqkv_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), f"{n} declared in mqa_qkv.h but not exported"
    assert set(lib.EXPORTS) <= set(declared_functions())


def test_status_strings(lib):
    L = lib.lib
    assert L.mqkv_status_string(0) == b"ok"
    assert L.mqkv_status_string(1) == b"invalid argument"
    assert L.mqkv_status_string(2) == b"unsupported configuration"
    assert L.mqkv_status_string(3) == b"HIP runtime error"
    assert L.mqkv_abi_version() == 108


def proj(lib, **kw):
    a = dict(x=A, w=A, bias=None, out=A, M=16, hidden=256, H_q=4, H_kv=2, d=64, dtype=BF16)
    a.update(kw)
    return lib.lib.qkv_proj(a["x"], a["w"], a["bias"], a["out"], a["M"], a["hidden"], a["H_q"], a["H_kv"],
                            a["d"], a["dtype"], a.get("ws"), a.get("wsb", 0), None)


def proj_append(lib, **kw):
    a = dict(x=A, w=A, bias=None, out=A, kc=A, vc=A, lens=A, B=8, hidden=256, H_q=4, H_kv=2, d=64, Lmax=64,
             dtype=BF16)
    a.update(kw)
    return lib.lib.qkv_proj_append(a["x"], a["w"], a["bias"], a["out"], a["kc"], a["vc"], a["lens"], a["B"],
                                   a["hidden"], a["H_q"], a["H_kv"], a["d"], a["Lmax"], a["dtype"], a.get("ws"),
                                   a.get("wsb", 0), None)


def prefill(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=None, B=1, Lq=16, Lkv=16, H_q=4, H_kv=2, d=64, qs=512, ks=512,
             causal=1, scale=0.125, dt=BF16, odt=BF16, ws=A, wsb=1 << 20)
    a.update(kw)
    return lib.lib.gqa_attn_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Lq"], a["Lkv"],
                                    a["H_q"], a["H_kv"], a["d"], a["qs"], a["ks"], a["causal"], a["scale"],
                                    a["dt"], a["odt"], a["ws"], a["wsb"], None)


def decode(lib, **kw):
    a = dict(q=A, k=A, v=A, lens=A, o=A, lse=None, B=2, H_q=8, H_kv=2, d=128, Lmax=100, qs=1024,
             scale=0.1, split=0, ws=A, wsb=1 << 20, dt=BF16, odt=BF16)
    a.update(kw)
    return lib.lib.gqa_attn_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["H_q"],
                                   a["H_kv"], a["d"], a["Lmax"], a["qs"], a["scale"], a["split"], a["ws"],
                                   a["wsb"], a["dt"], a["odt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), INV), (dict(out=None), INV), (dict(w=A + 2), INV), (dict(M=-1), INV),
    (dict(hidden=0), INV), (dict(hidden=260), INV), (dict(H_q=3, H_kv=2), INV), (dict(H_kv=0), INV),
    (dict(d=96), UNS), (dict(d=0), INV), (dict(dtype=7), INV), (dict(M=1 << 40), UNS),
    (dict(ws=A + 4, wsb=1 << 20), INV),
])
def test_qkv_proj_rejects(lib, kw, code):
    assert proj(lib, **kw) == code
    assert lib.lib.mqkv_last_error() != b""


def test_qkv_proj_empty_is_noop(lib):
    assert proj(lib, M=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), INV), (dict(vc=None), INV), (dict(lens=None), INV), (dict(kc=A + 8), INV),
    (dict(lens=A + 2), INV), (dict(B=-1), INV), (dict(Lmax=0), INV), (dict(x=None), INV),
    (dict(H_q=3, H_kv=2), INV), (dict(d=96), UNS), (dict(hidden=260), INV), (dict(dtype=7), INV),
    (dict(ws=A + 4, wsb=1 << 20), INV),
])
def test_qkv_proj_append_rejects(lib, kw, code):
    assert proj_append(lib, **kw) == code
    assert lib.lib.mqkv_last_error() != b""


def test_qkv_proj_append_empty_is_noop(lib):
    assert proj_append(lib, B=0) == 0


def proj_rope(lib, **kw):
    a = dict(x=A, w=A, bias=None, out=A, pos=A, th=A, M=16, hidden=256, H_q=4, H_kv=2, d=64, dtype=BF16)
    a.update(kw)
    return lib.lib.qkv_proj_rope(a["x"], a["w"], a["bias"], a["out"], a["pos"], a["th"], a["M"], a["hidden"],
                                 a["H_q"], a["H_kv"], a["d"], a["dtype"], a.get("ws"), a.get("wsb", 0), None)


def proj_append_rope(lib, **kw):
    a = dict(x=A, w=A, bias=None, out=A, kc=A, vc=A, lens=A, th=A, B=8, hidden=256, H_q=4, H_kv=2, d=64, Lmax=64,
             dtype=BF16)
    a.update(kw)
    return lib.lib.qkv_proj_append_rope(a["x"], a["w"], a["bias"], a["out"], a["kc"], a["vc"], a["lens"], a["th"],
                                        a["B"], a["hidden"], a["H_q"], a["H_kv"], a["d"], a["Lmax"], a["dtype"],
                                        a.get("ws"), a.get("wsb", 0), None)


@pytest.mark.parametrize("kw,code", [
    (dict(pos=None), INV), (dict(th=None), INV), (dict(pos=A + 2), INV), (dict(th=A + 1), INV),
    (dict(x=None), INV), (dict(M=-1), INV), (dict(hidden=260), INV), (dict(H_q=3, H_kv=2), INV),
    (dict(d=96), UNS), (dict(dtype=7), INV), (dict(M=1 << 40), UNS),
])
def test_qkv_proj_rope_rejects(lib, kw, code):
    assert proj_rope(lib, **kw) == code
    assert lib.lib.mqkv_last_error() != b""


@pytest.mark.parametrize("kw,code", [
    (dict(th=None), INV), (dict(th=A + 2), INV), (dict(kc=None), INV), (dict(lens=A + 2), INV),
    (dict(B=-1), INV), (dict(Lmax=0), INV), (dict(d=96), UNS), (dict(H_q=3, H_kv=2), INV),
])
def test_qkv_proj_append_rope_rejects(lib, kw, code):
    assert proj_append_rope(lib, **kw) == code
    assert lib.lib.mqkv_last_error() != b""


def test_rope_calls_empty_are_noops(lib):
    assert proj_rope(lib, M=0) == 0
    assert proj_append_rope(lib, B=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(o=A + 8), INV), (dict(lse=A + 4), INV), (dict(Lkv=0), INV),
    (dict(causal=1, Lq=17, Lkv=16), INV), (dict(causal=2), INV), (dict(scale=float("nan")), INV),
    (dict(scale=float("inf")), INV), (dict(scale=-1.0), INV), (dict(qs=100), INV), (dict(qs=516), INV),
    (dict(ks=130), INV), (dict(H_q=4, H_kv=3), INV), (dict(d=256, qs=1024, ks=512), UNS),
    (dict(dt=F32, odt=BF16), UNS), (dict(B=-1), INV), (dict(dt=3), INV),
    (dict(ws=None), INV), (dict(ws=A + 8), INV), (dict(wsb=18431), INV),
])
def test_prefill_rejects(lib, kw, code):
    assert prefill(lib, **kw) == code


def prefill_varlen(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=None, cuq=A, cuk=A, B=3, mq=64, mk=64, tq=100, tk=100, H_q=4, H_kv=2, d=64,
             qs=512, ks=512, causal=1, scale=0.125, dt=BF16, odt=BF16, ws=A, wsb=1 << 20)
    a.update(kw)
    return lib.lib.gqa_attn_prefill_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cuq"], a["cuk"], a["B"],
                                           a["mq"], a["mk"], a["tq"], a["tk"], a["H_q"], a["H_kv"], a["d"], a["qs"],
                                           a["ks"], a["causal"], a["scale"], a["dt"], a["odt"], a["ws"], a["wsb"],
                                           None)


@pytest.mark.parametrize("kw,code", [
    (dict(cuq=None), INV), (dict(cuk=A + 2), INV), (dict(q=None), INV), (dict(mk=0), INV), (dict(tk=0), INV),
    (dict(B=-1), INV), (dict(mq=-1), INV), (dict(causal=3), INV), (dict(scale=float("nan")), INV),
    (dict(qs=100), INV), (dict(dt=F32, odt=F32), UNS), (dict(d=96), UNS), (dict(ws=None), INV),
    (dict(wsb=1000), INV), (dict(H_q=4, H_kv=3), INV),
])
def test_prefill_varlen_rejects(lib, kw, code):
    assert prefill_varlen(lib, **kw) == code


def test_prefill_varlen_empty_is_noop(lib):
    assert prefill_varlen(lib, B=0) == 0
    assert prefill_varlen(lib, mq=0) == 0
    assert prefill_varlen(lib, tq=0) == 0


def test_prefill_empty_is_noop(lib):
    assert prefill(lib, B=0) == 0
    assert prefill(lib, Lq=0) == 0


def test_projection_workspace_query(lib):
    f = lib.qkv_proj_workspace_bytes
    # decode-sized M: the hidden dimension is split, partials need M*N*4 bytes per k range
    n = f(32, 4096, 32, 8, 128)
    assert n > 0 and n % (32 * 6144 * 4) == 0
    assert f(4096, 4096, 32, 8, 128) == 0      # large M: single pass, no workspace
    assert f(32, 4096, 32, 8, 128, 0) == 0     # fp32 path: no workspace
    assert f(32, 4096, 32, 3, 128) == 0        # invalid heads


def test_prefill_workspace_query(lib):
    f = lib.prefill_workspace_bytes
    # bf16: one fp16 V^T image of (d rows x (64 + 8) keys) per 64-key tile, batch and KV head
    assert f(2, 100, 4, 128) == 2 * 4 * 2 * 128 * 72 * 2
    assert f(1, 16, 2, 64) == 1 * 2 * 1 * 64 * 72 * 2 == 18432
    assert f(1, 64, 1, 64) == 9216 and f(1, 65, 1, 64) == 2 * 9216
    assert f(2, 100, 4, 128, 0) == 0          # fp32 inputs need none
    assert f(2, 100, 4, 96) == 0              # unsupported d
    assert f(2, 0, 4, 128) == 0               # L_kv < 1


def test_prefill_varlen_workspace_query(lib):
    """The packed-batch workspace: the V images (256-byte aligned), then a
    4-word header and one (sequence, query block) pair of int32 per row block.
    Row blocks hold P = W*32/F query positions (W = 8 waves at d = 128, 4 at
    d = 64; F = the largest power of two dividing G, at most 32), and the list
    holds B + ceil(total_q / P) of them, enough for any lengths summing to
    total_q."""
    f = lib.prefill_varlen_workspace_bytes
    img = lib.prefill_workspace_bytes
    r256 = lambda n: (n + 255) // 256 * 256
    # d = 64, G = 8: F = 8, P = 4*32/8 = 16; cap = 8 + 8000/16 = 508 pairs
    assert f(8, 2048, 8000, 32, 4, 64) == r256(img(8, 2048, 4, 64)) + r256(4 * (4 + 2 * 508))
    # d = 128, G = 4: F = 4, P = 8*32/4 = 64; cap = 3 + ceil(1000/64) = 19
    assert f(3, 700, 1000, 16, 4, 128) == r256(img(3, 700, 4, 128)) + r256(4 * (4 + 2 * 19))
    # G = 6: F = 2, P = 128 at d = 128
    assert f(2, 100, 300, 12, 2, 128) == r256(img(2, 100, 2, 128)) + r256(4 * (4 + 2 * (2 + 3)))
    assert f(1024, 64, 10, 8, 2, 128) > 0
    assert f(1025, 64, 10, 8, 2, 128) == 0    # no schedule past 1024 sequences
    assert f(0, 64, 10, 8, 2, 128) == 0
    assert f(2, 64, 10, 8, 3, 128) == 0       # H_q % H_kv
    assert f(2, 64, 10, 8, 2, 96) == 0        # d


def test_decode_workspace_query(lib):
    f = lib.decode_workspace_bytes
    n = f(32, 32, 8, 128, 4096, 0)
    assert n > 32 * 32 * 128 * 4
    assert f(32, 32, 8, 128, 4096, 64) == 32 * 32 * 64 * (128 * 4 + 16) + 256
    assert f(2, 8, 3, 128, 100, 0) == 0       # H_q % H_kv
    assert f(2, 8, 2, 128, 100, 100) == 0     # split not a multiple of 32
    assert f(2, 8, 2, 96, 100, 0) == 0        # d


@pytest.mark.parametrize("kw,code", [
    (dict(lens=None), INV), (dict(lens=A + 2), INV), (dict(ws=None), INV), (dict(wsb=16), INV),
    (dict(split=100), INV), (dict(split=16), INV), (dict(split=48), INV), (dict(Lmax=0), INV), (dict(qs=1000), INV),
    (dict(qs=512), INV), (dict(scale=float("nan")), INV), (dict(d=80, qs=1024), UNS),
    (dict(dt=F32, odt=BF16), UNS), (dict(H_q=8, H_kv=3), INV), (dict(ws=A + 8), INV),
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code



def decode_noalloc(lib, **kw):
    a = dict(q=A, k=A, v=A, lens=A, o=A, lse=None, B=2, H_q=8, H_kv=2, d=128, Lmax=100, qs=1024, scale=0.1,
             split=0, dt=BF16, odt=BF16)
    a.update(kw)
    return lib.lib.gqa_attn_decode_noalloc(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["H_q"],
                                           a["H_kv"], a["d"], a["Lmax"], a["qs"], a["scale"], a["split"], a["dt"],
                                           a["odt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(lens=None), INV), (dict(lens=A + 2), INV), (dict(split=48), INV), (dict(Lmax=0), INV),
    (dict(qs=512), INV), (dict(scale=float("nan")), INV), (dict(d=80, qs=1024), UNS),
    (dict(dt=F32, odt=BF16), UNS), (dict(H_q=8, H_kv=3), INV), (dict(o=A + 8), INV),
    # partials beyond the static scratch: rejected before any device call
    (dict(B=64, H_q=64, H_kv=8, Lmax=1 << 16, qs=8192), UNS),
    (dict(B=512, H_q=32, H_kv=8, Lmax=4096, qs=4096, split=32), UNS),
])
def test_decode_noalloc_rejects(lib, kw, code):
    assert decode_noalloc(lib, **kw) == code
    assert lib.lib.mqkv_last_error() != b""


def test_decode_noalloc_limit_covers_the_decode_workloads(lib):
    """The static scratch holds the MQA decode workload's partials in either
    dtype (the Llama-2-7B shapes are run on the GPU); the rejection message
    names the limit."""
    f = lib.decode_workspace_bytes
    assert f(8, 16, 1, 128, 1040) <= lib.DECODE_NOALLOC_SCRATCH_BYTES     # MQA decode
    assert decode_noalloc(lib, B=0) == 0
    assert decode_noalloc(lib, B=64, H_q=64, H_kv=8, Lmax=1 << 16, qs=8192) == UNS
    assert str(lib.DECODE_NOALLOC_SCRATCH_BYTES).encode() in lib.lib.mqkv_last_error()

def decode_paged(lib, **kw):
    a = dict(q=A, kp=A, vp=A, bt=A, lens=A, o=A, lse=None, B=2, H_q=8, H_kv=2, d=128, P=16, pps=8, npages=16,
             qs=1024, scale=0.1, split=0, ws=A, wsb=1 << 20, dt=BF16, odt=BF16)
    a.update(kw)
    return lib.lib.gqa_attn_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["lens"], a["o"], a["lse"], a["B"],
                                         a["H_q"], a["H_kv"], a["d"], a["P"], a["pps"], a["npages"], a["qs"],
                                         a["scale"], a["split"], a["ws"], a["wsb"], a["dt"], a["odt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bt=None), INV), (dict(kp=None), INV), (dict(bt=A + 2), INV), (dict(P=0), INV), (dict(P=24), INV),
    (dict(pps=0), INV), (dict(npages=0), INV), (dict(split=48), INV), (dict(scale=-1.0), INV),
    (dict(dt=F32, odt=F32), UNS), (dict(d=80, qs=1024), UNS), (dict(ws=None), INV), (dict(wsb=100), INV),
    (dict(B=-1), INV), (dict(P=1 << 20, pps=1 << 12), UNS),
])
def test_decode_paged_rejects(lib, kw, code):
    assert decode_paged(lib, **kw) == code


def test_decode_paged_empty_is_noop(lib):
    assert decode_paged(lib, B=0) == 0


def test_decode_empty_is_noop(lib):
    assert decode(lib, B=0) == 0


def test_python_layer_validates_without_gpu(lib):
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lib.qkv_proj(x, torch.zeros(256, 512, dtype=torch.bfloat16), 4, 2, 64)  # CPU tensors
    qkv = torch.zeros(2, 5, (8 + 2 * 2) * 64, dtype=torch.bfloat16)
    q, k, v = lib.split_qkv(qkv, 8, 2, 64)
    assert q.shape == (2, 5, 8, 64) and k.shape == (2, 5, 2, 64) and v.shape == (2, 5, 2, 64)
    assert q.data_ptr() == qkv.data_ptr()
    assert k.data_ptr() == qkv.data_ptr() + 8 * 64 * 2 and v.data_ptr() == qkv.data_ptr() + 10 * 64 * 2
    assert q.stride(1) == k.stride(1) == (8 + 4) * 64
    kc = torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # CPU tensors
        lib.qkv_proj_append(x, torch.zeros(256, 512, dtype=torch.bfloat16), kc, kc.clone(),
                            torch.ones(4, dtype=torch.int32), 4, 2, 64)



def test_decode_bindings_validate_operands(lib):
    """The decode kernels take their element type from q and address `out`,
    the caches and seq_lens as contiguous buffers, so a mismatch would read or
    write outside them.  The bindings reject each case before any device call
    (checked here with host tensors: the checks run before the device check)."""
    import torch
    B, H_q, H_kv, d, L = 2, 8, 2, 64, 32
    q = torch.zeros(B, H_q, d, dtype=torch.bfloat16)
    kc = torch.zeros(B, L, H_kv, d, dtype=torch.bfloat16)
    lens = torch.ones(B, dtype=torch.int32)
    kp = torch.zeros(4, 16, H_kv, d, dtype=torch.bfloat16)
    bt = torch.zeros(B, 2, dtype=torch.int32)

    def both(match, **kw):
        a = dict(q=q, k=kc, v=kc, lens=lens, out=None, out_dtype=None)
        a.update(kw)
        with pytest.raises(ValueError, match=match):
            lib.gqa_attn_decode(a["q"], a["k"], a["v"], a["lens"], out=a["out"], out_dtype=a["out_dtype"])
        pk = kp if a["k"] is kc else kp.to(a["k"].dtype)
        with pytest.raises(ValueError, match=match):
            lib.gqa_attn_decode_paged(a["q"], pk, kp if a["v"] is kc else kp.to(a["v"].dtype), bt, a["lens"],
                                      out=a["out"], out_dtype=a["out_dtype"])

    both("dtype", k=kc.float(), v=kc.float())                     # caches wider than q
    both("dtype", q=q.float())                                    # fp32 q over bf16 caches
    both("seq_lens", lens=torch.ones(2 * B, dtype=torch.int32)[::2])  # not contiguous
    both("seq_lens", lens=lens.long())
    both("out", out=torch.zeros(B, H_q, d, dtype=torch.float32))  # out of q's dtype, none asked
    both("out", out=torch.zeros(B, H_q, d + 8, dtype=torch.bfloat16))
    both("out", out=torch.zeros(B, d, H_q, dtype=torch.bfloat16).transpose(1, 2))
    both("out", out=torch.zeros(B, H_q, d, dtype=torch.bfloat16), out_dtype=torch.float32)
    both("out_dtype", out_dtype=torch.float16)
    # well-formed host tensors get as far as the device check
    with pytest.raises(ValueError, match="HIP device"):
        lib.gqa_attn_decode(q, kc, kc, lens, out=torch.zeros(B, H_q, d, dtype=torch.bfloat16))

def prefill_fp8(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=None, signs=A, B=1, Lq=16, Lkv=16, H_q=4, H_kv=2, d=128, qs=512, ks=256,
             causal=1, scale=0.125, odt=BF16, ws=A, wsb=1 << 20)
    a.update(kw)
    return lib.lib.gqa_attn_prefill_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["signs"], a["B"], a["Lq"],
                                        a["Lkv"], a["H_q"], a["H_kv"], a["d"], a["qs"], a["ks"], a["causal"],
                                        a["scale"], a["odt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(signs=A + 2), INV), (dict(signs=A + 4), INV), (dict(o=A + 8), INV),
    (dict(Lkv=0), INV),
    (dict(causal=1, Lq=17, Lkv=16), INV), (dict(causal=2), INV), (dict(scale=float("nan")), INV),
    (dict(scale=-1.0), INV), (dict(qs=500), INV), (dict(qs=516), INV), (dict(ks=200), INV),
    (dict(H_q=4, H_kv=3), INV), (dict(d=64, qs=256, ks=128), UNS), (dict(d=96), UNS), (dict(odt=5), INV),
    (dict(B=-1), INV), (dict(ws=None), INV), (dict(ws=A + 8), INV), (dict(wsb=1000), INV),
])
def test_prefill_fp8_rejects(lib, kw, code):
    assert prefill_fp8(lib, **kw) == code
    assert lib.lib.mqkv_last_error() != b""


def test_prefill_fp8_empty_is_noop(lib):
    assert prefill_fp8(lib, B=0) == 0
    assert prefill_fp8(lib, Lq=0) == 0
    assert prefill_fp8(lib, signs=None, B=0) == 0


def test_prefill_fp8_workspace_query(lib):
    f = lib.prefill_fp8_workspace_bytes
    r = lambda n: (n + 255) // 256 * 256
    B, Lq, Lkv, H_q, H_kv, d = 2, 100, 130, 8, 2, 128
    nt = 3
    v_img = B * H_kv * nt * d * 72 * 2         # the fp16 V^T tiles of the bf16 prefill
    k8 = B * H_kv * nt * 64 * (d + 16)          # e4m3 K tiles, 16 padding bytes per row
    assert f(B, Lq, Lkv, H_q, H_kv, d) == r(v_img) + r(k8)
    assert f(B, Lq, Lkv, H_q, H_kv, 64) == 0    # d = 128 only
    assert f(0, Lq, Lkv, H_q, H_kv, d) == 0


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback: importing the binding where the library is not built raises
    ImportError naming the build command (checked on a copy of the package)."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "mqa_qkv_proj_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "mqa_qkv_proj_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import mqa_qkv_proj_amd"], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "build.py" in r.stderr


def test_prefill_varlen_schedule_capacity_bound(lib):
    """The schedule's list holds B + ceil(total_q / P) row blocks: enough for any
    lengths that sum to total_q, since ceil(L / P) <= L / P + 1 per sequence.
    Checked on random and extreme length mixes against the size the library
    reports (the list bytes past the 256-aligned V images)."""
    rng = np.random.default_rng(5)
    r256 = lambda n: (n + 255) // 256 * 256
    for H_q, H_kv, d, P in ((32, 4, 64, 16), (16, 4, 128, 64), (12, 2, 128, 128), (64, 2, 64, 4)):
        for _ in range(50):
            B = int(rng.integers(1, 1025))
            lens = rng.integers(0, 3000, size=B)
            if rng.random() < 0.3:  # every sequence one token past a multiple of P
                lens = (rng.integers(0, 20, size=B) * P + 1)
            total_q, L_kv = int(lens.sum()), int(max(1, lens.max()))
            blocks = int(sum((int(n) + P - 1) // P for n in lens))
            size = lib.prefill_varlen_workspace_bytes(B, L_kv, total_q, H_q, H_kv, d)
            list_bytes = size - r256(lib.prefill_workspace_bytes(B, L_kv, H_kv, d))
            assert list_bytes >= 4 * (4 + 2 * blocks), (H_q, H_kv, d, B, total_q, blocks)


def test_plain_c_caller_links_and_queries(lib, tmp_path):
    """A C99 program built against include/mqa_qkv.h and linked with the
    library: the size queries and status calls answer as through the binding,
    and an invalid call returns MQKV_ERR_INVALID with a message (no GPU work)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(r'''
#include <stdio.h>
#include "mqa_qkv.h"
int main(void) {
  printf("%d\n", mqkv_abi_version());
  printf("%zu\n", gqa_attn_prefill_workspace_bytes(2, 100, 4, 128, MQKV_BF16));
  printf("%zu\n", gqa_attn_prefill_varlen_workspace_bytes(8, 2048, 8000, 32, 4, 64));
  printf("%zu\n", gqa_attn_decode_workspace_bytes(32, 32, 8, 128, 4096, 0));
  printf("%zu\n", qkv_proj_workspace_bytes(32, 4096, 32, 8, 128, MQKV_BF16));
  mqkv_status st = gqa_attn_prefill(0, 0, 0, 0, 0, 1, 8, 8, 4, 2, 64, 512, 256, 1, 0.125f, MQKV_BF16,
                                    MQKV_BF16, 0, 0, 0);
  printf("%d %s\n", (int)st, mqkv_status_string(st));
  printf("%d\n", mqkv_last_error()[0] != 0);
  return 0;
}
''')
    exe = tmp_path / "caller"
    libdir = os.path.dirname(lib.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        "-L", libdir, "-lmqa_qkv", f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    lines = out.stdout.split("\n")
    assert int(lines[0]) == lib.lib.mqkv_abi_version()
    assert int(lines[1]) == lib.prefill_workspace_bytes(2, 100, 4, 128)
    assert int(lines[2]) == lib.prefill_varlen_workspace_bytes(8, 2048, 8000, 32, 4, 64)
    assert int(lines[3]) == lib.decode_workspace_bytes(32, 32, 8, 128, 4096, 0)
    assert int(lines[4]) == lib.qkv_proj_workspace_bytes(32, 4096, 32, 8, 128)
    assert lines[5].startswith("1 ")  # NULL operands: MQKV_ERR_INVALID
    assert lines[6] == "1"
