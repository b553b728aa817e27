"""Python binding of libmqa_qkv.so: fused QKV projection + grouped-query attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
library (`include/mqa_qkv.h`).  PyTorch provides device memory and the current
stream.  Importing this module loads the built library and fails loudly if it
is missing (build it with `python mqa_qkv_proj_amd/build.py`); there is no
fallback implementation.

Functions mirror the C ABI:
    qkv_proj(x, w_qkv, bias=None, H_q, H_kv, d)     -> qkv [..., (H_q+2H_kv)*d]
    split_qkv(qkv, H_q, H_kv, d)                     -> (q, k, v) strided views, no copy
    gqa_attn_prefill(q, k, v, causal, scale, ...)    -> o [B, L_q, H_q, d] (, lse)
    gqa_attn_prefill_varlen(q, k, v, cu_q, cu_kv, ...) -> o [total_q, H_q, d] (, lse)
    gqa_attn_prefill_fp8(q, k, v, signs, ...)        -> o [B, L_q, H_q, d] (, lse), e4m3 scores
    gqa_attn_decode(q, k_cache, v_cache, seq_lens, ...) -> o [B, H_q, d] (, lse)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmqa_qkv.so")

MQKV_OK, MQKV_ERR_INVALID, MQKV_ERR_UNSUPPORTED, MQKV_ERR_HIP = 0, 1, 2, 3
MQKV_F32, MQKV_BF16 = 0, 1

EXPORTS = ("qkv_proj", "qkv_proj_workspace_bytes", "qkv_proj_append", "qkv_proj_rope", "qkv_proj_append_rope",
           "gqa_attn_prefill_workspace_bytes",
           "gqa_attn_prefill", "gqa_attn_decode_paged", "gqa_attn_prefill_varlen",
           "gqa_attn_prefill_varlen_workspace_bytes",
           "gqa_attn_prefill_fp8_workspace_bytes", "gqa_attn_prefill_fp8",
           "gqa_attn_decode_workspace_bytes", "gqa_attn_decode", "gqa_attn_decode_noalloc", "mqkv_status_string",
           "mqkv_last_error", "mqkv_abi_version")

DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20  # MQKV_DECODE_NOALLOC_SCRATCH_BYTES


class MqkvError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_status_string(status)}: {detail}")


class MqkvInvalid(MqkvError, ValueError):
    pass


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python mqa_qkv_proj_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.qkv_proj_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
    lib.qkv_proj_workspace_bytes.restype = sz
    lib.qkv_proj.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, vp, sz, vp]
    lib.qkv_proj.restype = i32
    lib.qkv_proj_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.qkv_proj_append.restype = i32
    lib.qkv_proj_rope.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, vp, sz, vp]
    lib.qkv_proj_rope.restype = i32
    lib.qkv_proj_append_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, vp,
                                         sz, vp]
    lib.qkv_proj_append_rope.restype = i32
    lib.gqa_attn_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.gqa_attn_prefill_workspace_bytes.restype = sz
    lib.gqa_attn_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, i64, i32,
                                     f32, i32, i32, vp, sz, vp]
    lib.gqa_attn_prefill.restype = i32
    lib.gqa_attn_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                            i64, i64, i32, f32, i32, i32, vp, sz, vp]
    lib.gqa_attn_prefill_varlen.restype = i32
    lib.gqa_attn_prefill_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.gqa_attn_prefill_varlen_workspace_bytes.restype = sz
    lib.gqa_attn_prefill_fp8_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.gqa_attn_prefill_fp8_workspace_bytes.restype = sz
    lib.gqa_attn_prefill_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, i64, i32,
                                         f32, i32, vp, sz, vp]
    lib.gqa_attn_prefill_fp8.restype = i32
    lib.gqa_attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.gqa_attn_decode_workspace_bytes.restype = sz
    lib.gqa_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, f32, i32, vp,
                                    sz, i32, i32, vp]
    lib.gqa_attn_decode.restype = i32
    lib.gqa_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, f32, i32, i32,
                                            i32, vp]
    lib.gqa_attn_decode_noalloc.restype = i32
    lib.gqa_attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64,
                                          f32, i32, vp, sz, i32, i32, vp]
    lib.gqa_attn_decode_paged.restype = i32
    lib.mqkv_status_string.argtypes = [i32]
    lib.mqkv_status_string.restype = ctypes.c_char_p
    lib.mqkv_last_error.argtypes = []
    lib.mqkv_last_error.restype = ctypes.c_char_p
    lib.mqkv_abi_version.argtypes = []
    lib.mqkv_abi_version.restype = i32
    return lib


lib = _load()


def _status_string(st: int) -> str:
    return lib.mqkv_status_string(st).decode()


def check(st: int, fn: str) -> None:
    """Raise for a non-OK status (ValueError subclass for INVALID/UNSUPPORTED)."""
    if st == MQKV_OK:
        return
    detail = lib.mqkv_last_error().decode()
    if st in (MQKV_ERR_INVALID, MQKV_ERR_UNSUPPORTED):
        raise MqkvInvalid(st, fn, detail)
    raise MqkvError(st, fn, detail)


# ----------------------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.bfloat16:
        return MQKV_BF16
    if t == torch.float32:
        return MQKV_F32
    raise TypeError(f"unsupported dtype {t} (bfloat16 or float32)")


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on a HIP device")


def _tok_stride(t, L: int, H: int, d: int, name: str) -> int:
    """Token stride of a [B, L, H, d] tensor whose rows may be views into packed qkv."""
    B = t.shape[0]
    s = t.stride()
    if s[3] != 1 or (H > 1 and s[2] != d):
        raise ValueError(f"{name}: heads must be contiguous [.., H, d] rows")
    if L > 1:
        if B > 1 and s[0] != L * s[1]:
            raise ValueError(f"{name}: batch stride must equal L * token stride")
        return s[1]
    if B > 1:
        return s[0]
    return H * d  # a single row: any stride >= H*d describes it


# ----------------------------------------------------------------------------- public API

def qkv_proj_workspace_bytes(M: int, hidden: int, H_q: int, H_kv: int, d: int, dtype_code: int = MQKV_BF16) -> int:
    return int(lib.qkv_proj_workspace_bytes(M, hidden, H_q, H_kv, d, dtype_code))


def _proj_operands(torch, x, w_qkv, H_q, H_kv, d, bias, out, workspace):
    """Checks shared by the projection calls; returns (M, hidden, out, ws_ptr, ws_bytes)."""
    hidden = x.shape[-1]
    N = (H_q + 2 * H_kv) * d
    if w_qkv.shape != (hidden, N):
        raise ValueError(f"w_qkv must be [{hidden}, {N}], got {tuple(w_qkv.shape)}")
    if not (x.is_contiguous() and w_qkv.is_contiguous()):
        raise ValueError("x and w_qkv must be contiguous")
    if w_qkv.dtype != x.dtype or (bias is not None and (bias.dtype != x.dtype or bias.shape != (N,))):
        raise ValueError("x, w_qkv and bias must share a dtype; bias is [N]")
    M = x.numel() // hidden if hidden else 0
    if out is None:
        out = torch.empty(*x.shape[:-1], N, dtype=x.dtype, device=x.device)
    elif out.shape != (*x.shape[:-1], N) or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError("out has the wrong shape, dtype or layout")
    if workspace is None:
        need = qkv_proj_workspace_bytes(M, hidden, H_q, H_kv, d, _dtype_code(x.dtype))
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return M, hidden, out, ws_ptr, ws_bytes


def _check_inv_freq(torch, inv_freq, d):
    if inv_freq.dtype != torch.float32 or inv_freq.shape != (d // 2,) or not inv_freq.is_contiguous():
        raise ValueError(f"inv_freq must be a contiguous float32 [{d // 2}] tensor")


def qkv_proj(x, w_qkv, H_q: int, H_kv: int, d: int, bias=None, out=None, workspace=None):
    """Fused projection qkv = x . W_qkv (+ bias): one GEMM for Q, K and V.

    x [..., hidden] (contiguous), w_qkv [hidden, N] row-major, N = (H_q + 2*H_kv)*d.
    Returns qkv [..., N] (or writes `out`).  `workspace` (uint8 device tensor) is
    allocated when the call can use one and none is given."""
    torch = _torch()
    _require_cuda(x, w_qkv, bias, out, workspace)
    M, hidden, out, ws_ptr, ws_bytes = _proj_operands(torch, x, w_qkv, H_q, H_kv, d, bias, out, workspace)
    st = lib.qkv_proj(x.data_ptr(), w_qkv.data_ptr(), bias.data_ptr() if bias is not None else None,
                      out.data_ptr(), M, hidden, H_q, H_kv, d, _dtype_code(x.dtype), ws_ptr, ws_bytes,
                      _stream(x.device))
    check(st, "qkv_proj")
    return out


def qkv_proj_rope(x, w_qkv, positions, inv_freq, H_q: int, H_kv: int, d: int, bias=None, out=None,
                  workspace=None):
    """qkv_proj with the rotary embedding of every Q and K head in the epilogue.

    positions: int32 [M] device tensor (one per row of x), inv_freq: float32
    [d/2] device tensor; plane i = components (2i, 2i+1) of a head turns by
    fp32(position * inv_freq[i]).  V is not rotated."""
    torch = _torch()
    _require_cuda(x, w_qkv, positions, inv_freq, bias, out, workspace)
    M, hidden, out, ws_ptr, ws_bytes = _proj_operands(torch, x, w_qkv, H_q, H_kv, d, bias, out, workspace)
    if positions.dtype != torch.int32 or positions.numel() != M or not positions.is_contiguous():
        raise ValueError(f"positions must be a contiguous int32 tensor of {M} elements")
    _check_inv_freq(torch, inv_freq, d)
    st = lib.qkv_proj_rope(x.data_ptr(), w_qkv.data_ptr(), bias.data_ptr() if bias is not None else None,
                           out.data_ptr(), positions.data_ptr(), inv_freq.data_ptr(), M, hidden, H_q, H_kv, d,
                           _dtype_code(x.dtype), ws_ptr, ws_bytes, _stream(x.device))
    check(st, "qkv_proj_rope")
    return out


def _append_call(fn_name, x, w_qkv, k_cache, v_cache, seq_lens, inv_freq, H_q, H_kv, d, bias, out, workspace):
    torch = _torch()
    _require_cuda(x, w_qkv, k_cache, v_cache, seq_lens, inv_freq, bias, out, workspace)
    if x.dim() != 2:
        raise ValueError("x must be [B, hidden]")
    B = x.shape[0]
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("the caches must be contiguous")
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[2:] != (H_kv, d) or v_cache.shape != k_cache.shape:
        raise ValueError(f"caches must be [{B}, L_max, {H_kv}, {d}]")
    if k_cache.dtype != x.dtype or v_cache.dtype != x.dtype:
        raise ValueError("x, w_qkv and the caches must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    if inv_freq is not None:
        _check_inv_freq(torch, inv_freq, d)
    _, hidden, out, ws_ptr, ws_bytes = _proj_operands(torch, x, w_qkv, H_q, H_kv, d, bias, out, workspace)
    head = (x.data_ptr(), w_qkv.data_ptr(), bias.data_ptr() if bias is not None else None, out.data_ptr(),
            k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr())
    tail = (B, hidden, H_q, H_kv, d, k_cache.shape[1], _dtype_code(x.dtype), ws_ptr, ws_bytes, _stream(x.device))
    if inv_freq is None:
        st = lib.qkv_proj_append(*head, *tail)
    else:
        st = lib.qkv_proj_append_rope(*head, inv_freq.data_ptr(), *tail)
    check(st, fn_name)
    return out


def qkv_proj_append(x, w_qkv, k_cache, v_cache, seq_lens, H_q: int, H_kv: int, d: int, bias=None, out=None,
                    workspace=None):
    """Decode-step projection that also appends the new token's K/V rows to the caches.

    x [B, hidden] (row b = sequence b's new token), caches [B, L_max, H_kv, d]
    contiguous, seq_lens [B] int32 on the device (lengths including the new
    token).  Returns qkv [B, N] like qkv_proj and writes k_cache[b, seq_lens[b]-1]
    and v_cache[b, seq_lens[b]-1] in place."""
    return _append_call("qkv_proj_append", x, w_qkv, k_cache, v_cache, seq_lens, None, H_q, H_kv, d, bias, out,
                        workspace)


def qkv_proj_append_rope(x, w_qkv, k_cache, v_cache, seq_lens, inv_freq, H_q: int, H_kv: int, d: int, bias=None,
                         out=None, workspace=None):
    """qkv_proj_append with Q and K rotated at each row's cache slot seq_lens[b] - 1
    (the rotation of qkv_proj_rope); the appended K is the rotated one."""
    return _append_call("qkv_proj_append_rope", x, w_qkv, k_cache, v_cache, seq_lens, inv_freq, H_q, H_kv, d, bias,
                        out, workspace)


def split_qkv(qkv, H_q: int, H_kv: int, d: int):
    """Q, K, V as strided views of the packed rows (column blocks Q | K | V); no copy.

    qkv [B, L, N] -> q [B, L, H_q, d], k [B, L, H_kv, d], v [B, L, H_kv, d]."""
    qe, ke = H_q * d, (H_q + H_kv) * d
    if qkv.shape[-1] != ke + H_kv * d:
        raise ValueError("qkv width does not match (H_q + 2*H_kv)*d")
    q = qkv[..., :qe].unflatten(-1, (H_q, d))
    k = qkv[..., qe:ke].unflatten(-1, (H_kv, d))
    v = qkv[..., ke:].unflatten(-1, (H_kv, d))
    return q, k, v


def prefill_workspace_bytes(B: int, L_kv: int, H_kv: int, d: int, dtype_code: int = MQKV_BF16) -> int:
    return int(lib.gqa_attn_prefill_workspace_bytes(B, L_kv, H_kv, d, dtype_code))


def prefill_varlen_workspace_bytes(B: int, max_L_kv: int, total_q: int, H_q: int, H_kv: int, d: int) -> int:
    """Workspace of a packed-batch prefill that also holds its row-block schedule
    (persistent heaviest-first workers); 0 when none is planned (B > 1024)."""
    return int(lib.gqa_attn_prefill_varlen_workspace_bytes(B, max_L_kv, total_q, H_q, H_kv, d))


def gqa_attn_prefill(q, k, v, causal: bool = True, scale: Optional[float] = None,
                     return_lse: bool = False, out_dtype=None, out=None, workspace=None):
    """Exact grouped-query attention over whole sequences.

    q [B, L_q, H_q, d], k/v [B, L_kv, H_kv, d]; token strides may be views into qkv.
    Returns o [B, L_q, H_q, d] (dtype out_dtype, default q.dtype) and, if asked,
    lse [B, H_q, L_q] float32.  `workspace` (uint8 device tensor of at least
    prefill_workspace_bytes(...) bytes) is allocated per call when not given."""
    torch = _torch()
    _require_cuda(q, k, v, out, workspace)
    B, L_q, H_q, d = q.shape
    _, L_kv, H_kv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, L_kv, H_kv, d] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    qs = _tok_stride(q, L_q, H_q, d, "q")
    ks = _tok_stride(k, L_kv, H_kv, d, "k")
    if _tok_stride(v, L_kv, H_kv, d, "v") != ks:
        raise ValueError("k and v must share a token stride")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, L_q, H_q, d, dtype=out_dtype, device=q.device)
    elif out.shape != (B, L_q, H_q, d) or not out.is_contiguous() or out.dtype != out_dtype:
        raise ValueError("out must be a contiguous [B, L_q, H_q, d] tensor of out_dtype")
    lse = torch.empty(B, H_q, L_q, dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        need = prefill_workspace_bytes(B, L_kv, H_kv, d, _dtype_code(q.dtype))
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.gqa_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr() if lse is not None else None, B, L_q, L_kv, H_q, H_kv, d,
                              qs, ks, int(bool(causal)), scale, _dtype_code(q.dtype),
                              _dtype_code(out_dtype), ws_ptr, ws_bytes, _stream(q.device))
    check(st, "gqa_attn_prefill")
    return (out, lse) if return_lse else out


def gqa_attn_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_L_q: int, max_L_kv: int,
                            causal: bool = True, scale: Optional[float] = None, return_lse: bool = False,
                            out_dtype=None, out=None, workspace=None, schedule: bool = True):
    """Exact grouped-query attention over a packed batch of variable-length sequences.

    q [total_q, H_q, d], k/v [total_kv, H_kv, d] (token strides may be views into
    qkv); cu_seqlens_q / cu_seqlens_kv [B+1] int32 on the device.  Sequence b owns
    tokens [cu[b], cu[b+1]).  Returns o [total_q, H_q, d] and, if asked,
    lse [H_q, total_q] float32.  When the workspace is allocated here, `schedule`
    sizes it for the row-block schedule (persistent heaviest-first workers);
    schedule=False sizes it for the V images only (one workgroup per row block)."""
    torch = _torch()
    _require_cuda(q, k, v, cu_seqlens_q, cu_seqlens_kv, out, workspace)
    total_q, H_q, d = q.shape
    total_kv, H_kv, _ = k.shape
    if k.shape != v.shape or k.shape[2] != d:
        raise ValueError("k and v must be [total_kv, H_kv, d] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    for name, t, H in (("q", q, H_q), ("k", k, H_kv), ("v", v, H_kv)):
        if t.stride(2) != 1 or (H > 1 and t.stride(1) != d):
            raise ValueError(f"{name}: heads must be contiguous [.., H, d] rows")
    if k.stride(0) != v.stride(0):
        raise ValueError("k and v must share a token stride")
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 [B+1] tensor")
    if cu_seqlens_q.shape != cu_seqlens_kv.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must both be [B+1]")
    B = cu_seqlens_q.shape[0] - 1
    out_dtype = q.dtype if out_dtype is None else out_dtype
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(total_q, H_q, d, dtype=out_dtype, device=q.device)
    elif out.shape != (total_q, H_q, d) or not out.is_contiguous() or out.dtype != out_dtype:
        raise ValueError("out must be a contiguous [total_q, H_q, d] tensor of out_dtype")
    lse = torch.empty(H_q, total_q, dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        need = prefill_varlen_workspace_bytes(max(B, 0), max_L_kv, total_q, H_q, H_kv, d) if schedule else 0
        if need == 0:
            need = prefill_workspace_bytes(max(B, 0), max_L_kv, H_kv, d, _dtype_code(q.dtype))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.gqa_attn_prefill_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None, cu_seqlens_q.data_ptr(),
                                     cu_seqlens_kv.data_ptr(), B, max_L_q, max_L_kv, total_q, total_kv, H_q, H_kv,
                                     d, q.stride(0), k.stride(0), int(bool(causal)), scale, _dtype_code(q.dtype),
                                     _dtype_code(out_dtype), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream(q.device))
    check(st, "gqa_attn_prefill_varlen")
    return (out, lse) if return_lse else out


def prefill_fp8_workspace_bytes(B: int, L_q: int, L_kv: int, H_q: int, H_kv: int, d: int) -> int:
    return int(lib.gqa_attn_prefill_fp8_workspace_bytes(B, L_q, L_kv, H_q, H_kv, d))


def gqa_attn_prefill_fp8(q, k, v, signs=None, causal: bool = True, scale: Optional[float] = None,
                         return_lse: bool = False, out_dtype=None, out=None, workspace=None):
    """Grouped-query attention with e4m3 scores after the incoherent map.

    q [B, L_q, H_q, d], k/v [B, L_kv, H_kv, d] bf16 (d = 128; token strides may be
    views into qkv); signs: float32 [d] device tensor of random +-1 (the
    Hadamard transform's signs), or None for plain FP8 scores.  Returns
    o [B, L_q, H_q, d] (out_dtype, default bf16) and, if asked, lse [B, H_q, L_q]."""
    torch = _torch()
    _require_cuda(q, k, v, signs, out, workspace)
    B, L_q, H_q, d = q.shape
    _, L_kv, H_kv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, L_kv, H_kv, d] matching q")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise ValueError("q, k and v must be bfloat16")
    if signs is not None and (signs.dtype != torch.float32 or tuple(signs.shape) != (d,)
                              or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 [d] tensor")
    qs = _tok_stride(q, L_q, H_q, d, "q")
    ks = _tok_stride(k, L_kv, H_kv, d, "k")
    if _tok_stride(v, L_kv, H_kv, d, "v") != ks:
        raise ValueError("k and v must share a token stride")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, L_q, H_q, d, dtype=out_dtype, device=q.device)
    elif out.shape != (B, L_q, H_q, d) or not out.is_contiguous() or out.dtype != out_dtype:
        raise ValueError("out must be a contiguous [B, L_q, H_q, d] tensor of out_dtype")
    lse = torch.empty(B, H_q, L_q, dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        need = prefill_fp8_workspace_bytes(B, L_q, L_kv, H_q, H_kv, d)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.gqa_attn_prefill_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None,
                                  signs.data_ptr() if signs is not None else None, B, L_q, L_kv, H_q, H_kv, d,
                                  qs, ks, int(bool(causal)), scale, _dtype_code(out_dtype), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream(q.device))
    check(st, "gqa_attn_prefill_fp8")
    return (out, lse) if return_lse else out


def _check_decode_operands(torch, q, caches, seq_lens, out, out_dtype, B: int, H_q: int, d: int):
    """Host checks shared by the decode calls; returns the output dtype.

    The kernels take their element type from q alone, so caches of another
    dtype, a non-contiguous seq_lens or an `out` of the wrong shape, layout or
    dtype would make them read or write outside those buffers."""
    if q.stride(2) != 1 or (H_q > 1 and q.stride(1) != d):
        raise ValueError("q rows must hold contiguous [H_q, d] heads")
    if any(c.dtype != q.dtype for c in caches):
        raise ValueError(f"the caches must have q's dtype ({q.dtype})")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"out_dtype must be bfloat16 or float32, got {out_dtype}")
    if out is not None and (tuple(out.shape) != (B, H_q, d) or not out.is_contiguous() or out.dtype != out_dtype):
        raise ValueError(f"out must be a contiguous [{B}, {H_q}, {d}] tensor of {out_dtype}")
    return out_dtype


def decode_workspace_bytes(B: int, H_q: int, H_kv: int, d: int, L_max: int, kv_split: int = 0) -> int:
    return int(lib.gqa_attn_decode_workspace_bytes(B, H_q, H_kv, d, L_max, kv_split))


def decode_workspace(B: int, H_q: int, H_kv: int, d: int, L_max: int, kv_split: int = 0, device="cuda"):
    """A decode workspace of the right size (its contents need no initialisation)."""
    torch = _torch()
    return torch.empty(max(decode_workspace_bytes(B, H_q, H_kv, d, L_max, kv_split), 16), dtype=torch.uint8,
                       device=device)


def gqa_attn_decode(q, k_cache, v_cache, seq_lens, scale: Optional[float] = None, out_dtype=None,
                    kv_split: int = 0, return_lse: bool = False, workspace=None, out=None):
    """One decode step over a contiguous KV cache.

    q [B, H_q, d] (rows may be views into qkv, i.e. any token stride), caches
    [B, L_max, H_kv, d] contiguous, seq_lens [B] int32 on the device.
    Returns o [B, H_q, d] (and lse [B, H_q] if asked)."""
    torch = _torch()
    B, H_q, d = q.shape
    _, L_max, H_kv, _ = k_cache.shape
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("caches must be [B, L_max, H_kv, d] matching q")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    out_dtype = _check_decode_operands(torch, q, (k_cache, v_cache), seq_lens, out, out_dtype, B, H_q, d)
    _require_cuda(q, k_cache, v_cache, seq_lens, workspace, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = decode_workspace_bytes(B, H_q, H_kv, d, L_max, kv_split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype, device=q.device)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=q.device) if return_lse else None
    st = lib.gqa_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                             out.data_ptr(), lse.data_ptr() if lse is not None else None, B, H_q, H_kv, d,
                             L_max, q.stride(0), scale, kv_split, workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _dtype_code(q.dtype),
                             _dtype_code(out_dtype), _stream(q.device))
    check(st, "gqa_attn_decode")
    return (out, lse) if return_lse else out


def gqa_attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: Optional[float] = None,
                          out_dtype=None, kv_split: int = 0, return_lse: bool = False, workspace=None,
                          out=None):
    """Decode over a paged KV cache: key j of sequence b is row j % page_size of
    page block_table[b, j // page_size].

    q [B, H_q, d] (any token stride), k_pages/v_pages [num_pages, page_size, H_kv, d]
    contiguous bf16, block_table [B, pages_per_seq] and seq_lens [B] int32 on the
    device.  Returns o [B, H_q, d] (and lse [B, H_q] if asked)."""
    torch = _torch()
    B, H_q, d = q.shape
    num_pages, page_size, H_kv, _ = k_pages.shape
    if v_pages.shape != k_pages.shape or k_pages.shape[3] != d:
        raise ValueError("pages must be [num_pages, page_size, H_kv, d] matching q")
    if not (k_pages.is_contiguous() and v_pages.is_contiguous() and block_table.is_contiguous()):
        raise ValueError("pages and block_table must be contiguous")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, pages_per_seq]")
    out_dtype = _check_decode_operands(torch, q, (k_pages, v_pages), seq_lens, out, out_dtype, B, H_q, d)
    _require_cuda(q, k_pages, v_pages, block_table, seq_lens, workspace, out)
    pages_per_seq = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = decode_workspace_bytes(B, H_q, H_kv, d, pages_per_seq * page_size, kv_split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype, device=q.device)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=q.device) if return_lse else None
    st = lib.gqa_attn_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                   seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
                                   B, H_q, H_kv, d, page_size, pages_per_seq, num_pages, q.stride(0), scale,
                                   kv_split, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _dtype_code(q.dtype), _dtype_code(out_dtype), _stream(q.device))
    check(st, "gqa_attn_decode_paged")
    return (out, lse) if return_lse else out
