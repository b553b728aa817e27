"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module holds no attention or projection arithmetic: it only draws random
numbers, encodes them as bfloat16 (round-to-nearest-even) and describes the
workload shapes.  Both sides receive bit-identical values from here.

Workload shapes follow the five benchmark configurations of the attention layer
(a tiny fp32 case, a TinyLlama-1.1B-shaped prefill, an MQA batched decode, a
Llama-2-7B-shaped decode sweep and a long-context prefill).  No public dataset
or trained weight is involved: every tensor is drawn from a seeded normal
distribution, so random-init weights and activations stand in for real ones.

Large tensors are drawn per leading index with an independent stream
``default_rng([seed, tag, i])`` so that any batch slice can be regenerated on
its own (the oracle checks sampled rows of full-size workloads that way).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "round_bf16", "normal", "WORKLOADS", "Workload",
    "proj_inputs", "prefill_inputs", "decode_inputs", "decode_step_q",
    "outlier_channels", "random_signs", "outlier_entries",
]

# ----------------------------------------------------------------------------- bf16 encoding

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generators never produce NaN/Inf)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exact fp32 values they encode."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded (RNE) to the nearest bf16 value, returned as fp32."""
    return bf16_to_f32(bf16_bits(a))


# ----------------------------------------------------------------------------- random draws

def normal(seed: int, tag: int, shape: Tuple[int, ...], std: float = 1.0,
           lead: Optional[range] = None) -> np.ndarray:
    """fp32 N(0, std^2) array of `shape`, one independent stream per leading index.

    `lead` selects a sub-range of the leading index (the slice is identical to
    the same slice of the full array)."""
    lead = range(shape[0]) if lead is None else lead
    out = np.empty((len(lead),) + tuple(shape[1:]), dtype=np.float32)
    for j, i in enumerate(lead):
        rng = np.random.default_rng([seed, tag, i])
        out[j] = rng.standard_normal(shape[1:], dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def outlier_channels(seed: int, tag: int, n_channels: int, frac: float = 0.001) -> np.ndarray:
    """Indices of the feature channels (columns H*d of one tensor) scaled as outliers.

    k = max(1, round(frac * n_channels)) distinct channels, seeded."""
    k = max(1, int(round(frac * n_channels)))
    rng = np.random.default_rng([seed, tag, 999_999])
    return np.sort(rng.choice(n_channels, size=k, replace=False))


def random_signs(seed: int, tag: int, n: int) -> np.ndarray:
    """n independent fair +-1 draws (fp32), seeded: the random signs of the
    incoherent map, drawn here and passed to both sides as an input."""
    rng = np.random.default_rng([seed, tag, 777_777])
    return np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)


def outlier_entries(a: np.ndarray, seed: int, tag: int, frac: float = 0.001, mult: float = 10.0) -> np.ndarray:
    """A copy of `a` with a seeded fraction `frac` of its entries (not whole
    channels) multiplied by `mult`: the outlier recipe of the FP8 error test."""
    rng = np.random.default_rng([seed, tag, 888_888])
    out = np.array(a, dtype=np.float32, copy=True)
    out[rng.random(out.shape) < frac] *= np.float32(mult)
    return out


# ----------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str                 # short id used by tests and the bench
    kind: str                 # "prefill" | "decode" | "proj"
    dtype: str                # "f32" | "bf16"
    seed: int
    B: int
    H_q: int
    H_kv: int
    d: int
    L: int = 0                # prefill sequence length (L_q = L_kv)
    hidden: int = 0           # projection input width (0: no projection)
    w_std: float = 0.0        # projection weight std
    causal: bool = True
    L_max: int = 0            # decode cache capacity
    len_lo: int = 0           # decode lengths: uniform integers in [len_lo, len_hi]
    len_hi: int = 0
    outlier_mult: float = 1.0 # >1: 0.1% of feature channels of Q, K and V scaled by this
    note: str = ""

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def N(self) -> int:
        return (self.H_q + 2 * self.H_kv) * self.d


def _mk() -> Dict[str, Workload]:
    w: List[Workload] = []
    # Tiny fp32 prefill (projection + attention), parity case.
    w.append(Workload("tiny_f32", "prefill", "f32", 1001, B=1, H_q=4, H_kv=2, d=64, L=128,
                      hidden=256, w_std=1.0 / 16.0, causal=True,
                      note="x~N(0,1); W variance 1/256 (std 1/16); no bias"))
    # TinyLlama-1.1B-shaped attention layer prefill, bf16.
    for i, L in enumerate((128, 512, 2048)):
        w.append(Workload(f"tinyllama_L{L}", "prefill", "bf16", 1002 + 100 * i, B=1, H_q=32, H_kv=4,
                          d=64, L=L, hidden=2048, w_std=0.02, causal=True,
                          note="x~N(0,1); W std 0.02"))
    # MQA batched decode, bf16 (cache grows 17..1040 over 1024 steps).
    w.append(Workload("mqa_decode", "decode", "bf16", 1003, B=8, H_q=16, H_kv=1, d=128,
                      hidden=2048, w_std=1.0 / math.sqrt(2048.0), L_max=1040, len_lo=17, len_hi=1040,
                      note="q,K,V~N(0,1); step s attends to 17+s keys; GEMM W variance 1/2048"))
    # Llama-2-7B-shaped decode sweep MHA->GQA, bf16.
    for i, hkv in enumerate((32, 8, 4)):
        w.append(Workload(f"llama7b_decode_kv{hkv}", "decode", "bf16", 1004 + 100 * i, B=32, H_q=32,
                          H_kv=hkv, d=128, hidden=4096, w_std=0.02, L_max=4096, len_lo=1024,
                          len_hi=4096, note="q,K,V~N(0,1); lengths U{1024..4096}; GEMM W std 0.02"))
    # Long-context prefill, bf16, outlier channels.
    i = 0
    for hkv in (16, 4):
        for causal in (True, False):
            w.append(Workload(f"long_kv{hkv}_{'causal' if causal else 'full'}", "prefill", "bf16",
                              1005 + 100 * i, B=2, H_q=16, H_kv=hkv, d=128, L=8192, causal=causal,
                              outlier_mult=20.0,
                              note="Q,K,V~N(0,1); 0.1% of feature channels x20"))
            i += 1
    return {x.name: x for x in w}


WORKLOADS: Dict[str, Workload] = _mk()

# Tensor tags (streams) -- distinct per logical tensor.
_T_X, _T_W, _T_Q, _T_K, _T_V, _T_LEN, _T_QSTEP, _T_B = 1, 2, 3, 4, 5, 6, 7, 8


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values the device receives, as fp32: bf16-rounded for bf16 workloads."""
    return round_bf16(a) if dtype == "bf16" else a.astype(np.float32)


def proj_inputs(wl: Workload, M: Optional[int] = None, step: int = 0,
                bias: bool = False) -> Dict[str, np.ndarray]:
    """Projection inputs: x [M, hidden], w [hidden, N] (row-major, x.W orientation).

    For decode workloads M defaults to B (one new token per sequence) and `step`
    selects the per-step activations."""
    if M is None:
        M = wl.B * wl.L if wl.kind == "prefill" else wl.B
    x = normal(wl.seed, _T_X * 1000 + step, (M, wl.hidden))
    w = normal(wl.seed, _T_W, (wl.hidden, wl.N), std=wl.w_std)
    out = {"x": _encode(x, wl.dtype), "w": _encode(w, wl.dtype)}
    if bias:
        out["bias"] = _encode(normal(wl.seed, _T_B, (1, wl.N))[0], wl.dtype)
    return out


def prefill_inputs(wl: Workload, batch: Optional[range] = None) -> Dict[str, np.ndarray]:
    """Q [B, L, H_q, d], K/V [B, L, H_kv, d] (contiguous), with the outlier channels applied."""
    batch = range(wl.B) if batch is None else batch
    res = {}
    for name, tag, H in (("q", _T_Q, wl.H_q), ("k", _T_K, wl.H_kv), ("v", _T_V, wl.H_kv)):
        a = normal(wl.seed, tag, (wl.B, wl.L, H, wl.d), lead=batch)
        if wl.outlier_mult != 1.0:
            ch = outlier_channels(wl.seed, tag, H * wl.d)
            a2 = a.reshape(a.shape[0], wl.L, H * wl.d)
            a2[:, :, ch] *= np.float32(wl.outlier_mult)
        res[name] = _encode(a, wl.dtype)
    return res


def decode_lengths(wl: Workload, step: int = 0) -> np.ndarray:
    """seq_lens [B] int32, the new token included (it already sits in the cache)."""
    if wl.name == "mqa_decode":
        return np.full(wl.B, wl.len_lo + step, dtype=np.int32)
    rng = np.random.default_rng([wl.seed, _T_LEN, 0])
    return rng.integers(wl.len_lo, wl.len_hi, size=wl.B, endpoint=True).astype(np.int32)


def decode_inputs(wl: Workload, batch: Optional[range] = None) -> Dict[str, np.ndarray]:
    """Caches [B, L_max, H_kv, d] and q [B, H_q, d] for step 0, plus seq_lens [B]."""
    batch = range(wl.B) if batch is None else batch
    k = normal(wl.seed, _T_K, (wl.B, wl.L_max, wl.H_kv, wl.d), lead=batch)
    v = normal(wl.seed, _T_V, (wl.B, wl.L_max, wl.H_kv, wl.d), lead=batch)
    lens = decode_lengths(wl)[list(batch)]
    return {"k_cache": _encode(k, wl.dtype), "v_cache": _encode(v, wl.dtype),
            "q": decode_step_q(wl, 0, batch), "seq_lens": lens}


def decode_step_q(wl: Workload, step: int, batch: Optional[range] = None) -> np.ndarray:
    batch = range(wl.B) if batch is None else batch
    q = normal(wl.seed, _T_QSTEP * 100_000 + step, (wl.B, wl.H_q, wl.d), lead=batch)
    return _encode(q, wl.dtype)


def rope_inv_freq(d: int, base: float = 10000.0) -> np.ndarray:
    """Rotary frequencies theta_i = base^(-2i/d), i < d/2, as fp32: the usual
    table of LLaMA-family models (TinyLlama and Llama-2 use base 10000).  An
    input of the projection, like its weight."""
    i = np.arange(d // 2, dtype=np.float64)
    return (base ** (-2.0 * i / d)).astype(np.float32)


def prefill_positions(B: int, L: int) -> np.ndarray:
    """Row positions of a [B*L]-row prefill batch: 0..L-1 for each sequence."""
    return np.tile(np.arange(L, dtype=np.int32), B)


def small(dtype: str, seed: int, B: int, L_q: int, L_kv: int, H_q: int, H_kv: int, d: int,
          std: float = 1.0) -> Dict[str, np.ndarray]:
    """Small random Q/K/V for parity cases that span several tiles and a ragged tail."""
    q = normal(seed, _T_Q, (B, L_q, H_q, d), std=std)
    k = normal(seed, _T_K, (B, L_kv, H_kv, d), std=std)
    v = normal(seed, _T_V, (B, L_kv, H_kv, d), std=std)
    return {"q": _encode(q, dtype), "k": _encode(k, dtype), "v": _encode(v, dtype)}
