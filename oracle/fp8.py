"""FP8 attention with incoherent processing, emulated in float64.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the tests, the
smoke check and the benchmark's CPU leg may use it; it shares no code with the
HIP path.

Source: FlashAttention-3 news page, the FP8 section ("low precision and
incoherent processing"): activations carry outlier features that inflate the
quantisation error; multiplying queries and keys by a random orthogonal matrix
spreads the outliers, and a Hadamard transform with random signs does this in
O(d log d) per head.  The page measures the error on N(0,1) data with 0.1% of
the entries given a large magnitude: incoherent processing lowers it 2.6x.

Readings where the page is silent (listed in the design notes):
  * the FP8 format is e4m3 (the OCP e4m3fn encoding: finite range +-448, no
    infinities), values rounded to nearest, ties to even, saturating at +-448;
  * Q and K are quantised, V and P are not (they stay in the 16-bit path of the
    bf16 kernel); the orthogonal matrix is diag(signs) . H / sqrt(d), H the
    Sylvester Hadamard matrix;
  * scales are plain fp32 factors: one per query row (max |q'| / 448)
    and one per 64-key tile of each KV head (max |k'| over the tile / 448), so
    that S = scale * (q8 . k8) * s_q * s_k;
  * the quantisation decision is taken in fp32 (the page fixes no precision
    for it): the mapped values rounded to fp32, s = fp32(max / 448) and the
    code of the correctly rounded fp32 quotient x / s.  The map and the
    attention around it stay in fp64.

Each function follows these steps in that order; the pins are in
tests/test_oracle.py.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import attention_rows, _softmax_rows  # noqa: F401  (attention math of the oracle)

F64 = np.float64
E4M3_MAX = 448.0
KEY_TILE = 64


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of 2), scaled to be orthogonal."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of 2")
    H = np.ones((1, 1), dtype=F64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(d)


def incoherent(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x . diag(signs) . H / sqrt(d) over the last axis (the random orthogonal map)."""
    x = np.asarray(x, dtype=F64)
    return (x * np.asarray(signs, dtype=F64)) @ hadamard(x.shape[-1])


def e4m3(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value (ties to even), saturating at +-448.

    e4m3: 3 mantissa bits, so in the binade [2^e, 2^(e+1)) the values are
    multiples of 2^(e-3); below the smallest normal 2^-6 the subnormals are
    multiples of 2^-9.  |x| is clipped to the largest finite value 448 first."""
    x = np.clip(np.asarray(x, dtype=F64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(x)
    _, ex = np.frexp(a)                            # a = m * 2^ex, m in [0.5, 1): binade ex - 1
    q = np.exp2(np.maximum(ex - 1, -6) - 3.0)      # spacing of the e4m3 values around a
    return np.copysign(np.rint(a / q) * q, x)      # np.rint rounds halves to even


def _quantize(x: np.ndarray, amax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """e4m3 codes of x / s with s = amax / 448 (1 where amax = 0), both the scale
    and the quotient rounded to fp32; amax broadcasts against x."""
    x32 = np.asarray(x, dtype=F64).astype(np.float32)
    a32 = np.asarray(amax, dtype=F64).astype(np.float32)
    s32 = np.where(a32 > 0, a32 / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return e4m3((x32 / s32).astype(F64)), s32.astype(F64)


def quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row (last axis) scale max|x| / 448 (1 for an all-zero row) and e4m3(x / s)."""
    x32 = np.asarray(x, dtype=F64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    q, s = _quantize(x32, amax[..., None])
    return q, s[..., 0]


def quantize_key_tiles(k: np.ndarray, tile: int = KEY_TILE) -> Tuple[np.ndarray, np.ndarray]:
    """k [B, L, H, d]: one scale per (batch, head, tile of `tile` keys), max over the tile."""
    k32 = np.asarray(k, dtype=F64).astype(np.float32)
    B, L, H, d = k32.shape
    nt = -(-L // tile)
    k8 = np.empty(k32.shape, dtype=F64)
    s = np.empty((B, H, nt), dtype=F64)
    for t in range(nt):
        blk = k32[:, t * tile:(t + 1) * tile]                     # [B, <=tile, H, d]
        amax = np.max(np.abs(blk), axis=(1, 3))                     # [B, H]
        k8[:, t * tile:(t + 1) * tile], st = _quantize(blk, amax[:, None, :, None])
        s[:, :, t] = st[:, 0, :, 0]
    return k8, s


def attention_fp8(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
                  signs: Optional[np.ndarray] = None, tile: int = KEY_TILE):
    """Attention with Q and K quantised to e4m3 (after the incoherent map when
    `signs` is given).  q [B, L_q, H_q, d], k/v [B, L_kv, H_kv, d] ->
    O [B, L_q, H_q, d], LSE [B, H_q, L_q] (float64, V exact)."""
    qi = incoherent(q, signs) if signs is not None else np.asarray(q, dtype=F64)
    ki = incoherent(k, signs) if signs is not None else np.asarray(k, dtype=F64)
    q8, sq = quantize_rows(qi)                                     # sq [B, L_q, H_q]
    k8, sk = quantize_key_tiles(ki, tile)                          # sk [B, H_kv, nt]
    B, L_q, H_q, d = q8.shape
    L_kv, H_kv = k8.shape[1], k8.shape[2]
    G = H_q // H_kv
    O = np.empty((B, L_q, H_q, d), dtype=F64)
    LSE = np.empty((B, H_q, L_q), dtype=F64)
    key_scale = np.repeat(sk, tile, axis=2)[:, :, :L_kv]             # [B, H_kv, L_kv]
    vv = np.asarray(v, dtype=F64)
    for b in range(B):
        for h in range(H_q):
            g = h // G
            S = scale * (q8[b, :, h] @ k8[b, :, g].T) * sq[b, :, h][:, None] * key_scale[b, g][None, :]
            if causal:
                lim = np.arange(L_q) + (L_kv - L_q)
                S = np.where(np.arange(L_kv)[None, :] <= lim[:, None], S, -np.inf)
            P, lse = _softmax_rows(S)
            O[b, :, h] = P @ vv[b, :, g]
            LSE[b, h] = lse
    return O, LSE


def attention_fp8_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, h: int, rows: np.ndarray,
                       causal: bool, scale: float, signs: Optional[np.ndarray] = None, tile: int = KEY_TILE):
    """attention_fp8 for selected query rows of one (batch, head): the same
    steps, restricted to those rows and to the one KV head they read (whose K
    tile scales still span every key).  Returns O [len(rows), d], LSE [len(rows)]."""
    H_q, H_kv = q.shape[2], k.shape[2]
    L_q, L_kv = q.shape[1], k.shape[1]
    g = h // (H_q // H_kv)
    rows = np.asarray(rows, dtype=np.int64)
    qr = np.asarray(q[b, rows, h], dtype=F64)
    kg = np.asarray(k[b:b + 1, :, g:g + 1], dtype=F64)               # [1, L_kv, 1, d]
    qi = incoherent(qr, signs) if signs is not None else qr
    ki = incoherent(kg, signs) if signs is not None else kg
    q8, sq = quantize_rows(qi)
    k8, sk = quantize_key_tiles(ki, tile)
    key_scale = np.repeat(sk[0, 0], tile)[:L_kv]
    S = scale * (q8 @ k8[0, :, 0].T) * sq[:, None] * key_scale[None, :]
    if causal:
        lim = rows + (L_kv - L_q)
        S = np.where(np.arange(L_kv)[None, :] <= lim[:, None], S, -np.inf)
    P, lse = _softmax_rows(S)
    return P @ np.asarray(v[b, :, g], dtype=F64), lse
