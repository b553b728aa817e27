"""CPU oracle for the fused-QKV-projection + grouped-query-attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and
this package imports nothing from the product path: the two share no code.

Everything here is plain numpy in float64 (inputs are up-cast exactly from
the fp32 / bf16 values the device receives).  Each function is the plain
definition of what it computes, with no tiling, online softmax, splitting or
reordering: the tiled and split methods reach the same result up to rounding
order, so the definition is the oracle.

Sources (page title, then the part of the page):
  * "Optimize LlamaAttention by fusing QKV projections" (transformers PR
    #40092), the review diff of LlamaAttention.forward: one qkv_proj linear
    layer, then query/key/value taken as consecutive column slices whose
    widths are num_attention_heads*head_dim, num_key_value_heads*head_dim and
    the remainder.
  * "MHA -> GQA" blog, section 3.2 (GQA attention computation): H_q query
    heads share H_kv KV heads, groups of H_q/H_kv query heads per KV head;
    the PR thread's repeat_kv remark fixes the contiguous grouping.
  * FlashAttention-3 news page, HN comment thread (the answer on what
    FlashAttention computes): attention is Softmax(Q K^T) V and is exact;
    the 1/sqrt(d) scale and the causal flag are parameters of the op.

Readings where the pages are silent (all listed in the design notes):
  * W is [hidden, N] row-major (x . W orientation), optional bias [N].
  * query head h reads KV head floor(h / (H_q/H_kv)).
  * causal masking is bottom-right aligned: query i of L_q sits at absolute
    position L_kv - L_q + i and sees keys j <= that position.
  * decode: the new token is already in the cache; sequence b attends to
    keys [0, seq_lens[b]).
  * rotary position embedding: the RoFormer rotation of consecutive pairs
    (2i, 2i+1) of every Q and K head by the angle p * theta_i, the angle
    rounded to fp32 (rope_angles); a decode token's position is
    seq_lens[b] - 1, the slot its key is appended to.

Parity pins for every function live in tests/test_oracle.py (brute force,
closed forms, invariants, a library-routine reduction); none is unpinned.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

__all__ = ["qkv_proj", "split_qkv", "attention", "attention_rows", "decode",
           "brute_attention", "kv_head_of", "kv_append", "decode_step", "decode_paged",
           "attention_varlen", "rope_angles", "rope", "qkv_proj_rope", "append_positions"]

F64 = np.float64


def qkv_proj(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Fused projection qkv = x . W (+ bias), one product for Q, K and V together.

    PR #40092 "Optimize LlamaAttention by fusing QKV projections", diff of
    LlamaAttention.forward: a single qkv_proj replaces q_proj, k_proj, v_proj.
    x: [..., hidden], w: [hidden, N], bias: [N] or None -> [..., N] float64.
    """
    x = np.asarray(x, dtype=F64)
    w = np.asarray(w, dtype=F64)
    out = x @ w
    if bias is not None:
        out = out + np.asarray(bias, dtype=F64)
    return out


def split_qkv(qkv: np.ndarray, H_q: int, H_kv: int, d: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Split the fused output by column offset into Q, K, V heads.

    PR #40092, diff of LlamaAttention.forward: query = columns [0, H_q*d),
    key = [H_q*d, (H_q+H_kv)*d), value = the rest; within a block the column
    is head*d + c.  Returns [..., H, d] views.
    """
    qe = H_q * d
    ke = qe + H_kv * d
    if qkv.shape[-1] != ke + H_kv * d:
        raise ValueError("qkv width does not match (H_q + 2*H_kv)*d")
    lead = qkv.shape[:-1]
    q = qkv[..., :qe].reshape(*lead, H_q, d)
    k = qkv[..., qe:ke].reshape(*lead, H_kv, d)
    v = qkv[..., ke:].reshape(*lead, H_kv, d)
    return q, k, v


def kv_head_of(h: int, H_q: int, H_kv: int) -> int:
    """KV head read by query head h: contiguous groups of G = H_q/H_kv heads.

    "MHA -> GQA" blog, section 3.2 (query heads of one group share one KV
    head); the grouping is the one repeat_kv produces (PR #40092 thread)."""
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return h // (H_q // H_kv)


def _softmax_rows(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax of a score block and its natural-log normaliser (LSE).

    Rows with every entry -inf cannot occur (causal needs L_q <= L_kv)."""
    m = np.max(S, axis=-1, keepdims=True)
    E = np.exp(S - m)
    s = np.sum(E, axis=-1, keepdims=True)
    return E / s, (m + np.log(s))[..., 0]


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, h: int,
                   rows: np.ndarray, causal: bool, scale: float,
                   L_q: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention for selected query rows of one (batch, head).

    softmax(scale * q K^T) V over the keys visible to each row (FlashAttention-3
    page, HN thread: attention = Softmax(QK^T)V).  q: [B, L_q, H_q, d] (only
    row indices in `rows` are read), k/v: [B, L_kv, H_kv, d].
    Returns O [len(rows), d] and LSE [len(rows)] (natural log).
    """
    H_q = q.shape[2]
    H_kv = k.shape[2]
    L_q = q.shape[1] if L_q is None else L_q
    L_kv = k.shape[1]
    g = kv_head_of(h, H_q, H_kv)
    rows = np.asarray(rows, dtype=np.int64)
    Q = np.asarray(q[b, rows, h, :], dtype=F64)
    K = np.asarray(k[b, :, g, :], dtype=F64)
    V = np.asarray(v[b, :, g, :], dtype=F64)
    S = float(scale) * (Q @ K.T)
    if causal:
        if L_q > L_kv:
            raise ValueError("causal attention needs L_q <= L_kv")
        limit = rows + (L_kv - L_q)                       # last visible key per row
        cols = np.arange(L_kv)
        S = np.where(cols[None, :] <= limit[:, None], S, -np.inf)
    P, lse = _softmax_rows(S)
    return P @ V, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
              row_block: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """Grouped-query attention for all rows.

    q [B, L_q, H_q, d], k/v [B, L_kv, H_kv, d] -> O [B, L_q, H_q, d] float64 and
    LSE [B, H_q, L_q].  H_kv = H_q is MHA, H_kv = 1 is MQA.  Rows are handled
    in blocks only to bound memory; every row takes its full softmax.
    """
    B, L_q, H_q, d = q.shape
    if k.shape[0] != B or v.shape != k.shape or k.shape[3] != d:
        raise ValueError("shape mismatch")
    O = np.empty((B, L_q, H_q, d), dtype=F64)
    LSE = np.empty((B, H_q, L_q), dtype=F64)
    for b in range(B):
        for h in range(H_q):
            for r0 in range(0, L_q, row_block):
                rows = np.arange(r0, min(L_q, r0 + row_block))
                o, l = attention_rows(q, k, v, b, h, rows, causal, scale)
                O[b, rows, h, :] = o
                LSE[b, h, rows] = l
    return O, LSE


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q: np.ndarray, cu_kv: np.ndarray,
                     causal: bool, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over a packed batch of variable-length sequences (the variable
    length case the FlashAttention-3 page lists among its further optimisations).

    Sequence b is the packed rows [cu_q[b], cu_q[b+1]) of q [total_q, H_q, d]
    and [cu_kv[b], cu_kv[b+1]) of k, v [total_kv, H_kv, d]; each is attended on
    its own as attention() attends one sequence (bottom-right causal alignment).
    A query row that sees no key has no softmax: it is given O = 0 and
    LSE = -inf.  Returns O [total_q, H_q, d], LSE [H_q, total_q].
    """
    total_q, H_q, d = q.shape
    O = np.zeros((total_q, H_q, d), dtype=F64)
    LSE = np.full((H_q, total_q), -np.inf, dtype=F64)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_kv[b]), int(cu_kv[b + 1])
        Lq, Lkv = q1 - q0, k1 - k0
        if Lq == 0 or Lkv == 0:
            continue
        qb, kb, vb = q[None, q0:q1], k[None, k0:k1], v[None, k0:k1]
        # rows that see at least one key: all of them unless causal with L_q > L_kv
        first = max(0, Lq - Lkv) if causal else 0
        rows = np.arange(first, Lq)
        for h in range(H_q):
            # a row's visible keys depend only on its offset from the end, so
            # dropping the blind leading rows keeps the alignment
            o, l = attention_rows(qb[:, first:], kb, vb, 0, h, rows - first, causal, scale)
            O[q0 + first:q1, h] = o
            LSE[h, q0 + first:q1] = l
    return O, LSE


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, seq_lens: np.ndarray,
           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step: each sequence's single query attends to its first seq_lens[b] keys.

    The per-token decode of the "MHA -> GQA" blog, section 3.1 (batched
    matrix-vector attention with per-request lengths).  q [B, H_q, d], caches
    [B, L_max, H_kv, d], seq_lens [B] in [0, L_max] -> O [B, H_q, d], LSE [B, H_q].
    A sequence with no keys (seq_lens[b] = 0) has no softmax: like a query row
    that sees no key in attention_varlen, it is given O = 0 and LSE = -inf.
    """
    B, H_q, d = q.shape
    O = np.zeros((B, H_q, d), dtype=F64)
    LSE = np.full((B, H_q), -np.inf, dtype=F64)
    for b in range(B):
        n = int(seq_lens[b])
        if not 0 <= n <= k_cache.shape[1]:
            raise ValueError("seq_lens out of range")
        if n == 0:
            continue
        kb = k_cache[b:b + 1, :n]
        vb = v_cache[b:b + 1, :n]
        qb = q[b:b + 1, None]                              # [1, 1, H_q, d]
        for h in range(H_q):
            o, l = attention_rows(qb, kb, vb, 0, h, np.array([0]), False, scale)
            O[b, h] = o[0]
            LSE[b, h] = l[0]
    return O, LSE


def kv_append(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              seq_lens: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Caches with each sequence's new token written at position seq_lens[b] - 1.

    The decode convention read from the "MHA -> GQA" blog, section 3.1: the
    token being generated attends to itself, so its key/value row is in the
    cache, as the last of the seq_lens[b] attended keys, when decode runs.
    k_cache, v_cache [B, L_max, H_kv, d]; k_new, v_new [B, H_kv, d]; rows whose
    length is outside [1, L_max] are left as they are.  Returns new arrays.
    """
    kc = np.array(k_cache, dtype=F64, copy=True)
    vc = np.array(v_cache, dtype=F64, copy=True)
    for b in range(kc.shape[0]):
        n = int(seq_lens[b])
        if 1 <= n <= kc.shape[1]:
            kc[b, n - 1] = k_new[b]
            vc[b, n - 1] = v_new[b]
    return kc, vc


def rope_angles(positions: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """Rotation angles angle[..., i] = p * theta_i for positions [...] and theta [d/2].

    The pages name the rotary embedding without fixing its arithmetic (the
    "custom op overhead" gist applies a positional step to q and k right after
    the split; the FlashAttention-3 news page, FP8 section, calls rotary a
    memory-bound step ahead of attention).  Reading: the position and theta are
    fp32 values and the angle is their fp32 product (one IEEE rounding, as an
    fp32 position table times an fp32 frequency table gives); sine and cosine
    are then taken of that fp32 angle exactly (in float64 here).
    """
    p = np.asarray(positions).astype(np.float32)            # exact for |p| < 2^24
    th = np.asarray(inv_freq, dtype=np.float32)
    return (p[..., None] * th).astype(F64)                   # float32 product, then widened


def rope(t: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """Rotary position embedding of head vectors t [..., H, d] at positions [...].

    Reading of the rotation (the pages give none): RoFormer's definition, in
    which the head dimension is a sum of d/2 planes, plane i spanned by
    components (2i, 2i+1), each turned counter-clockwise by angle p * theta_i:

        y[2i]   = t[2i] cos a - t[2i+1] sin a
        y[2i+1] = t[2i] sin a + t[2i+1] cos a,   a = rope_angles(p, theta)[i]

    The "MHA -> GQA" blog's conversion section treats the rotary embedding as
    acting on such 2-dimensional subspaces of the Q and K heads.  Returns a new
    float64 array.
    """
    t = np.asarray(t, dtype=F64)
    d = t.shape[-1]
    if d % 2 != 0 or np.asarray(inv_freq).shape != (d // 2,):
        raise ValueError("d must be even and inv_freq of length d/2")
    a = rope_angles(positions, inv_freq)[..., None, :]      # [..., 1 (heads), d/2]
    c, s = np.cos(a), np.sin(a)
    x0, x1 = t[..., 0::2], t[..., 1::2]
    y = np.empty_like(t)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def qkv_proj_rope(x: np.ndarray, w: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray,
                  H_q: int, H_kv: int, d: int, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """The fused projection (PR #40092 diff) with the rotary embedding applied to
    its Q and K heads after the bias, V untouched: the order of the "custom op
    overhead" gist's forward (projection, split, positional step on q and k).

    x [M, hidden], positions [M] -> qkv [M, N] float64.
    """
    qkv = qkv_proj(x, w, bias)
    q, k, _ = split_qkv(qkv, H_q, H_kv, d)
    out = qkv.copy()
    qo, ko, _ = split_qkv(out, H_q, H_kv, d)
    qo[...] = rope(q, positions, inv_freq)
    ko[...] = rope(k, positions, inv_freq)
    return out


def append_positions(seq_lens: np.ndarray, L_max: int) -> np.ndarray:
    """Position of each decode row's new token: the cache slot seq_lens[b] - 1 it
    is appended to (kv_append), clamped to [0, L_max - 1] for the rows that are
    not appended."""
    return np.clip(np.asarray(seq_lens, dtype=np.int64) - 1, 0, L_max - 1)


def decode_step(x: np.ndarray, w: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                seq_lens: np.ndarray, H_q: int, H_kv: int, d: int, scale: float,
                bias: Optional[np.ndarray] = None, inv_freq: Optional[np.ndarray] = None):
    """One whole decode step: project the new tokens, append their K/V, attend.

    x [B, hidden] (one new token per sequence) -> (qkv [B, N], k_cache',
    v_cache', O [B, H_q, d], LSE [B, H_q]): the fused projection (PR #40092
    diff), its column split, the append above, then decode.  With inv_freq,
    Q and K are rotated at the new token's position (append_positions) first.
    """
    if inv_freq is None:
        qkv = qkv_proj(x, w, bias)
    else:
        qkv = qkv_proj_rope(x, w, append_positions(seq_lens, k_cache.shape[1]), inv_freq, H_q, H_kv, d, bias)
    q, k, v = split_qkv(qkv[:, None, :], H_q, H_kv, d)
    kc, vc = kv_append(k_cache, v_cache, k[:, 0], v[:, 0], seq_lens)
    O, LSE = decode(q[:, 0], kc, vc, seq_lens, scale)
    return qkv, kc, vc, O, LSE


def decode_paged(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Decode over a paged cache (the PagedAttention layout the "MHA -> GQA" blog,
    section 3.2, describes as non-contiguous KV storage).

    Key j of sequence b is row j % P of page block_table[b, j // P]; a page id
    outside the pool stands for zero rows.  The pages are gathered into the
    contiguous cache they describe and decode runs on it.
    k_pages, v_pages [num_pages, P, H_kv, d]; block_table [B, pages_per_seq].
    """
    n_pages, P = k_pages.shape[0], k_pages.shape[1]
    B, pps = block_table.shape
    kc = np.zeros((B, pps * P) + k_pages.shape[2:], dtype=F64)
    vc = np.zeros_like(kc)
    for b in range(B):
        for i in range(pps):
            pg = int(block_table[b, i])
            if 0 <= pg < n_pages:
                kc[b, i * P:(i + 1) * P] = k_pages[pg]
                vc[b, i * P:(i + 1) * P] = v_pages[pg]
    return decode(q, kc, vc, seq_lens, scale)


def brute_attention(q, k, v, causal: bool, scale: float):
    """Pure-Python loop version of `attention` for tiny inputs (math.exp, math.fsum).

    Written independently of numpy's vector routines; the oracle is pinned to it."""
    B, L_q, H_q, d = (len(q), len(q[0]), len(q[0][0]), len(q[0][0][0]))
    L_kv, H_kv = len(k[0]), len(k[0][0])
    G = H_q // H_kv
    O = [[[[0.0] * d for _ in range(H_q)] for _ in range(L_q)] for _ in range(B)]
    LSE = [[[0.0] * L_q for _ in range(H_q)] for _ in range(B)]
    for b in range(B):
        for h in range(H_q):
            g = h // G
            for i in range(L_q):
                last = i + (L_kv - L_q) if causal else L_kv - 1
                scores = []
                for j in range(last + 1):
                    scores.append(scale * math.fsum(float(q[b][i][h][c]) * float(k[b][j][g][c])
                                                    for c in range(d)))
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = math.fsum(w)
                for c in range(d):
                    O[b][i][h][c] = math.fsum(w[j] * float(v[b][j][g][c]) for j in range(len(w))) / tot
                LSE[b][h][i] = mx + math.log(tot)
    return O, LSE
