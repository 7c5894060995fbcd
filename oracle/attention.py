"""Unsplit fp64 paged attention — the definition the split path must reach
(test infrastructure; see oracle/__init__.py).

What is computed [PR, Motivation and Modifications; RFC, Background]: for each
sequence of a verify/decode batch, each of its 1..4 query tokens and each query
head, softmax(q.K^T / sqrt(D)).V over the sequence's KV tokens, which live in
16- or 32-token pages reached through a page table; query heads map onto KV heads in
contiguous groups of G = Hq / Hkv (grouped-query attention).

Readings where the pages are silent (each also listed in the design notes):
  * mask: a sequence's q_i query tokens are its last q_i KV tokens, so query j
    sees keys [0, L - q + j] ("bottom-right" causal); causal=0 means all L keys;
  * softmax scale 1/sqrt(D); natural-log LSE;
  * a row with no visible key outputs exact zeros and LSE -inf;
  * head mapping g = h // G.
"""
import math

import numpy as np

from .fp8 import decode_kv


def visible_keys(L: int, q: int, j: int, causal: int) -> int:
    """Number of keys query j (0-based, of q) of a length-L sequence may see."""
    if not causal:
        return int(L)
    return int(min(max(L - q + j + 1, 0), L))


def gather_standard(kv, table_row, L: int, page_size: int):
    """Standard pages [blocks, Hkv, P, 2D] -> (K, V) as [L, Hkv, D] element codes.

    Token p sits in physical block table_row[p // P], slot p % P; per head its
    row holds K in channels [0, D) and V in [D, 2D) [RFC, Background].
    """
    D = kv.shape[-1] // 2
    p = np.arange(L)
    blocks = np.asarray(table_row, dtype=np.int64)[p // page_size]
    slots = p % page_size
    rows = kv[blocks, :, slots, :]            # [L, Hkv, 2D]
    return rows[..., :D], rows[..., D:]


def gather_shuffled(k_plane, v_plane, table_row, L: int, page_size: int):
    """Shuffled planes -> (K, V) as [L, Hkv, D] element codes.

    K plane block [Hkv, D/x, P, x]: element (token s, dim d) at [d // x, s, d % x].
    V plane block [Hkv, P/x, D, x]: element (token s, dim d) at [s // x, d, s % x].
    [RFC, Background]
    """
    x = k_plane.shape[-1]
    D = k_plane.shape[2] * x
    p = np.arange(L)
    blocks = np.asarray(table_row, dtype=np.int64)[p // page_size][:, None]
    s = (p % page_size)[:, None]
    d = np.arange(D)[None, :]
    K = k_plane[blocks, :, d // x, s, d % x]          # [L, D, Hkv]
    V = v_plane[blocks, :, s // x, d, s % x]          # [L, D, Hkv]
    return np.moveaxis(K, 2, 1), np.moveaxis(V, 2, 1)


def attend_one(qvec, K, V):
    """softmax(q.K^T/sqrt(D)).V for one query row over n keys (fp64).

    Returns (out [D], lse). n == 0 gives zeros and -inf.
    """
    qvec = np.asarray(qvec, dtype=np.float64)
    D = qvec.shape[-1]
    if K.shape[0] == 0:
        return np.zeros(D), -math.inf
    s = (K @ qvec) / math.sqrt(D)
    m = s.max()
    w = np.exp(s - m)
    tot = w.sum()
    return (w @ V) / tot, m + math.log(tot)


def sequence_kv(kv, kv_dtype, k_scale, v_scale, table_row, L, page_size,
                planes=None):
    """Gathered, dequantized fp64 (K, V) [L, Hkv, D] of one sequence."""
    if planes is None:
        Kr, Vr = gather_standard(kv, table_row, L, page_size)
    else:
        Kr, Vr = gather_shuffled(planes[0], planes[1], table_row, L, page_size)
    return decode_kv(Kr, kv_dtype, k_scale), decode_kv(Vr, kv_dtype, v_scale)


def decode_attention(q, kv, kv_dtype, table, seq_lens, cu_seqlens_q, kv_heads,
                     page_size, causal=1, k_scale=None, v_scale=None,
                     planes=None, rows=None):
    """Unsplit attention for a whole batch (or a sample of its output rows).

    q        fp64 [total_q, Hq, D] (already decoded)
    kv       standard pages of element codes, or None when `planes` is given
    planes   (k_plane, v_plane) of element codes for the shuffled layout
    rows     optional iterable of (t, h) to compute; others stay NaN
    Returns (out fp64 [total_q, Hq, D], lse fp64 [total_q, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    total_q, Hq, D = q.shape
    G = Hq // kv_heads
    out = np.full((total_q, Hq, D), np.nan)
    lse = np.full((total_q, Hq), np.nan)
    want = None
    if rows is not None:
        want = {}
        for t, h in rows:
            want.setdefault(int(t), set()).add(int(h))
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for i, L in enumerate(np.asarray(seq_lens, dtype=np.int64)):
        toks = range(int(cu[i]), int(cu[i + 1]))
        if want is not None and not any(t in want for t in toks):
            continue
        K, V = sequence_kv(kv, kv_dtype, k_scale, v_scale, table[i], int(L),
                           page_size, planes)
        qn = len(toks)
        for j, t in enumerate(toks):
            vis = visible_keys(int(L), qn, j, causal)
            for h in range(Hq):
                if want is not None and h not in want.get(t, ()):
                    continue
                g = h // G
                out[t, h], lse[t, h] = attend_one(q[t, h], K[:vis, g], V[:vis, g])
    return out, lse
