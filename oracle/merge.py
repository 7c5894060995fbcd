"""Per-segment partials and their log-sum-exp merge (test infrastructure; see
oracle/__init__.py).

[PR, Motivation/Modifications]: each work-group computes attention over one KV
segment of one sequence and KV head, and a separate reduce combines a query
token's segment results, reading only that token's segment count. Split-KV
reaches the unsplit result exactly up to rounding, which is what these
functions let the tests show on the oracle itself.

Partial format (reading): per segment the softmax-normalized output o_s over
the segment's visible keys and its natural-log LSE; segment s of a token covers
keys [s*T*P, min((s+1)*T*P, visible)).
"""
import math

import numpy as np

from .attention import attend_one, sequence_kv, visible_keys


def segment_partials(qvec, K, V, seg_tokens: int):
    """Partials (o_s, lse_s) of one query row over consecutive key segments."""
    n = K.shape[0]
    parts = []
    for start in range(0, n, seg_tokens):
        stop = min(start + seg_tokens, n)
        parts.append(attend_one(qvec, K[start:stop], V[start:stop]))
    return parts


def lse_merge(outs, lses, dim=None):
    """Merge normalized partials: out = sum_s exp(lse_s - lse) o_s,
    lse = M + ln sum_s exp(lse_s - M), M = max_s lse_s. No partial: zeros of
    length `dim`, -inf. A partial with lse -inf covers no key and has weight
    exp(-inf) = 0; when every partial is such, the sum has no term, which is
    the merge of no partial (reading: the formula's 0/0 there is taken as the
    empty merge)."""
    if len(lses) == 0:
        return np.zeros(0 if dim is None else dim), -math.inf
    lses = np.asarray(lses, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    if np.all(lses == -math.inf):
        return np.zeros(outs.shape[1] if dim is None else dim), -math.inf
    M = lses.max()
    tot = np.exp(lses - M).sum()
    lse = M + math.log(tot)
    w = np.exp(lses - lse)
    return (w[:, None] * outs).sum(axis=0), lse


def split_decode_attention(q, kv, kv_dtype, table, seq_lens, cu_seqlens_q,
                           kv_heads, page_size, pages_per_segment, causal=1,
                           k_scale=None, v_scale=None, planes=None):
    """Attention computed segment by segment and merged (no blocking beyond
    the segments themselves). `pages_per_segment` is one length for every
    sequence (the planned split) or one per sequence (the fixed split).
    Returns (out, lse, nseg per token)."""
    q = np.asarray(q, dtype=np.float64)
    total_q, Hq, D = q.shape
    G = Hq // kv_heads
    out = np.zeros((total_q, Hq, D))
    lse = np.zeros((total_q, Hq))
    nseg = np.zeros(total_q, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    per_seq = np.broadcast_to(np.asarray(pages_per_segment, dtype=np.int64), lens.shape)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for i, L in enumerate(lens):
        seg_tokens = max(int(per_seq[i]), 1) * page_size
        K, V = sequence_kv(kv, kv_dtype, k_scale, v_scale, table[i], int(L),
                           page_size, planes)
        qn = int(cu[i + 1] - cu[i])
        for j in range(qn):
            t = int(cu[i]) + j
            vis = visible_keys(int(L), qn, j, causal)
            for h in range(Hq):
                g = h // G
                parts = segment_partials(q[t, h], K[:vis, g], V[:vis, g], seg_tokens)
                nseg[t] = len(parts)
                out[t, h], lse[t, h] = lse_merge([p[0] for p in parts],
                                                 [p[1] for p in parts], D)
    return out, lse, nseg
