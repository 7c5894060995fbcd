"""Length-aware segment planner and the fixed split it replaces (test
infrastructure; see oracle/__init__.py).

[PR, Modifications]: one segment length T is chosen from the batch's sequence
lengths — the smallest T for which the total segment count stays within
num_CUs / kv_heads and no sequence needs more than seg_max segments — and a work
list of (sequence << 16 | segment) words is written, padded with -1, together
with a per-query-token segment count that the reduce reads. The kernel takes
the tiles per segment from the first plan word.

[PR, Motivation]: the fixed split gives every sequence
max(1, min(64, pow2floor(256 / (bs * kv_heads)))) segments.

Readings (pages silent; also in the design notes):
  * T counts pages ("tiles" = pages of the given size, 16 or 32 tokens), searched over all integers
    1..max(max_pages, 1); feasibility is monotone in T, so the smallest is unique;
  * no feasible T (more non-empty sequences than num_CUs // kv_heads): T is the
    longest sequence's page count, i.e. one segment per non-empty sequence;
  * num_CUs / kv_heads is floored; the work list has max(that, bs) entries;
  * work list order: sequence-major, segments ascending;
  * per-token count: the number of the sequence's segments that hold at least
    one key the token may see, ceil(visible / (T * P)).
"""
import numpy as np

from .attention import visible_keys


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def plan_segments(seq_lens, cu_seqlens_q, kv_heads, page_size, num_cus, seg_max,
                  causal=1):
    """Returns (plan, tok_nseg) as Python int lists.

    plan[0] = T (pages per segment); plan[1 + k] = (i << 16) | s for the k-th
    work item, -1 past the last; len(plan) = 1 + max(num_cus // kv_heads, bs).
    tok_nseg[t] = segments of t's sequence holding keys t may see.
    """
    lens = [int(v) for v in seq_lens]
    bs = len(lens)
    # step 1: pages per sequence, the CU budget per kv head, the longest sequence
    pages = [_ceil_div(L, page_size) for L in lens]
    cap = num_cus // kv_heads
    longest = max(pages) if pages else 0

    # step 2: feasibility of a candidate segment length (numpy only to keep
    # the upward scan affordable for 10^5-page sequences)
    pages_np = np.asarray(pages, dtype=np.int64)

    def feasible(T):
        segs = -(-pages_np // T)
        return int(segs.sum()) <= cap and int(segs.max(initial=0)) <= seg_max

    # step 3: smallest feasible T, scanning upward; fallback when none is
    upper = max(longest, 1)
    T = None
    for cand in range(1, upper + 1):
        if feasible(cand):
            T = cand
            break
    if T is None:
        T = upper

    # step 4: segments per sequence and the sequence-major work list
    nseg = [_ceil_div(n, T) for n in pages]
    items = []
    for i in range(bs):
        for s in range(nseg[i]):
            items.append((i << 16) | s)

    # step 5: pad with -1 to the work-list capacity
    width = max(cap, bs)
    assert len(items) <= width
    plan = [T] + items + [-1] * (width - len(items))

    # step 6: per-query-token segment counts
    tok_nseg = []
    for i in range(bs):
        qn = int(cu_seqlens_q[i + 1]) - int(cu_seqlens_q[i])
        for j in range(qn):
            vis = visible_keys(lens[i], qn, j, causal)
            tok_nseg.append(_ceil_div(vis, T * page_size))
    return plan, tok_nseg


def pow2floor(v: int) -> int:
    """Largest power of two <= v; 0 for v <= 0."""
    v = int(v)
    if v <= 0:
        return 0
    p = 1
    while p * 2 <= v:
        p *= 2
    return p


def fixed_split_segments(bs: int, kv_heads: int, num_cus: int = 256,
                         seg_max: int = 64) -> int:
    """Segments per sequence under the fixed split [PR, Motivation]."""
    return max(1, min(seg_max, pow2floor(num_cus // (bs * kv_heads))))


def fixed_split_plan(seq_lens, cu_seqlens_q, kv_heads, page_size, num_cus=256,
                     seg_max=64, causal=1):
    """The fixed split as a segmentation [PR, Motivation: every sequence gets the
    same number of KV segments; Modifications: bs == 1 runs this split].

    Reading (the pages give the count, not the boundaries): sequence i's n_i
    pages are cut into S contiguous segments of ceil(n_i / S) pages, S =
    fixed_split_segments(...), the last shorter and trailing ones empty when
    n_i < S. Returns (S, seg_pages per sequence, tok_nseg), tok_nseg[t] being
    the number of t's segments that hold at least one key t may see.
    """
    lens = [int(v) for v in seq_lens]
    bs = len(lens)
    S = fixed_split_segments(bs, kv_heads, num_cus, seg_max)
    seg_pages = [_ceil_div(_ceil_div(L, page_size), S) for L in lens]
    tok_nseg = []
    for i in range(bs):
        qn = int(cu_seqlens_q[i + 1]) - int(cu_seqlens_q[i])
        for j in range(qn):
            vis = visible_keys(lens[i], qn, j, causal)
            tok_nseg.append(_ceil_div(vis, seg_pages[i] * page_size) if vis > 0 else 0)
    return S, seg_pages, tok_nseg
