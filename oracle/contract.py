"""The device-data contract of the plan and attention calls, checked input by
input (test infrastructure; see oracle/__init__.py).

[PR, Modifications]: the plan and the segment kernel take, per sequence, its
KV length (seq_lens), its query tokens as a range of the prefix sums
cu_seqlens_q, and its pages through its page-table row. The contract these
inputs must meet is the one the library states with those calls:
  * 0 <= L_i, and the row holds the sequence: L_i <= pt_stride * page_size;
  * cu[0] = 0, cu non-decreasing, cu[bs] = total_q;
  * every sequence has at most max_q query tokens;
  * the entries the attention reads, p < ceil(L_i / page_size) of row i, name
    blocks of the pool: 0 <= id < num_blocks.
Readings (the pages state no checker; also in the design notes): a violation
is reported as a bit per rule and the smallest offending sequence index;
cu[0] != 0 counts against sequence 0 and cu[bs] != total_q against sequence
bs - 1; a sequence with a negative query count is a prefix-sum violation, not a
query-count one; a row shorter than its length is checked over the entries it
has.
"""

BAD_LEN_NEGATIVE = 1
BAD_LEN_TABLE = 2
BAD_CU = 4
BAD_QLEN = 8
BAD_PAGE_ID = 16


def check_inputs(page_table, seq_lens, cu_seqlens_q, total_q, max_q, page_size, num_blocks):
    """(violation bits OR-ed over all sequences, smallest offending sequence
    index or -1). page_table is a 2-D [bs, pt_stride] array of block ids."""
    rows = [[int(v) for v in r] for r in page_table]
    lens = [int(v) for v in seq_lens]
    cu = [int(v) for v in cu_seqlens_q]
    bs = len(lens)
    stride = len(rows[0])
    found = {}                                  # sequence -> bits

    def report(bit, i):
        found[i] = found.get(i, 0) | bit

    for i in range(bs):
        L = lens[i]
        if L < 0:
            report(BAD_LEN_NEGATIVE, i)
        elif L > stride * page_size:
            report(BAD_LEN_TABLE, i)
        q = cu[i + 1] - cu[i]
        if q < 0 or (i == 0 and cu[0] != 0) or (i == bs - 1 and cu[bs] != total_q):
            report(BAD_CU, i)
        elif q > max_q:
            report(BAD_QLEN, i)
        if L > 0:
            read = min((L + page_size - 1) // page_size, stride)
            if any(not (0 <= rows[i][p] < num_blocks) for p in range(read)):
                report(BAD_PAGE_ID, i)
    mask = 0
    for bits in found.values():
        mask |= bits
    return mask, (min(found) if found else -1)
