"""Pins of the oracle's contract checker (oracle/contract.py): one hand-derived
case per rule, each at its boundary, the bits combined, and the bench
workloads' own inputs (which meet the contract by construction).

The contract is the one stated with the plan and attention calls: 0 <= L_i <=
pt_stride * page_size; cu[0] = 0, cu non-decreasing, cu[bs] = total_q; at most
max_q query tokens per sequence; the entries p < ceil(L_i / page_size) of row i
name blocks in [0, num_blocks).
"""
import numpy as np
import pytest

import oracle
from workloads import configs, gen

NEG, TABLE, CU, QLEN, PAGE = 1, 2, 4, 8, 16


def chk(table, lens, cu, total_q=None, max_q=4, page_size=16, num_blocks=8):
    total_q = cu[-1] if total_q is None else total_q
    return oracle.check_inputs(np.array(table), lens, cu, total_q, max_q, page_size, num_blocks)


# two sequences, rows of two entries: 17 tokens read entries 0 and 1, 32 tokens
# (exactly the row's capacity of 2 * 16) read entries 0 and 1
VALID = dict(table=[[0, 1], [2, 3]], lens=[17, 32], cu=[0, 1, 3])


def test_valid_input_passes():
    assert chk(**VALID) == (0, -1)


def test_length_at_row_capacity_passes_one_more_token_fails():
    assert chk([[0, 1], [2, 3]], [17, 33], [0, 1, 3]) == (TABLE, 1)


def test_negative_length():
    assert chk([[0, 1], [2, 3]], [-1, 32], [0, 1, 3]) == (NEG, 0)


def test_empty_sequence_reads_nothing():
    # L = 0 reads no entry, so a garbage row is fine
    assert chk([[0, 1], [-5, 99]], [17, 0], [0, 1, 3]) == (0, -1)


def test_prefix_sums_start_at_zero():
    assert chk([[0, 1], [2, 3]], [17, 32], [1, 1, 3], total_q=3) == (CU, 0)


def test_prefix_sums_end_at_total_q():
    assert chk([[0, 1], [2, 3]], [17, 32], [0, 1, 3], total_q=4) == (CU, 1)


def test_decreasing_prefix_sums_are_not_a_query_count_violation():
    # sequence 1 has 2 - 5 = -3 query tokens: a prefix-sum violation only;
    # sequence 0's 5 tokens exceed max_q = 4
    assert chk([[0, 1], [2, 3]], [17, 32], [0, 5, 2], total_q=2) == (CU | QLEN, 0)


def test_query_count_above_max_q():
    assert chk([[0, 1], [2, 3]], [17, 32], [0, 1, 6]) == (QLEN, 1)
    assert chk([[0, 1], [2, 3]], [17, 32], [0, 1, 5]) == (0, -1)      # 4 = max_q


def test_page_ids_read_range_only():
    # 17 tokens read entries 0 and 1; 16 tokens read entry 0 alone
    assert chk([[0, 8], [2, 3]], [17, 32], [0, 1, 3]) == (PAGE, 0)    # 8 = num_blocks
    assert chk([[0, 8], [2, 3]], [16, 32], [0, 1, 3]) == (0, -1)
    assert chk([[0, 1], [-1, 3]], [17, 32], [0, 1, 3]) == (PAGE, 1)
    assert chk([[0, 1], [2, 7]], [17, 32], [0, 1, 3]) == (0, -1)      # 7 = num_blocks - 1


def test_thirty_two_token_pages():
    # 33 tokens of 32-token pages read entries 0 and 1; 32 tokens read entry 0
    assert chk([[0, 9], [1, 2]], [33, 64], [0, 1, 2], page_size=32) == (PAGE, 0)
    assert chk([[0, 9], [1, 2]], [32, 64], [0, 1, 2], page_size=32) == (0, -1)
    assert chk([[0, 1], [2, 3]], [33, 65], [0, 1, 2], page_size=32) == (TABLE, 1)


def test_short_row_is_checked_over_the_entries_it_has():
    # 40 tokens need 3 entries, the row has 2: a length violation, and the two
    # entries that exist are still checked
    assert chk([[0, 1], [2, 3]], [17, 40], [0, 1, 3]) == (TABLE, 1)
    assert chk([[0, 1], [2, -3]], [17, 40], [0, 1, 3]) == (TABLE | PAGE, 1)


def test_bits_combine_and_the_first_sequence_is_reported():
    table = [[0, 1], [2, 3], [9, 4], [5, 6]]
    lens = [17, -4, 20, 31]
    cu = [0, 1, 2, 8, 9]
    assert chk(table, lens, cu) == (NEG | PAGE | QLEN, 1)


@pytest.mark.parametrize("cfg", configs.CONFIGS + configs.EXTRA + configs.BS1,
                         ids=lambda c: c.name)
def test_bench_workloads_meet_the_contract(cfg):
    meta = gen.layout_metadata(cfg)
    got = oracle.check_inputs(np.asarray(meta["table"]), meta["seq_lens"], meta["cu"],
                              cfg.total_q, cfg.max_q, cfg.page_size, meta["pool"])
    assert got == (0, -1)
