"""The device-data contract checker (skv_check_inputs) against the oracle's
(oracle/contract.py), bit-exact: the bench workloads' inputs pass; hand cases
of every rule; and random batches with planted violations of every kind,
short rows (one thread per row) and long ones (one wave per row), more
sequences than the work-group has threads."""
import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_amd as skv
from gpu_harness import say
from workloads import configs, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _device_check(table, lens, cu, total_q, max_q, page_size, num_blocks):
    t = torch.as_tensor(np.ascontiguousarray(table, dtype=np.int32), device=DEV)
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32), device=DEV)
    c = torch.as_tensor(np.asarray(cu, dtype=np.int32), device=DEV)
    res = skv.check_inputs(t, sl, c, total_q, max_q, num_blocks, page_size=page_size)
    torch.cuda.synchronize()
    r = res.cpu().tolist()
    return r[0], r[1]


def _both(table, lens, cu, total_q, max_q, page_size, num_blocks):
    want = oracle.check_inputs(np.asarray(table), lens, cu, total_q, max_q, page_size,
                               num_blocks)
    got = _device_check(table, lens, cu, total_q, max_q, page_size, num_blocks)
    return got, want


@pytest.mark.parametrize("cfg", configs.CONFIGS + configs.EXTRA + configs.BS1,
                         ids=lambda c: c.name)
def test_bench_workloads_pass(cfg):
    meta = gen.layout_metadata(cfg)
    got = _device_check(meta["table"], meta["seq_lens"], meta["cu"], cfg.total_q, cfg.max_q,
                        cfg.page_size, meta["pool"])
    assert got == (0, -1)


HAND = [
    # table, lens, cu, total_q, max_q, page_size, num_blocks
    ([[0, 1], [2, 3]], [17, 32], [0, 1, 3], 3, 4, 16, 8),          # valid
    ([[0, 1], [2, 3]], [17, 33], [0, 1, 3], 3, 4, 16, 8),          # row too short
    ([[0, 1], [2, 3]], [-1, 32], [0, 1, 3], 3, 4, 16, 8),          # negative length
    ([[0, 1], [-5, 99]], [17, 0], [0, 1, 3], 3, 4, 16, 8),         # empty: nothing read
    ([[0, 1], [2, 3]], [17, 32], [1, 1, 3], 3, 4, 16, 8),          # cu[0] != 0
    ([[0, 1], [2, 3]], [17, 32], [0, 1, 3], 4, 4, 16, 8),          # cu[bs] != total_q
    ([[0, 1], [2, 3]], [17, 32], [0, 5, 2], 2, 4, 16, 8),          # decreasing + q > max_q
    ([[0, 8], [2, 3]], [17, 32], [0, 1, 3], 3, 4, 16, 8),          # id = num_blocks, read
    ([[0, 8], [2, 3]], [16, 32], [0, 1, 3], 3, 4, 16, 8),          # id = num_blocks, unread
    ([[0, 9], [1, 2]], [33, 64], [0, 1, 2], 2, 4, 32, 8),          # 32-token pages
    ([[0, 1], [2, -3]], [17, 40], [0, 1, 3], 3, 4, 16, 8),         # short row, bad entry
    ([[0, 1], [2, 3], [9, 4], [5, 6]], [17, -4, 20, 31], [0, 1, 2, 8, 9], 9, 4, 16, 8),
]


@pytest.mark.parametrize("case", HAND, ids=range(len(HAND)))
def test_hand_cases(case):
    got, want = _both(*case)
    assert got == want, (got, want)


def _valid_batch(rng, bs, page_size, long_rows):
    lens = rng.integers(0, 2000, size=bs)
    if long_rows:
        k = max(1, bs // 8)
        lens[rng.choice(bs, size=k, replace=False)] = rng.integers(64 * page_size + 1, 100_000,
                                                                   size=k)
    q = rng.integers(1, 5, size=bs)
    n = (lens + page_size - 1) // page_size
    stride = max(int(n.max()), 1) + int(rng.integers(0, 3))
    num_blocks = int(n.sum()) + 16
    ids = rng.permutation(num_blocks)
    table = np.full((bs, stride), -7, dtype=np.int64)       # unread entries: garbage
    off = 0
    for i in range(bs):
        table[i, :n[i]] = ids[off: off + n[i]]
        off += int(n[i])
    cu = np.concatenate([[0], np.cumsum(q)])
    return table, lens, cu, int(cu[-1]), 4, num_blocks


def _plant(rng, table, lens, cu, total_q, max_q, num_blocks, page_size):
    bs, stride = table.shape
    kind = int(rng.integers(0, 7))
    i = int(rng.integers(0, bs))
    if kind == 0:
        lens[i] = -int(rng.integers(1, 1000))
    elif kind == 1:
        lens[i] = stride * page_size + int(rng.integers(1, 100))
    elif kind == 2 and bs > 1:
        cu[i + 1] = cu[i] - int(rng.integers(1, 3))
    elif kind == 3:
        cu[i + 1:] += 5                                  # sequence i gets 5 more tokens
        total_q += 5
    elif kind == 4:
        n = min((max(int(lens[i]), 0) + page_size - 1) // page_size, stride)
        if n > 0:
            table[i, int(rng.integers(0, n))] = int(rng.choice([-1, num_blocks,
                                                                num_blocks + 1000]))
    elif kind == 5:
        total_q += 1
    else:
        cu[0] = 1
    return table, lens, cu, total_q, max_q


@pytest.mark.parametrize("trial", range(40))
def test_planted_violations_match_oracle(trial):
    rng = np.random.default_rng(900 + trial)
    bs = int(rng.choice([1, 3, 17, 300, 1100]))
    page_size = int(rng.choice([16, 32]))
    table, lens, cu, total_q, max_q, num_blocks = _valid_batch(rng, bs, page_size,
                                                               long_rows=trial % 2 == 0)
    for _ in range(int(rng.integers(0, 4))):
        table, lens, cu, total_q, max_q = _plant(rng, table, lens, cu, total_q, max_q,
                                                 num_blocks, page_size)
    say("check", trial, bs, page_size)
    got, want = _both(table, lens.tolist(), cu.tolist(), total_q, max_q, page_size,
                      num_blocks)
    assert got == want, (trial, got, want)
