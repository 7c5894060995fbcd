"""Pins for the oracle's segment planner and fixed split (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle
from conftest import load_golden
from workloads import configs


def _cu(q_lens):
    return [0] + list(itertools.accumulate(q_lens))


def _expand(case):
    if "seq_lens" in case:
        return case["seq_lens"], case["q_lens"]
    v, n = case["seq_lens_repeat"]
    qv, qn = case["q_lens_repeat"]
    return [v] * n, [qv] * qn


@pytest.mark.parametrize("case", load_golden("planner_hand_examples.json")["cases"],
                         ids=lambda c: c["name"])
def test_hand_derived_examples(case):
    lens, ql = _expand(case)
    plan, tok = oracle.plan_segments(lens, _cu(ql), case["kv_heads"], 16,
                                     case["num_cus"], case["seg_max"], case["causal"])
    assert plan[0] == case["T"]
    assert len(plan) == 1 + case["width"]
    items = [w for w in plan[1:] if w != -1]
    if "items" in case:
        assert items == case["items"]
        assert tok == case["tok_nseg"]
    else:
        assert len(items) == case["n_items"]
        assert set(tok) == {case["tok_nseg_all"]}
    n = len(items)
    assert all(w == -1 for w in plan[1 + n:])


def _brute_force_T(pages, cap, seg_max):
    """Every T tried, the per-sequence segments counted by walking pages."""
    best = None
    upper = max(max(pages, default=0), 1)
    for T in range(upper, 0, -1):
        counts = []
        for n in pages:
            c, covered = 0, 0
            while covered < n:
                covered += T
                c += 1
            counts.append(c)
        if sum(counts) <= cap and max(counts, default=0) <= seg_max:
            best = T
    return best if best is not None else upper


@pytest.mark.parametrize("P", [16, 32])
def test_brute_force_and_invariants_random(P):
    rng = np.random.default_rng(11 + P)
    for trial in range(300):
        bs = int(rng.integers(1, 9))
        lens = [int(v) for v in rng.integers(0, 400, size=bs)]
        if trial % 7 == 0:
            lens[0] = 0
        ql = [int(v) for v in rng.integers(1, 5, size=bs)]
        kvh = int(rng.choice([1, 2, 4, 8]))
        ncu = int(rng.integers(1, 40))
        smax = int(rng.integers(1, 9))
        causal = int(rng.integers(0, 2))
        plan, tok = oracle.plan_segments(lens, _cu(ql), kvh, P, ncu, smax, causal)
        pages = [-(-L // P) for L in lens]
        cap = ncu // kvh
        T = plan[0]
        assert T == _brute_force_T(pages, cap, smax)
        width = max(cap, bs)
        assert len(plan) == 1 + width
        items = [w for w in plan[1:] if w != -1]
        k = len(items)
        assert all(w == -1 for w in plan[1 + k:])            # -1 only after the end
        pairs = [(w >> 16, w & 0xFFFF) for w in items]
        assert len(set(pairs)) == k                           # each (seq, seg) once
        assert pairs == sorted(pairs)                          # sequence-major
        nseg = [-(-n // T) for n in pages]
        assert pairs == [(i, s) for i in range(bs) for s in range(nseg[i])]
        feasible = sum(nseg) <= cap and max(nseg) <= smax
        if feasible and T > 1:
            prev = [-(-n // (T - 1)) for n in pages]
            assert not (sum(prev) <= cap and max(prev) <= smax)   # T is the smallest
        if not feasible:
            assert T == max(max(pages), 1)
            assert all(c <= 1 for c in nseg)
        t = 0
        for i in range(bs):
            for j in range(ql[i]):
                assert tok[t] <= nseg[i]
                assert tok[t] <= max(smax, 1)
                vis = min(max(lens[i] - ql[i] + j + 1, 0), lens[i]) if causal else lens[i]
                # the count covers the visible keys and no segment beyond them
                assert tok[t] * T * P >= vis
                assert (tok[t] - 1) * T * P < vis or tok[t] == 0
                t += 1


def test_fixed_split_printed_values():
    g = load_golden("fixed_split_values.json")
    for c in g["cases"]:
        for bs in range(c["bs_from"], c["bs_to"] + 1):
            assert oracle.fixed_split_segments(bs, c["kv_heads"], g["num_cus"],
                                               g["seg_max"]) == c["segments"], (bs, c)
    lr = g["long_request"]
    assert lr["tokens"] // lr["segments"] == lr["segment_tokens"]


def test_pow2floor():
    assert [oracle.pow2floor(v) for v in [0, 1, 2, 3, 4, 7, 8, 255, 256]] == \
        [0, 1, 2, 2, 4, 4, 8, 128, 256]


def test_uniform_lengths_match_fixed_split():
    """With equal lengths and a feasible plan the planner gives every sequence the
    fixed split's segment count: the verify 16 x 119k row of the benchmark table
    shows identical times for both arms."""
    cfg = configs.UNIFORM_VERIFY
    plan, _ = oracle.plan_segments(cfg.seq_lens, _cu(cfg.q_lens), cfg.kv_heads, 16,
                                   cfg.num_cus, cfg.seg_max, 1)
    per_seq = sum(1 for w in plan[1:] if w != -1) // cfg.bs
    assert per_seq == oracle.fixed_split_segments(cfg.bs, cfg.kv_heads) == 8


def test_all_configs_plan_bounds():
    for cfg in configs.CONFIGS:
        plan, tok = oracle.plan_segments(cfg.seq_lens, _cu(cfg.q_lens), cfg.kv_heads,
                                         cfg.page_size, cfg.num_cus, cfg.seg_max,
                                         cfg.causal)
        items = [w for w in plan[1:] if w != -1]
        assert len(items) * cfg.kv_heads <= max(cfg.num_cus, cfg.bs * cfg.kv_heads)
        assert len(tok) == cfg.total_q
        assert max(tok) <= cfg.seg_max


def test_fixed_split_plan_long_request():
    """[PR, Motivation]: at bs 17-32 with one kv head the fixed split gives 8
    segments, so a 248k request runs as ~31k-token segments (page granularity)."""
    g = load_golden("fixed_split_values.json")
    lr = g["long_request"]
    lens = [lr["tokens"]] + [1000] * 19
    S, seg_pages, _ = oracle.fixed_split_plan(lens, list(range(21)), 1, 16, g["num_cus"],
                                              g["seg_max"], 1)
    assert S == lr["segments"]
    assert abs(seg_pages[0] * 16 - lr["segment_tokens"]) < 16


@pytest.mark.parametrize("seed", range(40))
def test_fixed_split_plan_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    bs = int(rng.integers(1, 40))
    kv_heads = int(rng.choice([1, 2, 4, 8]))
    num_cus = int(rng.choice([8, 64, 256, 304]))
    seg_max = int(rng.integers(1, 65))
    lens = [int(v) for v in rng.integers(0, 3000, size=bs)]
    q = [int(v) for v in rng.integers(1, 5, size=bs)]
    cu = _cu(q)
    causal = int(rng.integers(0, 2))
    S, seg_pages, tok = oracle.fixed_split_plan(lens, cu, kv_heads, 16, num_cus, seg_max,
                                                causal)
    assert S == oracle.fixed_split_segments(bs, kv_heads, num_cus, seg_max)
    t = 0
    for i, L in enumerate(lens):
        n = -(-L // 16)
        P = seg_pages[i]
        # segments [s*P, min((s+1)*P, n)) for s < S tile the pages exactly
        covered = [p for s in range(S) for p in range(s * P, min((s + 1) * P, n))]
        assert covered == list(range(n))
        for j in range(q[i]):
            vis = L if not causal else min(max(L - q[i] + j + 1, 0), L)
            assert tok[t] == sum(1 for s in range(S) if s * P * 16 < vis)
            t += 1


def test_uniform_fixed_split_equals_planned():
    """Equal lengths: the fixed split cuts every sequence exactly as the planner
    does (same T, same counts)."""
    cfg = configs.UNIFORM_VERIFY
    cu = _cu(cfg.q_lens)
    plan, tok = oracle.plan_segments(cfg.seq_lens, cu, cfg.kv_heads, 16, cfg.num_cus,
                                     cfg.seg_max, 1)
    S, seg_pages, ftok = oracle.fixed_split_plan(cfg.seq_lens, cu, cfg.kv_heads, 16,
                                                 cfg.num_cus, cfg.seg_max, 1)
    assert S == 8 and set(seg_pages) == {plan[0]} and ftok == tok


def test_hand_derived_32_token_pages():
    """num_CUs 8, kv_heads 2 (cap 4), L {160, 16, 0}, one query each, 32-token
    pages: page counts {5, 1, 0}; T = 1 needs 6 > 4 segments, T = 2 needs
    3 + 1 = 4, so T = 2 with items (0,0) (0,1) (0,2) (1,0); the counts are
    ceil(vis / 64) = {3, 1, 0}."""
    plan, tok = oracle.plan_segments([160, 16, 0], [0, 1, 2, 3], 2, 32, 8, 64, 1)
    assert plan == [2, 0, 1, 2, 65536]
    assert tok == [3, 1, 0]
