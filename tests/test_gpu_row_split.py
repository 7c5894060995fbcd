"""Attention when fewer work-groups than half the CUs carry work (single
sequences, small batches): two work-groups then share each work item, 32 query
rows each. For fp8 every row's arithmetic is that of the unsplit launch, so on
the same segments the outputs and log-sum-exps match it bit for bit; the
unsplit reference keeps the same segments with a smaller CU budget (the fixed
split's segment count is capped by seg_max in both), and ragged query counts
leave some second halves without rows. 16-bit KV moves to the private-ring
kernel (another summation order): checked against the oracle and for
run-to-run identity."""
import numpy as np
import pytest

from gpu_harness import TOL, compare, run_hip, run_oracle, say
from workloads import configs, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # name, seq_lens, q_lens, Hq, Hkv, layout, page_size, seg_max, split CUs, unsplit CUs
    ("bs1_64rows", [70_000], [4], 32, 2, "standard", 16, 64, 256, 128),
    ("bs1_64rows_shuf_p32", [40_001], [4], 32, 2, "shuffled", 32, 64, 256, 128),
    ("bs1_48rows", [9_000], [3], 32, 2, "standard", 16, 64, 256, 128),
    ("bs3_ragged", [5_000, 777, 12_345], [1, 4, 2], 32, 2, "standard", 16, 8, 256, 64),
    ("bs2_gqa12_rows48", [3_000, 20], [4, 3], 24, 2, "shuffled", 16, 4, 256, 24),
]


def _case(name, lens, ql, hq, hkv, layout, page, seg_max):
    cfg = gen.small_config(configs.FP8_KV, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                           page_size=page, seg_max=seg_max, causal=1, seed=31,
                           kv_dtype="fp8")
    return gen.make_case(cfg, DEV)


@pytest.mark.parametrize("spec", CASES, ids=lambda c: c[0])
def test_fixed_split_rows_shared_bit_exact(spec):
    name, lens, ql, hq, hkv, layout, page, seg_max, cus_split, cus_whole = spec
    say("row split, fixed", name)
    case = _case(name, lens, ql, hq, hkv, layout, page, seg_max)
    split = run_hip(case, fixed=True, num_cus=cus_split)
    whole = run_hip(case, fixed=True, num_cus=cus_whole, planes=split["planes"])
    assert split["tok"] == whole["tok"], "the same segments on both sides"
    assert np.array_equal(split["out_bits"], whole["out_bits"])
    assert np.array_equal(split["lse"].view(np.int64), whole["lse"].view(np.int64))
    ref_out, ref_lse = run_oracle(case)
    r = compare(split["out"], split["lse"], ref_out, ref_lse, "fp8")
    say(name, r)
    assert r["max_abs"] <= TOL["fp8"], r
    assert r["lse_err"] <= 1e-3, r


@pytest.mark.parametrize("spec", CASES, ids=lambda c: c[0])
def test_planned_split_rows_shared(spec):
    name, lens, ql, hq, hkv, layout, page, seg_max, cus_split, _ = spec
    say("row split, planned", name)
    case = _case(name, lens, ql, hq, hkv, layout, page, seg_max)
    got = run_hip(case, num_cus=cus_split)
    ref_out, ref_lse = run_oracle(case)
    r = compare(got["out"], got["lse"], ref_out, ref_lse, "fp8")
    say(name, r)
    assert r["max_abs"] <= TOL["fp8"], r
    assert r["lse_err"] <= 1e-3, r
    # two runs agree bit for bit (the fixed, deterministic order)
    again = run_hip(case, num_cus=cus_split, planes=got["planes"])
    assert np.array_equal(got["out_bits"], again["out_bits"])


def _fixed_S(bs, kvh, ncu, smax):
    """Segments per sequence of the fixed split (the library's rule)."""
    q = ncu // (bs * kvh)
    p = 1
    while p * 2 <= q:
        p *= 2
    return min(p if q >= 1 else 1, smax)


def _draw(seed):
    """A seeded launch that takes the row split: fp8, head dim 128, more than
    32 rows, and at most half the CUs busy."""
    rng = np.random.default_rng(40_000 + seed)
    while True:
        g, max_q = [(16, 3), (16, 4), (32, 2), (12, 4), (24, 2)][int(rng.integers(0, 5))]
        kvh = int(rng.choice([1, 2, 4]))
        bs = int(rng.integers(1, 5))
        smax = int(rng.integers(1, 65))
        ncu = int(rng.integers(16, 305))
        fixed = bool(rng.random() < 0.5)
        busy = (_fixed_S(bs, kvh, ncu, smax) * bs if fixed
                else min(max(ncu // kvh, bs), bs * smax)) * kvh
        if 2 * busy <= ncu:
            break
    page = int(rng.choice([16, 32]))
    lens = [int(rng.choice([0, 1, page, page + 1])) if rng.random() < 0.2
            else int(rng.integers(2, 6000)) for _ in range(bs)]
    ql = [int(rng.integers(1, max_q + 1)) for _ in range(bs)]
    ql[int(rng.integers(0, bs))] = max_q
    return dict(g=g, kvh=kvh, lens=lens, ql=ql, smax=smax, ncu=ncu, fixed=fixed, page=page,
                layout=str(rng.choice(["standard", "shuffled"])), causal=int(rng.integers(0, 2)))


@pytest.mark.parametrize("seed", range(24), ids=lambda s: f"split{s}")
def test_random_row_split(seed):
    d = _draw(seed)
    say("row split fuzz", seed, d)
    cfg = gen.small_config(configs.FP8_KV, d["lens"], d["ql"], q_heads=d["g"] * d["kvh"],
                           kv_heads=d["kvh"], layout=d["layout"], page_size=d["page"],
                           seg_max=d["smax"], causal=d["causal"], num_cus=d["ncu"],
                           seed=seed, kv_dtype="fp8")
    case = gen.make_case(cfg, DEV)
    got = run_hip(case, fixed=d["fixed"])
    ref_out, ref_lse = run_oracle(case)
    r = compare(got["out"], got["lse"], ref_out, ref_lse, "fp8")
    assert r["max_abs"] <= TOL["fp8"], r
    assert r["lse_err"] <= 1e-3, r
    if d["fixed"]:
        # the same segments without the split: a budget of exactly the busy
        # work-groups, rounded up to a power of two segments per sequence
        bs = len(d["lens"])
        S = _fixed_S(bs, d["kvh"], d["ncu"], d["smax"])
        p2 = 1
        while p2 < S:
            p2 *= 2
        whole = run_hip(case, fixed=True, num_cus=p2 * bs * d["kvh"], planes=got["planes"])
        assert got["tok"] == whole["tok"]
        assert np.array_equal(got["out_bits"], whole["out_bits"])
        assert np.array_equal(got["lse"].view(np.int64), whole["lse"].view(np.int64))


CASES16 = [
    # name, kv dtype, seq_lens, q_lens, Hq, Hkv, layout, page_size, seg_max
    ("bf16_bs1_64rows", "bf16", [50_000], [4], 32, 2, "standard", 16, 64),
    ("fp16_bs1_48rows_shuf", "fp16", [20_001], [3], 32, 2, "shuffled", 16, 64),
    ("bf16_bs3_ragged_p32", "bf16", [4_000, 33, 9_999], [2, 4, 1], 32, 2, "standard", 32, 8),
]


@pytest.mark.parametrize("fixed", [True, False], ids=["fixed", "planned"])
@pytest.mark.parametrize("spec", CASES16, ids=lambda c: c[0])
def test_16bit_rows_shared(spec, fixed):
    name, dt, lens, ql, hq, hkv, layout, page, seg_max = spec
    say("row split, 16-bit", name, "fixed" if fixed else "planned")
    cfg = gen.small_config(configs.TINY, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                           page_size=page, seg_max=seg_max, causal=1, seed=33, kv_dtype=dt,
                           num_cus=256)
    case = gen.make_case(cfg, DEV)
    got = run_hip(case, fixed=fixed)
    ref_out, ref_lse = run_oracle(case)
    r = compare(got["out"], got["lse"], ref_out, ref_lse, dt)
    say(name, r)
    assert r["max_abs"] <= TOL[dt], r
    assert r["lse_err"] <= 1e-3, r
    again = run_hip(case, fixed=fixed, planes=got["planes"])
    assert np.array_equal(got["out_bits"], again["out_bits"])
