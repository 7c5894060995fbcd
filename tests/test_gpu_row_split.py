"""fp8 attention when fewer work-groups than half the CUs carry work (single
sequences, small batches): two work-groups then share each work item, 32 query
rows each. Every row's arithmetic is that of the unsplit launch, so on the same
segments the outputs and log-sum-exps match it bit for bit; against the oracle
they meet the usual bars. The unsplit reference keeps the same segments with a
smaller CU budget (the fixed split's segment count is capped by seg_max in
both), and ragged query counts leave some second halves without rows."""
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
