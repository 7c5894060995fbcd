"""Randomised attention parity: every axis of the attention call drawn at once.

The enumerated cases in test_gpu_parity.py and test_gpu_head_dims.py pick one
kernel route at a time; here each seeded case draws the element type (bf16,
fp16, fp8 e4m3fn), layout (standard or shuffled), page size (16 or 32),
head dim (64, 128, 256), GQA group and query tokens (up to 64 rows), causal
or not, planned or fixed split, the fp8 claim order, the work-list budget and
seg_max, and ragged lengths with empty, one-token and page-boundary
sequences. Outputs and log-sum-exps are compared with the fp64 oracle at the
usual bars; the plan (or the fixed split's per-token counts) bit-exact.
"""
import numpy as np
import pytest

import oracle
from gpu_harness import compare, oracle_plan, run_hip, run_oracle, say
from workloads import configs, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 160


def _draw(seed):
    rng = np.random.default_rng(10_000 + seed)
    dt = str(rng.choice(["bf16", "fp16", "fp8"]))
    layout = str(rng.choice(["standard", "shuffled"]))
    page_size = int(rng.choice([16, 32]))
    head_dim = int(rng.choice([64, 128, 256]))
    kvh = int(rng.choice([1, 2, 4, 8]))
    max_q = int(rng.integers(1, 5))
    g = int(rng.choice([g for g in (1, 2, 4, 8, 16) if g * max_q <= 64]))
    bs = int(rng.integers(1, 7))
    special = [0, 1, page_size - 1, page_size, page_size + 1, 2 * page_size + 1]
    lens = [int(rng.choice(special)) if rng.random() < 0.3 else int(rng.integers(2, 3000))
            for _ in range(bs)]
    ql = [int(rng.integers(1, max_q + 1)) for _ in range(bs)]
    ql[int(rng.integers(0, bs))] = max_q
    causal = int(rng.integers(0, 2))
    fixed = bool(rng.random() < 0.3)
    claim = dt == "fp8" and bool(rng.random() < 0.5)
    ncu = int(rng.integers(4, 305))
    smax = int(rng.integers(1, 65))
    return dict(dt=dt, layout=layout, page_size=page_size, head_dim=head_dim, kvh=kvh,
                g=g, lens=lens, ql=ql, causal=causal, fixed=fixed, claim=claim, ncu=ncu,
                smax=smax)


@pytest.mark.parametrize("seed", range(N_CASES), ids=lambda s: f"fuzz{s}")
def test_random_attention_matches_oracle(seed):
    d = _draw(seed)
    say("fuzz", seed, d)
    base = configs.FP8_KV if d["dt"] == "fp8" else configs.TINY
    cfg = gen.small_config(base, d["lens"], d["ql"], q_heads=d["g"] * d["kvh"],
                           kv_heads=d["kvh"], head_dim=d["head_dim"], layout=d["layout"],
                           causal=d["causal"], num_cus=d["ncu"], seg_max=d["smax"],
                           seed=seed, page_size=d["page_size"], kv_dtype=d["dt"])
    case = gen.make_case(cfg, DEV)
    hip = run_hip(case, fixed=d["fixed"], claim=d["claim"])
    if d["fixed"]:
        _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                                 cfg.kv_heads, cfg.page_size, cfg.num_cus,
                                                 cfg.seg_max, cfg.causal)
        assert hip["tok"] == want_tok
    else:
        wp, wt = oracle_plan(case)
        assert hip["plan"] == wp and hip["tok"] == wt
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, cfg.kv_dtype)
    say("fuzz", seed, r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r
