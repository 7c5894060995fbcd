"""Full-size workloads on the GPU: the plan bit-exact, the shuffled planes
bit-exact on sampled blocks, and the attention output on sampled (token, head)
rows against the oracle, in the same launch configuration the benchmark
times. Whole-output properties (finite everywhere; exact zeros where a token
sees no key) are checked on every row."""
import gc

import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_amd as skv
from gpu_harness import compare, oracle_plan, run_hip, run_oracle, say
from workloads import configs, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _free():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _sample_rows(cfg, seqs, n_heads=6, seed=0):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(cfg.q_lens)])
    rows = []
    for i in seqs:
        for t in range(cu[i], cu[i + 1]):
            for h in sorted(rng.choice(cfg.q_heads, size=min(n_heads, cfg.q_heads), replace=False)):
                rows.append((int(t), int(h)))
    return rows


SAMPLES = {
    "uniform_verify": [0, 7, 15],
    "agentic_skew": [0, 1, 2, 3, 4, 5, 19],
    "fp8_kv": [0, 15, 16, 29, 48, 63],
    "shuffled_decode": [0, 64, 127],
    "uniform_verify_fp8": [0, 15],
    "agentic_skew_fp8": [0, 3, 4, 19],
    "uniform_verify_fp16": [0, 15],
    "uniform_verify_d64": [0, 15],
    "uniform_verify_d256": [0, 15],
}


@pytest.mark.parametrize("name", list(SAMPLES), ids=str)
def test_full_size_sampled(name):
    cfg = configs.BY_NAME[name]
    say("fullsize", name, "generating")
    case = gen.make_case(cfg, DEV)
    torch.cuda.synchronize()
    say("fullsize", name, "hip")
    hip = run_hip(case)
    wp, wt = oracle_plan(case)
    assert hip["plan"] == wp and hip["tok"] == wt
    if cfg.layout == "shuffled":
        say("fullsize", name, "shuffle check")
        kp, vp = hip["planes"]
        rng = np.random.default_rng(1)
        blocks = sorted(rng.choice(case.num_pool_blocks, size=48, replace=False).tolist())
        std_h = gen.raw_u16(case.kv[blocks])
        wk, wv = oracle.shuffle_blocks(std_h)
        assert np.array_equal(gen.raw_u16(kp[blocks]), wk)
        assert np.array_equal(gen.raw_u16(vp[blocks]), wv)
        del kp, vp
    hip.pop("planes")
    # whole-output properties
    assert np.all(np.isfinite(hip["out"]))
    cu = np.concatenate([[0], np.cumsum(cfg.q_lens)])
    for i, L in enumerate(cfg.seq_lens):
        qn = cfg.q_lens[i]
        for j in range(qn):
            vis = oracle.visible_keys(L, qn, j, cfg.causal)
            if vis == 0:
                assert np.all(hip["out"][cu[i] + j] == 0)
                assert np.all(hip["lse"][cu[i] + j] == -np.inf)
    say("fullsize", name, "oracle")
    rows = _sample_rows(cfg, SAMPLES[name])
    ref_out, ref_lse = run_oracle(case, rows=rows)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, cfg.kv_dtype, rows=rows)
    say("fullsize", name, r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r


def test_full_size_convert_round_trip():
    """The shuffled-decode batch's pool (65,544 blocks x 8 heads, 4.3 GB of
    bf16 pages) received as byte halves, converted in place: sampled blocks
    bit-exact against the oracle, every block equal to the out-of-place repack,
    and the inverse restoring every byte."""
    cfg = configs.BY_NAME["shuffled_decode"]
    say("fullsize convert", "generating")
    case = gen.make_case(cfg, DEV)
    B, H = case.kv.shape[0], cfg.kv_heads
    x = 8
    half = H * 16 * 128
    flat = case.kv.view(torch.int16).view(B, 2 * half)
    kp = flat[:, :half].contiguous().view(B, H, 128 // x, 16, x)
    vp = flat[:, half:].contiguous().view(B, H, 16 // x, 128, x)
    k0, v0 = kp.clone(), vp.clone()
    torch.cuda.synchronize()
    say("fullsize convert", "to_shuffled")
    skv.kv_page_convert(kp, vp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    blocks = sorted(rng.choice(B, size=32, replace=False).tolist())
    std_h = gen.raw_u16(case.kv[blocks])
    wk, wv = oracle.shuffle_blocks(std_h)
    assert np.array_equal(gen.raw_u16(kp[blocks]), wk)
    assert np.array_equal(gen.raw_u16(vp[blocks]), wv)
    say("fullsize convert", "vs out-of-place repack")
    ks, vs = skv.kv_page_shuffle(case.kv)
    assert torch.equal(kp, ks.view(torch.int16)) and torch.equal(vp, vs.view(torch.int16))
    del ks, vs, case
    say("fullsize convert", "to_standard")
    skv.kv_page_convert(kp, vp, direction="to_standard")
    torch.cuda.synchronize()
    assert torch.equal(kp, k0) and torch.equal(vp, v0)


@pytest.mark.parametrize("name", ["agentic_skew", "fp8_kv"], ids=str)
def test_full_size_fixed_split(name):
    """The fixed split (no plan) on a full-size skewed batch: per-token counts
    bit-exact, sampled rows against the oracle."""
    cfg = configs.BY_NAME[name]
    say("fullsize fixed", name, "generating")
    case = gen.make_case(cfg, DEV)
    hip = run_hip(case, fixed=True)
    hip.pop("planes")
    _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                             cfg.kv_heads, 16, cfg.num_cus, cfg.seg_max,
                                             cfg.causal)
    assert hip["tok"] == want_tok
    assert np.all(np.isfinite(hip["out"]))
    rows = _sample_rows(cfg, SAMPLES[name], n_heads=4, seed=9)
    ref_out, ref_lse = run_oracle(case, rows=rows)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, cfg.kv_dtype, rows=rows)
    say("fullsize fixed", name, r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r
