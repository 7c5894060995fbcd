"""GPU parity of the HIP path (through the C ABI) against the CPU oracle."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_amd as skv
from gpu_harness import TOL, compare, oracle_plan, run_hip, run_oracle, say
from workloads import configs, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skv.load()
    yield
    torch.cuda.synchronize()


def _cu(q):
    return [0] + list(itertools.accumulate(q))


# ---- planner: bit-exact ------------------------------------------------------

@pytest.mark.parametrize("cfg", configs.CONFIGS, ids=lambda c: c.name)
def test_plan_bit_exact_on_configs(cfg):
    say("plan", cfg.name)
    meta = gen.layout_metadata(cfg)
    sl = torch.as_tensor(meta["seq_lens"], device=DEV)
    cu = torch.as_tensor(meta["cu"], device=DEV)
    plan, tok = skv.plan_build(sl, cu, cfg.total_q, cfg.kv_heads, cfg.num_cus, cfg.seg_max,
                               cfg.causal)
    want_plan, want_tok = oracle.plan_segments(cfg.seq_lens, meta["cu"], cfg.kv_heads, 16,
                                               cfg.num_cus, cfg.seg_max, cfg.causal)
    assert plan.cpu().tolist() == want_plan
    assert tok.cpu().tolist() == want_tok


def test_plan_bit_exact_fuzz():
    rng = np.random.default_rng(2024)
    for trial in range(120):
        bs = int(rng.integers(1, 301))
        big = trial % 3 == 0
        lens = rng.integers(0, 300_001 if big else 3000, size=bs)
        lens[rng.random(bs) < 0.1] = 0
        ql = rng.integers(1, 5, size=bs)
        kvh = int(rng.choice([1, 2, 4, 8]))
        ncu = int(rng.integers(4, 305))
        smax = int(rng.integers(1, 65))
        causal = int(rng.integers(0, 2))
        sl = torch.as_tensor(lens.astype(np.int32), device=DEV)
        cu_h = np.array(_cu(ql.tolist()), dtype=np.int32)
        cu = torch.as_tensor(cu_h, device=DEV)
        plan, tok = skv.plan_build(sl, cu, int(cu_h[-1]), kvh, ncu, smax, causal)
        wp, wt = oracle.plan_segments(lens.tolist(), cu_h, kvh, 16, ncu, smax, causal)
        assert plan.cpu().tolist() == wp, (trial, bs, kvh, ncu, smax)
        assert tok.cpu().tolist() == wt, trial


def test_plan_large_batch():
    rng = np.random.default_rng(7)
    bs = 32767
    lens = rng.integers(0, 5000, size=bs).astype(np.int32)
    ql = np.ones(bs, dtype=np.int64)
    cu_h = np.array(_cu(ql.tolist()), dtype=np.int32)
    plan, tok = skv.plan_build(torch.as_tensor(lens, device=DEV), torch.as_tensor(cu_h, device=DEV),
                               bs, 1, 256, 64, 1)
    wp, wt = oracle.plan_segments(lens.tolist(), cu_h, 1, 16, 256, 64, 1)
    assert plan.cpu().tolist() == wp and tok.cpu().tolist() == wt


@pytest.mark.parametrize("bs", [1023, 1024, 1025, 4096, 4097], ids=str)
def test_plan_batch_size_boundaries(bs):
    """Batch sizes on both sides of the planner's internal limits (one sequence
    per thread up to 1024; page counts cached for the wave-parallel search up
    to 4096, a binary search beyond): short batches that fall back to one
    segment per sequence, long ones with a work-list budget above the batch
    size, and three sequences just under INT32_MAX tokens; plan and per-token
    counts bit-exact."""
    rng = np.random.default_rng(bs)
    for trial in range(3):
        lens = rng.integers(0, 3000 if trial == 0 else 300_000, size=bs)
        lens[rng.random(bs) < 0.1] = 0
        smax = int(rng.integers(1, 65))
        ncu = 256 if trial == 0 else 65536
        if trial == 2:
            lens[rng.choice(bs, size=3, replace=False)] = 2**31 - 1 - rng.integers(0, 100, size=3)
            smax = 65535
        ql = rng.integers(1, 5, size=bs)
        kvh = int(rng.choice([1, 2, 8]))
        causal = trial % 2
        cu_h = np.array(_cu(ql.tolist()), dtype=np.int32)
        say("plan boundary", bs, trial)
        plan, tok = skv.plan_build(torch.as_tensor(lens.astype(np.int32), device=DEV),
                                   torch.as_tensor(cu_h, device=DEV), int(cu_h[-1]), kvh, ncu,
                                   smax, causal)
        wp, wt = oracle.plan_segments(lens.tolist(), cu_h, kvh, 16, ncu, smax, causal)
        assert plan.cpu().tolist() == wp, (bs, trial)
        assert tok.cpu().tolist() == wt, (bs, trial)


# ---- page shuffle: bit-exact -------------------------------------------------

@pytest.mark.parametrize("e,H,subset,N", [(2, 1, False, 16), (2, 3, False, 16), (2, 8, True, 16),
                                           (1, 2, False, 16), (1, 3, True, 16), (2, 2, True, 16),
                                           (2, 3, True, 32), (1, 5, False, 32)])
def test_shuffle_bit_exact(e, H, subset, N):
    say("shuffle", e, H, subset, N)
    g = torch.Generator(device=DEV).manual_seed(11 + H)
    B = 37
    n_el = B * H * N * 256
    raw = torch.randint(0, 256, (n_el * e,), generator=g, device=DEV, dtype=torch.uint8)
    std = raw.view(torch.int16 if e == 2 else torch.uint8).view(B, H, N, 256)
    if e == 2:
        std = std.view(torch.bfloat16)
    x = 16 // e
    kp = torch.full((B, H, 128 // x, N, x), 7, dtype=std.dtype, device=DEV) if e == 1 else \
        torch.zeros((B, H, 128 // x, N, x), dtype=std.dtype, device=DEV)
    vp = torch.zeros((B, H, N // x, 128, x), dtype=std.dtype, device=DEV)
    ids = None
    if subset:
        ids_h = np.random.default_rng(H).choice(B, size=11, replace=False).astype(np.int32)
        ids = torch.as_tensor(ids_h, device=DEV)
    before_k = (kp.view(torch.uint8) if e == 1 else kp.view(torch.int16)).cpu().numpy()
    skv.kv_page_shuffle(std, kp, vp, block_ids=ids)
    torch.cuda.synchronize()
    host = (std.view(torch.int16).cpu().numpy().view(np.uint16) if e == 2
            else std.cpu().numpy())
    wk, wv = oracle.shuffle_blocks(host, block_ids=None if ids is None else ids_h)
    gk = kp.view(torch.int16).cpu().numpy().view(np.uint16) if e == 2 else kp.cpu().numpy()
    gv = vp.view(torch.int16).cpu().numpy().view(np.uint16) if e == 2 else vp.cpu().numpy()
    listed = range(B) if ids is None else ids_h
    for b in listed:
        assert np.array_equal(gk[b], wk[b]) and np.array_equal(gv[b], wv[b]), b
    if ids is not None:
        for b in set(range(B)) - set(ids_h.tolist()):
            assert np.array_equal(gk[b], before_k[b].view(gk.dtype)), "unlisted block written"


# ---- attention parity on small and edge cases --------------------------------

CASES = [
    # name, seq_lens, q_lens, Hq, Hkv, dtype, layout, causal, num_cus, seg_max
    ("tiny_std", [37, 100], [1, 1], 8, 2, "bf16", "standard", 1, 256, 64),
    ("tiny_shuf", [37, 100], [1, 1], 8, 2, "bf16", "shuffled", 1, 256, 64),
    ("rows8_ragged", [1, 5, 17, 300, 1000], [2, 2, 1, 2, 2], 8, 2, "bf16", "standard", 1, 64, 8),
    ("rows8_shuf", [1, 5, 17, 300, 1000], [2, 2, 1, 2, 2], 8, 2, "bf16", "shuffled", 1, 64, 8),
    ("fp8_rows4_std", [3, 77, 513, 2049], [1, 1, 1, 1], 16, 4, "fp8", "standard", 1, 40, 16),
    ("fp8_rows4_shuf", [3, 77, 513, 2049], [1, 1, 1, 1], 16, 4, "fp8", "shuffled", 1, 40, 16),
    ("valu_g1_q1", [7, 300, 5000, 33, 0], [1, 1, 1, 1, 1], 2, 2, "bf16", "standard", 1, 64, 16),
    ("valu_g1_q3", [50, 700, 3, 129], [3, 3, 2, 1], 2, 2, "bf16", "standard", 1, 32, 64),
    ("valu_g2_q2_shuf", [1, 17, 999, 4096], [2, 1, 2, 2], 4, 2, "bf16", "shuffled", 1, 32, 64),
    ("valu_g4_noncausal", [100, 2000, 16], [1, 1, 1], 8, 2, "bf16", "standard", 0, 256, 64),
    ("valu_g4_shuf_tails", [15, 31, 33, 1023], [1, 1, 1, 1], 32, 8, "bf16", "shuffled", 1, 128, 64),
    ("bf16_rows32_shuf", [3, 40, 777, 2500], [4, 2, 4, 3], 16, 2, "bf16", "shuffled", 1, 32, 64),
    ("fp8_rows64_std", [1, 50, 1500, 333], [4, 4, 3, 2], 32, 2, "fp8", "standard", 1, 64, 64),
    ("fp8_rows64_shuf", [1, 50, 1500, 333], [4, 4, 3, 2], 32, 2, "fp8", "shuffled", 1, 64, 64),
    ("mfma1_g16_q1", [0, 1, 5, 17, 4000, 2333], [1, 1, 1, 1, 1, 1], 32, 2, "bf16", "standard", 1, 256, 64),
    ("mfma2_g8_q4", [1, 5, 17, 900, 3000], [4, 3, 2, 4, 1], 16, 2, "bf16", "standard", 1, 32, 64),
    ("mfma4_g16_q4", [0, 1, 5, 17, 5000, 1234], [4, 4, 4, 2, 4, 3], 32, 2, "bf16", "standard", 1, 64, 64),
    ("mfma4_g16_q4_shuf", [0, 1, 5, 17, 5000, 1234], [4, 4, 4, 2, 4, 3], 32, 2, "bf16", "shuffled", 1, 64, 64),
    ("mfma4_noncausal", [3, 60, 2000], [4, 4, 4], 32, 2, "bf16", "standard", 0, 48, 64),
    ("mfma_fp8_std", [1, 8, 700, 4100], [4, 1, 3, 2], 16, 2, "fp8", "standard", 1, 64, 64),
    ("mfma_fp8_shuf", [1, 8, 700, 4100], [4, 1, 3, 2], 16, 2, "fp8", "shuffled", 1, 64, 64),
    ("mfma_g4_q3", [33, 1000], [3, 3], 16, 4, "bf16", "standard", 1, 256, 64),
    ("seg_max_binds", [1600, 16, 9999], [2, 4, 3], 16, 2, "bf16", "standard", 1, 512, 3),
    ("infeasible_fallback", [100, 200, 300, 400, 500], [1, 2, 3, 4, 1], 8, 4, "bf16", "standard", 1, 8, 64),
    # more work-groups than num_cus (more sequences than num_cus / kv_heads): the
    # two-per-CU forms with half-size rings (4 waves in the private-ring kernels)
    ("dual_valu_shuf", [1, 17, 300, 999, 64, 5000, 0, 2049], [1] * 8, 8, 2, "bf16", "shuffled", 1, 4, 64),
    ("dual_valu_std", [1, 17, 300, 999, 64, 5000, 0, 2049], [1] * 8, 8, 2, "bf16", "standard", 1, 4, 64),
    ("dual_fp8_rows8", [3, 77, 513, 2049, 16, 0, 4000], [1] * 7, 16, 2, "fp8", "standard", 1, 4, 64),
    ("dual_fp8_rows32_shuf", [3, 77, 513, 2049, 16, 1, 4000], [4, 2, 3, 4, 1, 1, 4], 16, 2, "fp8",
     "shuffled", 1, 4, 64),
    ("dual_bf16_rows16_shuf", [5, 300, 2000, 17, 999], [2, 1, 2, 2, 1], 16, 2, "bf16", "shuffled", 1, 4, 64),
    ("dual_bf16_rows32", [5, 300, 2000, 17, 999], [4, 3, 4, 1, 2], 16, 2, "bf16", "standard", 1, 4, 64),
    ("dual_bf16_rows32_noncausal", [5, 300, 2000, 17, 999], [4, 3, 4, 1, 2], 16, 2, "bf16", "standard", 0, 4,
     64),
]


def _mk(name, lens, ql, hq, hkv, dt, layout, causal, ncu, smax, seed=5, poison="finite",
        page_size=16):
    base = configs.FP8_KV if dt == "fp8" else configs.TINY
    cfg = gen.small_config(base, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                           causal=causal, num_cus=ncu, seg_max=smax, seed=seed,
                           page_size=page_size, kv_dtype=dt)
    return gen.make_case(cfg, DEV, poison=poison)


@pytest.mark.parametrize("spec", CASES, ids=lambda c: c[0])
def test_attention_matches_oracle(spec):
    say("attn", spec[0])
    case = _mk(*spec)
    hip = run_hip(case)
    wp, wt = oracle_plan(case)
    assert hip["plan"] == wp and hip["tok"] == wt
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, case.cfg.kv_dtype)
    say(spec[0], r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r


# 32-token pages (the kernels stream 16-token sub-pages): every kernel variant,
# both layouts, lengths around sub-page and page boundaries
P32_CASES = [
    ("p32_valu_std", [1, 15, 16, 17, 31, 32, 33, 1000], [1] * 8, 8, 2, "bf16", "standard", 1, 64, 64),
    ("p32_valu_shuf", [33, 4097, 64, 2], [1, 1, 1, 1], 8, 2, "bf16", "shuffled", 1, 32, 64),
    ("p32_valu_q3", [50, 700, 3, 129], [3, 3, 2, 1], 2, 2, "bf16", "standard", 1, 32, 64),
    ("p32_bf16_rows16", [5, 17, 900, 3000], [2, 1, 2, 2], 16, 2, "bf16", "standard", 1, 32, 64),
    ("p32_bf16_rows32_shuf", [3, 40, 777, 2500], [4, 2, 4, 3], 16, 2, "bf16", "shuffled", 1, 32, 64),
    ("p32_bf16_rows64", [0, 1, 5, 17, 5000, 1234], [4, 4, 4, 2, 4, 3], 32, 2, "bf16", "standard", 1, 64, 64),
    ("p32_bf16_rows64_shuf", [31, 33, 2049, 777], [4, 4, 3, 4], 32, 2, "bf16", "shuffled", 0, 64, 64),
    ("p32_fp8_rows8", [3, 77, 513, 2049], [1, 2, 1, 1], 16, 4, "fp8", "standard", 1, 40, 16),
    ("p32_fp8_rows8_shuf", [3, 77, 513, 2049], [1, 2, 1, 1], 16, 4, "fp8", "shuffled", 1, 40, 16),
    ("p32_fp8_rows32", [1, 8, 700, 4100], [4, 1, 3, 2], 16, 2, "fp8", "standard", 1, 64, 64),
    ("p32_fp8_rows64", [1, 50, 1500, 333], [4, 4, 3, 2], 32, 2, "fp8", "standard", 1, 64, 64),
    ("p32_fp8_rows64_shuf", [1, 50, 1500, 333], [4, 4, 3, 2], 32, 2, "fp8", "shuffled", 1, 64, 64),
    ("p32_infeasible", [100, 200, 300, 400, 500], [1, 2, 3, 4, 1], 8, 4, "bf16", "standard", 1, 8, 64),
    ("p32_dual_valu_shuf", [33, 4097, 64, 2, 1000, 31], [1] * 6, 8, 2, "bf16", "shuffled", 1, 4, 64),
    ("p32_dual_fp8_rows16", [3, 77, 513, 2049, 33, 4000], [2, 2, 1, 2, 1, 2], 16, 2, "fp8", "standard", 1, 4, 64),
    ("p32_dual_bf16_rows32_shuf", [3, 40, 777, 2500, 65], [4, 2, 4, 3, 1], 16, 2, "bf16", "shuffled", 1, 4, 64),
]


@pytest.mark.parametrize("spec", P32_CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("fixed", [False, True], ids=["planned", "fixed"])
def test_32_token_pages_match_oracle(spec, fixed):
    say("p32", spec[0], "fixed" if fixed else "planned")
    case = _mk(*spec, page_size=32)
    cfg = case.cfg
    hip = run_hip(case, fixed=fixed)
    if fixed:
        _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                                 cfg.kv_heads, 32, cfg.num_cus, cfg.seg_max,
                                                 cfg.causal)
        assert hip["tok"] == want_tok
    else:
        wp, wt = oracle_plan(case)
        assert hip["plan"] == wp and hip["tok"] == wt
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, cfg.kv_dtype)
    say(spec[0], r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r


def test_plan_bit_exact_fuzz_32_token_pages():
    rng = np.random.default_rng(2032)
    for trial in range(60):
        bs = int(rng.integers(1, 301))
        lens = rng.integers(0, 300_001 if trial % 3 == 0 else 3000, size=bs)
        lens[rng.random(bs) < 0.1] = 0
        ql = rng.integers(1, 5, size=bs)
        kvh = int(rng.choice([1, 2, 4, 8]))
        ncu = int(rng.integers(4, 305))
        smax = int(rng.integers(1, 65))
        causal = int(rng.integers(0, 2))
        cu_h = np.array(_cu(ql.tolist()), dtype=np.int32)
        plan, tok = skv.plan_build(torch.as_tensor(lens.astype(np.int32), device=DEV),
                                   torch.as_tensor(cu_h, device=DEV), int(cu_h[-1]), kvh, ncu,
                                   smax, causal, page_size=32)
        wp, wt = oracle.plan_segments(lens.tolist(), cu_h, kvh, 32, ncu, smax, causal)
        assert plan.cpu().tolist() == wp, (trial, bs, kvh, ncu, smax)
        assert tok.cpu().tolist() == wt, trial


# fp16 Q and KV: every 16-bit kernel route (vector ALU up to 4 rows, private
# rings up to 32, shared ring up to 64), both layouts
FP16_CASES = [
    ("f16_valu_std", [7, 300, 5000, 33, 0], [1, 1, 1, 1, 1], 2, 2, "fp16", "standard", 1, 64, 16),
    ("f16_valu_q3", [50, 700, 3, 129], [3, 3, 2, 1], 2, 2, "fp16", "standard", 1, 32, 64),
    ("f16_valu_shuf_tails", [15, 31, 33, 1023], [1, 1, 1, 1], 32, 8, "fp16", "shuffled", 1, 128, 64),
    ("f16_rows8_ragged", [1, 5, 17, 300, 1000], [2, 2, 1, 2, 2], 8, 2, "fp16", "standard", 1, 64, 8),
    ("f16_rows32_shuf", [3, 40, 777, 2500], [4, 2, 4, 3], 16, 2, "fp16", "shuffled", 1, 32, 64),
    ("f16_rows64", [0, 1, 5, 17, 5000, 1234], [4, 4, 4, 2, 4, 3], 32, 2, "fp16", "standard", 1, 64, 64),
    ("f16_rows64_shuf", [0, 1, 5, 17, 5000, 1234], [4, 4, 4, 2, 4, 3], 32, 2, "fp16", "shuffled", 1, 64, 64),
    ("f16_noncausal", [3, 60, 2000], [4, 4, 4], 32, 2, "fp16", "standard", 0, 48, 64),
    ("f16_dual_valu_shuf", [1, 17, 300, 999, 64, 5000], [1] * 6, 8, 2, "fp16", "shuffled", 1, 4, 64),
    ("f16_dual_rows32", [5, 300, 2000, 17, 999], [4, 3, 4, 1, 2], 16, 2, "fp16", "standard", 1, 4, 64),
]


@pytest.mark.parametrize("spec", FP16_CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("fixed", [False, True], ids=["planned", "fixed"])
@pytest.mark.parametrize("page_size", [16, 32])
def test_fp16_matches_oracle(spec, fixed, page_size):
    say("fp16", spec[0], fixed, page_size)
    case = _mk(*spec, page_size=page_size)
    cfg = case.cfg
    hip = run_hip(case, fixed=fixed)
    if fixed:
        _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                                 cfg.kv_heads, page_size, cfg.num_cus,
                                                 cfg.seg_max, cfg.causal)
        assert hip["tok"] == want_tok
    else:
        wp, wt = oracle_plan(case)
        assert hip["plan"] == wp and hip["tok"] == wt
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, cfg.kv_dtype)
    say(spec[0], r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r


@pytest.mark.parametrize("qmul", [6.0, 24.0])
@pytest.mark.parametrize("spec", [c for c in FP16_CASES if c[0] in ("f16_valu_q3", "f16_rows8_ragged",
                                                                    "f16_rows64")],
                         ids=lambda c: c[0])
def test_fp16_sharp_scores_match_oracle(spec, qmul):
    """fp16 weights underflow below 2^-24 where bf16 ones would not: sharp
    scores check that this changes nothing beyond the bar."""
    case = _mk(*spec)
    case.q.copy_((case.q.float() * qmul).to(torch.float16))
    hip = run_hip(case)
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, "fp16")
    say(spec[0], qmul, r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3 * max(1.0, float(np.abs(ref_lse[np.isfinite(ref_lse)]).max())), r


@pytest.mark.parametrize("spec", [c for c in FP16_CASES if c[0] in ("f16_valu_shuf_tails",
                                                                    "f16_rows8_ragged",
                                                                    "f16_rows64_shuf")],
                         ids=lambda c: c[0])
def test_fp16_nan_poison_does_not_leak(spec):
    a = run_hip(_mk(*spec, poison="finite"))
    b = run_hip(_mk(*spec, poison="nan"))
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.all(np.isfinite(b["out"]))
    c = run_hip(_mk(*spec, poison="nan"), claim=True)
    assert np.all(np.isfinite(c["out"]))
    assert np.max(np.abs(c["out"] - a["out"])) <= TOL["fp16"]


FIXED_CASES = CASES + [
    # bs 1: the fixed split's own case (64 segments), and S = 1 (bs * kv_heads > num_cus)
    ("bs1_long", [70000], [4], 32, 2, "bf16", "standard", 1, 256, 64),
    ("bs1_fp8_q1", [9000], [1], 16, 2, "fp8", "shuffled", 1, 256, 64),
    ("fixed_S1", [50, 900, 17, 3000], [1, 2, 3, 4], 16, 4, "bf16", "standard", 1, 8, 64),
]


@pytest.mark.parametrize("spec", FIXED_CASES, ids=lambda c: c[0])
def test_fixed_split_matches_oracle(spec):
    """No plan: the fixed split's segment counts bit-exact, the output within
    tolerance of the unsplit oracle, and within the split-KV PR's
    planned-vs-fixed bound (Accuracy Tests: at most 0.007 apart, the fp32
    summation order across segment boundaries being the only difference) of
    the planned split's output."""
    say("fixed", spec[0])
    case = _mk(*spec)
    cfg = case.cfg
    hip = run_hip(case, fixed=True)
    planned = run_hip(case)
    diff = np.abs(hip["out"] - planned["out"])
    say(spec[0], "planned vs fixed max abs", float(diff.max()))
    # the PR's 0.007, plus one bf16 rounding step of the value (outputs near
    # or above 1 can round one unit apart: 2^-7 at [1, 2))
    assert np.all(diff <= 0.007 + 2.0 ** -7 * np.abs(planned["out"]))
    _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                             cfg.kv_heads, 16, cfg.num_cus, cfg.seg_max,
                                             cfg.causal)
    assert hip["tok"] == want_tok
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, cfg.kv_dtype)
    say(spec[0], r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r


_BY = {c[0]: c for c in CASES}

SHARP = [
    # name, seq_lens, q_lens, Hq, Hkv, dtype, layout, causal, num_cus, seg_max
    ("sharp_fp8_rows8", [3, 700, 2100], [1, 4, 2], 8, 4, "fp8", "standard", 1, 16, 64),
    ("sharp_fp8_rows32_shuf", [40, 3000], [4, 3], 16, 2, "fp8", "shuffled", 1, 16, 64),
    ("sharp_fp8_rows64", [17, 4100, 999], [4, 4, 3], 32, 2, "fp8", "standard", 1, 16, 64),
    ("sharp_fp8_rows64_shuf", [17, 4100, 999], [4, 4, 3], 32, 2, "fp8", "shuffled", 0, 16, 64),
    ("sharp_bf16_rows16", [5, 2222, 900], [2, 2, 1], 16, 2, "bf16", "standard", 1, 16, 64),
    ("sharp_bf16_rows32_shuf", [33, 3000], [4, 2], 16, 2, "bf16", "shuffled", 1, 16, 64),
    ("sharp_bf16_rows64", [17, 4100, 999], [4, 4, 3], 32, 2, "bf16", "standard", 1, 16, 64),
    ("sharp_bf16_rows4", [17, 4100, 999], [1, 1, 1], 8, 2, "bf16", "standard", 1, 16, 64),
]


@pytest.mark.parametrize("qmul", [6.0, 24.0])
@pytest.mark.parametrize("spec", SHARP, ids=lambda c: c[0])
def test_sharp_scores_match_oracle(spec, qmul):
    """Q scaled so scores spread over tens of units in the exp2 domain: the
    running row maxima rise many times and by large steps inside one segment,
    and the outputs are dominated by a few keys (O(1) values, so the max-abs
    bar is tight). Few segments per sequence (num_cus 16) keep many blocks in
    each work-group."""
    say("sharp", spec[0], qmul)
    case = _mk(*spec)
    case.q.copy_((case.q.float() * qmul).to(torch.bfloat16))
    hip = run_hip(case)
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, case.cfg.kv_dtype)
    say(spec[0], qmul, r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3 * max(1.0, float(np.abs(ref_lse[np.isfinite(ref_lse)]).max())), r


@pytest.mark.parametrize("spec", [_BY[n] for n in ("fp8_rows4_std", "mfma_fp8_shuf",
                                                   "fp8_rows64_std")], ids=lambda c: c[0])
def test_fp8_negative_k_scale(spec):
    """A negative K scale flips every score; the kernels move it into Q's sign."""
    name, lens, ql, hq, hkv, dt, layout, causal, ncu, smax = spec
    cfg = gen.small_config(configs.FP8_KV, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                           causal=causal, num_cus=ncu, seg_max=smax, seed=9,
                           k_scale=-0.0173, v_scale=-0.0211)
    case = gen.make_case(cfg, DEV)
    hip = run_hip(case)
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, "fp8")
    say(name, "negative scales", r)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r


@pytest.mark.parametrize("bs,dt,layout", [(3000, "bf16", "standard"), (1500, "fp8", "shuffled"),
                                          (2000, "bf16", "shuffled")])
def test_many_short_sequences(bs, dt, layout):
    """Thousands of sequences of 0-40 tokens: more non-empty sequences than the
    work-list budget (the planner's fallback, one segment per sequence), grids of
    thousands of work-groups, and the reduce over tens of thousands of rows; the
    plan bit-exact and the outputs within the bars, planned and fixed split."""
    say("many short", bs, dt, layout)
    rng = np.random.default_rng(bs)
    lens = rng.integers(0, 41, size=bs).tolist()
    ql = rng.integers(1, 5, size=bs).tolist()
    base = configs.FP8_KV if dt == "fp8" else configs.TINY
    cfg = gen.small_config(base, lens, ql, q_heads=16, kv_heads=2, layout=layout, num_cus=256,
                           seg_max=64, seed=12, kv_dtype=dt)
    case = gen.make_case(cfg, DEV)
    ref_out, ref_lse = run_oracle(case)
    for fixed in (False, True):
        hip = run_hip(case, fixed=fixed)
        if not fixed:
            wp, wt = oracle_plan(case)
            assert hip["plan"] == wp and hip["tok"] == wt
        r = compare(hip["out"], hip["lse"], ref_out, ref_lse, dt)
        say("many short", bs, dt, layout, "fixed" if fixed else "planned", r)
        # sequences of a key or two output single V rows, N(0,1) values that
        # reach beyond 4 among this many rows: the bar adds the output's own
        # rounding, 2^-8 of the value (reading 27)
        assert np.all(np.abs(hip["out"] - ref_out) <= r["tol"] + 2.0 ** -8 * np.abs(ref_out)), r
        assert r["lse_err"] <= 1e-3, r


@pytest.mark.parametrize("ncu", [1, 2, 3])
def test_budget_below_kv_heads(ncu):
    """num_cus below kv_heads (4): the work-list budget num_cus / kv_heads is 0,
    so the planner falls back to one segment per non-empty sequence and the
    fixed split to one segment; plan, counts and outputs against the oracle."""
    say("budget", ncu)
    lens, ql = [0, 1, 17, 300, 2049], [1, 2, 3, 4, 2]
    cfg = gen.small_config(configs.TINY, lens, ql, q_heads=16, kv_heads=4, num_cus=ncu,
                           seg_max=64, seed=13)
    case = gen.make_case(cfg, DEV)
    ref_out, ref_lse = run_oracle(case)
    for fixed in (False, True):
        hip = run_hip(case, fixed=fixed)
        if fixed:
            _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                                     cfg.kv_heads, 16, ncu, 64, cfg.causal)
            assert hip["tok"] == want_tok
        else:
            wp, wt = oracle_plan(case)
            assert hip["plan"] == wp and hip["tok"] == wt
        r = compare(hip["out"], hip["lse"], ref_out, ref_lse, "bf16")
        assert r["max_abs"] <= r["tol"], r
        assert r["lse_err"] <= 1e-3, r


@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("spec", [_BY[n] for n in ("fp8_rows4_std", "fp8_rows64_std")],
                         ids=lambda c: c[0])
def test_fp8_zero_scales(spec, head_dim):
    """K scale 0: every score is 0, so each row averages the V rows it sees
    (the kernels clamp the score scale to the least normal float); V scale 0:
    the output is 0 and the log-sum-exp unchanged."""
    name, lens, ql, hq, hkv, dt, layout, causal, ncu, smax = spec
    for ks, vs in ((0.0, 0.0211), (0.0173, 0.0)):
        cfg = gen.small_config(configs.FP8_KV, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                               causal=causal, num_cus=ncu, seg_max=smax, seed=10,
                               head_dim=head_dim, k_scale=ks, v_scale=vs)
        case = gen.make_case(cfg, DEV)
        hip = run_hip(case)
        ref_out, ref_lse = run_oracle(case)
        r = compare(hip["out"], hip["lse"], ref_out, ref_lse, "fp8")
        say(name, head_dim, "scales", ks, vs, r)
        assert r["max_abs"] <= r["tol"], r
        assert r["lse_err"] <= 1e-3, r
        if vs == 0.0:
            assert np.all(hip["out"] == 0.0)


@pytest.mark.parametrize("spec", [_BY[n] for n in ("rows8_ragged", "mfma4_g16_q4", "mfma_fp8_std",
                                                   "mfma_fp8_shuf", "fp8_rows64_std",
                                                   "fp8_rows64_shuf", "fp8_rows4_shuf",
                                                   "valu_g1_q3", "valu_g4_shuf_tails", "dual_valu_shuf",
                                                   "dual_fp8_rows32_shuf", "dual_bf16_rows16_shuf")],
                         ids=lambda c: c[0])
def test_nan_poison_does_not_leak(spec):
    a = run_hip(_mk(*spec, poison="finite"))
    b = run_hip(_mk(*spec, poison="nan"))
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.all(np.isfinite(b["out"]))
    # claimed units (opt-in): the same tail masking, summed in run-time order
    c = run_hip(_mk(*spec, poison="nan"), claim=True)
    assert np.all(np.isfinite(c["out"]))
    assert np.max(np.abs(c["out"] - a["out"])) <= TOL[spec[5]]


_BY32 = {c[0]: c for c in P32_CASES}


@pytest.mark.parametrize("spec", [_BY32[n] for n in ("p32_valu_std", "p32_bf16_rows32_shuf",
                                                     "p32_bf16_rows64", "p32_fp8_rows8_shuf",
                                                     "p32_fp8_rows64")], ids=lambda c: c[0])
def test_nan_poison_does_not_leak_32_token_pages(spec):
    a = run_hip(_mk(*spec, poison="finite", page_size=32))
    b = run_hip(_mk(*spec, poison="nan", page_size=32))
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.all(np.isfinite(b["out"]))


@pytest.mark.parametrize("spec", [_BY[n] for n in ("tiny_shuf", "mfma4_g16_q4_shuf",
                                                   "valu_g1_q1", "fp8_rows64_std", "dual_fp8_rows8",
                                                   "dual_bf16_rows16_shuf")], ids=lambda c: c[0])
def test_deterministic(spec):
    case = _mk(*spec)
    a = run_hip(case)
    b = run_hip(case)
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.array_equal(a["lse"], b["lse"])


def test_fp8_codes_decode_exactly():
    """A one-token sequence returns its V row: every e4m3fn code (NaN codes
    aside) must come back as its exact value (v_scale = 1)."""
    cfg = gen.small_config(configs.FP8_KV, [1, 1], [1, 1], q_heads=2, kv_heads=1,
                           k_scale=1.0, v_scale=1.0, seed=3)
    case = gen.make_case(cfg, DEV)
    codes = np.arange(256, dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    table = case.page_table.cpu().numpy()
    for i in range(2):
        case.kv[int(table[i, 0]), 0, 0, 128:] = torch.as_tensor(codes[128 * i:128 * (i + 1)],
                                                                 device=DEV)
    hip = run_hip(case)
    want = oracle.decode_e4m3fn(codes).reshape(2, 128)
    for i in range(2):
        for h in range(2):
            assert np.array_equal(hip["out"][i, h], want[i]), (i, h)


@pytest.mark.parametrize("D", [128, 64, 256])
@pytest.mark.parametrize("total_q", [9, 300])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("smax", [7, 64, 100, 256, 300])
def test_split_reduce_alone(smax, out_dtype, total_q, D):
    """Every merge path (up to 64 segments, up to 256 with four per lane, and
    more) in both launch forms: one work-group per row (36 rows) and four rows
    per work-group (1200 rows). Some segments carry no key (log-sum-exp -inf,
    zero output, as the segment kernel writes them)."""
    rng = np.random.default_rng(3 + smax + total_q + D)
    hq = 4
    nseg = rng.integers(0, smax + 1, size=total_q).astype(np.int32)
    po = rng.standard_normal((total_q, hq, smax, D)).astype(np.float32)
    pl = (rng.standard_normal((total_q, hq, smax)) * 4).astype(np.float32)
    empty = rng.random((total_q, hq, smax)) < 0.05
    pl[empty] = -np.inf
    po[empty] = 0.0
    pl[0, 0, :] = -np.inf                      # a row whose segments all carry no key
    po[0, 0, :] = 0.0
    for t in range(total_q):                   # entries past the count are unspecified
        po[t, :, nseg[t]:] = np.nan
        pl[t, :, nseg[t]:] = np.nan
    out, lse = skv.split_reduce(torch.as_tensor(po.reshape(-1), device=DEV),
                                torch.as_tensor(pl.reshape(-1), device=DEV),
                                torch.as_tensor(nseg, device=DEV), total_q=total_q,
                                q_heads=hq, seg_max=smax, out_dtype=out_dtype, head_dim=D,
                                out_lse=torch.empty(total_q * hq, device=DEV))
    torch.cuda.synchronize()
    assert out.dtype == (torch.float16 if out_dtype == "fp16" else torch.bfloat16)
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy().reshape(total_q, hq)
    for t in range(total_q):
        for h in range(hq):
            k = int(nseg[t])
            wo, wl = oracle.lse_merge(po[t, h, :k].astype(np.float64),
                                      pl[t, h, :k].astype(np.float64), D)
            # outputs here reach |4|: rounding to bf16 (nearest even) adds up to
            # 2^-9 of the value on top of the absolute bar
            np.testing.assert_allclose(out[t, h], wo, atol=1e-2, rtol=2.0 ** -8)
            if k == 0 or np.all(pl[t, h, :k] == -np.inf):
                assert lse[t, h] == -np.inf and np.all(out[t, h] == 0)
            else:
                assert abs(lse[t, h] - wl) <= 1e-5 * max(1.0, abs(wl))


@pytest.mark.parametrize("fixed", [False, True], ids=["planned", "fixed"])
@pytest.mark.parametrize("seg_max", [100, 128, 300])
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_many_segments_per_token(dt, seg_max, fixed):
    """More than 64 segments per query token end to end: a CU budget of
    2 * seg_max (planned) or 4 * seg_max (fixed) for two sequences at two kv
    heads lets the planner cut the 60k-token sequence into up to seg_max
    segments and the fixed split into the largest power of two within seg_max,
    so the reduce takes its four-per-lane path (up to 256) or its plain loop
    (beyond); plan or counts bit-exact, outputs against the oracle."""
    say("many segments", dt, seg_max, "fixed" if fixed else "planned")
    base = configs.FP8_KV if dt == "fp8" else configs.TINY
    cfg = gen.small_config(base, [60_000, 3_000], [4, 2], q_heads=32, kv_heads=2,
                           num_cus=(4 if fixed else 2) * seg_max, seg_max=seg_max, seed=17,
                           kv_dtype=dt)
    case = gen.make_case(cfg, DEV)
    hip = run_hip(case, fixed=fixed)
    if fixed:
        _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                                 cfg.kv_heads, cfg.page_size, cfg.num_cus,
                                                 seg_max, cfg.causal)
        assert hip["tok"] == want_tok
    else:
        wp, wt = oracle_plan(case)
        assert hip["plan"] == wp and hip["tok"] == wt
    if seg_max >= 128:
        assert max(hip["tok"]) > 64, "the case reaches past 64 segments per token"
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, dt)
    say(r)
    assert r["max_abs"] <= TOL[dt], r
    assert r["lse_err"] <= 1e-3, r
