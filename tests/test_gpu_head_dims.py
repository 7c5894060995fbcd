"""GPU parity at head dims 64 and 256 (the generic-width segment kernel, the
split reduce and the page shuffle at those widths) against the CPU oracle,
through the C ABI: every element type, both layouts, 16- and 32-token pages,
the planned and the fixed split, 1 to 64 query rows, ragged lengths around
sub-page, page and ring-stage boundaries, NaN page-tail poison."""
import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_amd as skv
from gpu_harness import compare, oracle_plan, run_hip, run_oracle, say
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


# (name, seq_lens, q_lens, q_heads, kv_heads, causal, num_cus, seg_max)
SHAPES = [
    # 64 rows (GQA 16 x 4 query tokens), empty and one-token sequences
    ("rows64", [0, 1, 17, 300, 2500], [4, 4, 3, 1, 2], 32, 2, 1, 64, 64),
    # 4 rows, lengths at sub-page and page edges, seg_max binding
    ("rows4", [15, 16, 33, 700, 4097], [1, 2, 1, 2, 1], 8, 4, 1, 32, 8),
    # 24 rows (two row tiles, the second ragged), non-causal
    ("rows24", [5, 129, 1000, 64], [3, 3, 2, 1], 16, 2, 0, 48, 64),
]


def _mk(shape, D, dt, layout, page_size, poison="finite"):
    name, lens, ql, hq, hkv, causal, ncu, smax = shape
    base = configs.FP8_KV if dt == "fp8" else configs.TINY
    cfg = gen.small_config(base, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                           causal=causal, num_cus=ncu, seg_max=smax, seed=7 + D,
                           page_size=page_size, kv_dtype=dt, head_dim=D)
    return gen.make_case(cfg, DEV, poison=poison)


def _check(case, hip):
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, case.cfg.kv_dtype)
    assert r["max_abs"] <= r["tol"], r
    assert r["lse_err"] <= 1e-3, r
    return r


@pytest.mark.parametrize("page_size", [16, 32])
@pytest.mark.parametrize("layout", ["standard", "shuffled"])
@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp8"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s[0])
@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_matches_oracle(D, shape, dt, layout, page_size):
    say("head_dim", D, shape[0], dt, layout, page_size)
    case = _mk(shape, D, dt, layout, page_size)
    hip = run_hip(case)
    wp, wt = oracle_plan(case)
    assert hip["plan"] == wp and hip["tok"] == wt
    say(_check(case, hip))


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_fixed_split(D, dt):
    shape = SHAPES[0]
    say("head_dim fixed", D, dt)
    case = _mk(shape, D, dt, "standard", 16)
    cfg = case.cfg
    hip = run_hip(case, fixed=True)
    _, _, want_tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(),
                                             cfg.kv_heads, 16, cfg.num_cus, cfg.seg_max,
                                             cfg.causal)
    assert hip["tok"] == want_tok
    say(_check(case, hip))


@pytest.mark.parametrize("layout", ["standard", "shuffled"])
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_nan_poison_does_not_leak(D, dt, layout):
    say("head_dim poison", D, dt, layout)
    shape = SHAPES[1]
    fin = _mk(shape, D, dt, layout, 16, poison="finite")
    nan = _mk(shape, D, dt, layout, 16, poison="nan")
    a, b = run_hip(fin), run_hip(nan)
    assert np.all(np.isfinite(b["out"]))
    # the kernel's order is fixed: poison values never enter the arithmetic
    assert np.array_equal(a["out"].view(np.uint16), b["out"].view(np.uint16))


@pytest.mark.parametrize("e,N", [(2, 16), (1, 16), (2, 32), (1, 32)])
@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_shuffle_bit_exact(D, e, N):
    say("head_dim shuffle", D, e, N)
    g = torch.Generator(device=DEV).manual_seed(3 + D + e + N)
    B, H = 13, 3
    raw = torch.randint(0, 256, (B * H * N * 2 * D * e,), generator=g, device=DEV,
                        dtype=torch.uint8)
    std = raw.view(torch.int16 if e == 2 else torch.uint8).view(B, H, N, 2 * D)
    kp, vp = skv.kv_page_shuffle(std)
    torch.cuda.synchronize()
    host = std.cpu().numpy().view(np.uint16) if e == 2 else std.cpu().numpy()
    wk, wv = oracle.shuffle_blocks(host)
    gk = kp.cpu().numpy().view(np.uint16) if e == 2 else kp.cpu().numpy()
    gv = vp.cpu().numpy().view(np.uint16) if e == 2 else vp.cpu().numpy()
    assert np.array_equal(gk, wk) and np.array_equal(gv, wv)


# long segments (num_cus 16: few segments, many blocks per work-group) so the
# running row maxima rise many times inside one work-group
SHARP_SHAPES = [
    ("sharp_rows64", [0, 1, 17, 3000, 9000], [4, 4, 3, 1, 2], 32, 2, 1, 16, 64),
    ("sharp_rows4", [15, 700, 5000], [1, 2, 1], 8, 4, 1, 16, 8),
]


@pytest.mark.parametrize("qmul", [6.0, 24.0])
@pytest.mark.parametrize("layout", ["standard", "shuffled"])
@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp8"])
@pytest.mark.parametrize("shape", SHARP_SHAPES, ids=lambda s: s[0])
@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_sharp_scores(D, shape, dt, layout, qmul):
    """Q scaled so that scores spread over tens of units: the generic-width
    kernel's lazy row-max rescale runs often and by large steps, and outputs
    are dominated by a few keys (O(1) values, so the max-abs bar is tight)."""
    say("head_dim sharp", D, shape[0], dt, layout, qmul)
    case = _mk(shape, D, dt, layout, 16)
    case.q.copy_((case.q.float() * qmul).to(case.q.dtype))
    hip = run_hip(case)
    ref_out, ref_lse = run_oracle(case)
    r = compare(hip["out"], hip["lse"], ref_out, ref_lse, dt)
    say(r)
    assert r["max_abs"] <= r["tol"], r
    assert r["max_rel_rms"] <= 1e-2, r
    assert r["lse_err"] <= 1e-3 * max(1.0, float(np.abs(ref_lse[np.isfinite(ref_lse)]).max())), r


@pytest.mark.parametrize("layout", ["standard", "shuffled"])
@pytest.mark.parametrize("shape", SHAPES[:2], ids=lambda s: s[0])
@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_fp8_negative_scales(D, shape, layout):
    """Negative fp8 scales flip every score and every V value."""
    say("head_dim negative scales", D, shape[0], layout)
    name, lens, ql, hq, hkv, causal, ncu, smax = shape
    cfg = gen.small_config(configs.FP8_KV, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                           causal=causal, num_cus=ncu, seg_max=smax, seed=11 + D,
                           head_dim=D, k_scale=-0.0173, v_scale=-0.0211)
    case = gen.make_case(cfg, DEV)
    hip = run_hip(case)
    say(_check(case, hip))
