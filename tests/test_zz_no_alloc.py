"""The allocation-free attention entry point (skv_paged_decode_attn_static,
partials in the library's own device array) against the workspace entry point
(skv_paged_decode_attn) on the same inputs, through the C ABI: two calls in a
row, the second on a smaller input, so the second runs over the first's
leftovers in the shared array. Same kernels and summation order, so the
outputs must agree bit for bit (which is within the attention tolerance)."""
import numpy as np
import pytest
import torch

import split_kv_paged_amd as skv
from split_kv_paged_amd import _lib
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


def _both(cfg, fixed=False):
    """(workspace out, lse, tok), (static out, lse, tok) on one case."""
    print("no-alloc", cfg.name, cfg.bs, cfg.total_q, cfg.kv_dtype, cfg.layout, "fixed" if fixed
          else "planned", flush=True)
    case = gen.make_case(cfg, DEV)
    kv_a, kv_b = case.kv, None
    if cfg.layout == "shuffled":
        kv_a, kv_b = skv.kv_page_shuffle(case.kv)
    res = []
    for static in (False, True):
        if fixed:
            plan, tok = None, torch.full((cfg.total_q,), -7, dtype=torch.int32, device=DEV)
        else:
            plan, tok = skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q,
                                       cfg.kv_heads, cfg.num_cus, cfg.seg_max, cfg.causal,
                                       page_size=cfg.page_size)
        lse = torch.full((cfg.total_q, cfg.q_heads), 7.0, dtype=torch.float32, device=DEV)
        kw = dict(kv_heads=cfg.kv_heads, max_q=cfg.max_q, num_cus=cfg.num_cus,
                  seg_max=cfg.seg_max, kv_dtype=cfg.kv_dtype, layout=cfg.layout,
                  k_scale=case.k_scale, v_scale=case.v_scale, causal=cfg.causal,
                  out_lse=lse, page_size=cfg.page_size)
        fn = skv.paged_decode_attn_static if static else skv.paged_decode_attn
        out, _ = fn(case.q, kv_a, kv_b, case.page_table, case.seq_lens, case.cu_seqlens_q,
                    plan, tok, **kw)
        torch.cuda.synchronize()
        res.append((gen.raw_u16(out), lse.cpu().numpy(), tok.cpu().numpy()))
    return res


def _same(a, b):
    assert np.array_equal(a[0], b[0]), "outputs differ"
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32)), "lse differs"
    assert np.array_equal(a[2], b[2]), "tok_nseg differs"


def test_static_entry_point_two_calls_second_smaller():
    # 1: the full agentic skew batch (55 query tokens x 32 heads x 64 segments
    #    at head dim 128: 58 MB of partials, close to the 64 MiB array)
    big = configs.AGENTIC_SKEW
    need = skv.workspace_bytes(big.total_q, big.q_heads, big.head_dim, big.seg_max)
    assert 48 << 20 < need <= skv.STATIC_SCRATCH_BYTES
    ws, st = _both(big)
    _same(ws, st)
    # 2: a smaller batch over the first call's leftovers
    small = gen.small_config(configs.AGENTIC_SKEW, [0, 1, 17, 3000, 900], [4, 1, 2, 3, 4],
                             num_cus=64, seg_max=16, seed=31)
    ws, st = _both(small)
    _same(ws, st)


@pytest.mark.parametrize("name,fixed", [("fp8_small", False), ("shuffled_small", True)])
def test_static_entry_point_variants(name, fixed):
    """fp8 KV on the private-ring kernel and the shuffled fixed split (the
    segment kernel writes tok_nseg), each after the calls above."""
    if name == "fp8_small":
        cfg = gen.small_config(configs.FP8_KV, [40, 3000, 17, 1200], [4, 3, 1, 2], seed=32,
                               num_cus=32, seg_max=8)
    else:
        cfg = gen.small_config(configs.SHUFFLED_DECODE, [8192] * 6 + [5], [1] * 7, seed=33)
    ws, st = _both(cfg, fixed=fixed)
    _same(ws, st)


def test_static_entry_point_rejects_oversize():
    """Partials beyond the array: EUNSUPPORTED, before anything is enqueued."""
    cfg = configs.UNIFORM_VERIFY              # 64 x 32 x 64 x 129 x 4 B = 67.6 MB > 64 MiB
    assert skv.workspace_bytes(cfg.total_q, cfg.q_heads, cfg.head_dim,
                               cfg.seg_max) > skv.STATIC_SCRATCH_BYTES
    q = torch.zeros((cfg.total_q, cfg.q_heads, cfg.head_dim), dtype=torch.bfloat16, device=DEV)
    i32 = torch.zeros(cfg.bs + 1, dtype=torch.int32, device=DEV)
    tab = torch.zeros((cfg.bs, 1), dtype=torch.int32, device=DEV)
    kv = torch.zeros((1, cfg.kv_heads, 16, 2 * cfg.head_dim), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(_lib.SkvError) as ei:
        skv.paged_decode_attn_static(q, kv, None, tab, i32[:cfg.bs], i32, None,
                                     torch.zeros(cfg.total_q, dtype=torch.int32, device=DEV),
                                     kv_heads=cfg.kv_heads, max_q=cfg.max_q,
                                     num_cus=cfg.num_cus, seg_max=cfg.seg_max)
    assert ei.value.status == _lib.SKV_EUNSUPPORTED
