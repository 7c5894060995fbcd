"""Every entry point only enqueues kernels whose grids depend on host integers,
so a forward can be captured into a HIP graph. A captured plan + attention
(planned and fixed split) + shuffle + conversion + cache write, replayed
several times with eager work and synchronisations between replays, must give
the eager results bit for bit on every replay (attention in its deterministic
order; the default order, captured too, agrees to rounding)."""
import numpy as np
import pytest
import torch

import split_kv_paged_amd as skv
from gpu_harness import say
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


@pytest.mark.parametrize("dtype,layout", [("bf16", "standard"), ("bf16", "shuffled"),
                                          ("fp8", "standard")])
def test_graph_replays_match_eager(dtype, layout):
    say("graph", dtype, layout)
    base = configs.FP8_KV if dtype == "fp8" else configs.TINY
    cfg = gen.small_config(base, [0, 37, 900, 5000, 16, 2049], [1, 4, 2, 3, 1, 4], q_heads=16,
                           kv_heads=2, layout=layout, num_cus=64, seg_max=32, seed=41)
    case = gen.make_case(cfg, DEV)
    rows = cfg.total_q * cfg.q_heads * cfg.seg_max
    part_o = torch.zeros(rows * 128, dtype=torch.float32, device=DEV)
    part_lse = torch.zeros(rows, dtype=torch.float32, device=DEV)
    plan = torch.zeros(skv.plan_words(cfg.bs, cfg.kv_heads, cfg.num_cus), dtype=torch.int32,
                       device=DEV)
    tok = torch.zeros(cfg.total_q, dtype=torch.int32, device=DEV)
    ftok = torch.zeros(cfg.total_q, dtype=torch.int32, device=DEV)
    out = torch.zeros((cfg.total_q, cfg.q_heads, 128), dtype=torch.bfloat16, device=DEV)
    fout = torch.zeros_like(out)
    lse = torch.zeros((cfg.total_q, cfg.q_heads), dtype=torch.float32, device=DEV)
    x = 16 // case.kv.element_size()
    B = case.kv.shape[0]
    kp = torch.zeros((B, 2, 128 // x, 16, x), dtype=case.kv.dtype, device=DEV)
    vp = torch.zeros((B, 2, 16 // x, 128, x), dtype=case.kv.dtype, device=DEV)
    # byte halves of the same pool for the in-place conversion
    flat = case.kv.view(torch.uint8).view(B, -1)
    hb = flat.shape[1] // 2
    kh0 = flat[:, :hb].contiguous().view(case.kv.dtype).view(kp.shape)
    vh0 = flat[:, hb:].contiguous().view(case.kv.dtype).view(vp.shape)
    kh, vh = kh0.clone(), vh0.clone()
    slots = torch.tensor([5, 40, -1, 77], dtype=torch.int64, device=DEV)
    knew = case.kv[:4, :, 0, :128].contiguous()
    vnew = case.kv[:4, :, 0, 128:].contiguous()
    kw = dict(kv_heads=cfg.kv_heads, max_q=cfg.max_q, num_cus=cfg.num_cus,
              seg_max=cfg.seg_max, kv_dtype=dtype, layout=layout, k_scale=case.k_scale,
              v_scale=case.v_scale, causal=cfg.causal)
    cout = torch.zeros_like(out)          # claimed units (opt-in order): to rounding

    def forward():                        # library calls only: nothing else is captured
        skv.kv_page_shuffle(case.kv, kp, vp)
        skv.kv_page_convert(kh, vh)       # in place: the halves become shuffled planes
        skv.kv_cache_write(knew, vnew, slots, kh, vh)
        kv_a, kv_b = (kp, vp) if layout == "shuffled" else (case.kv, None)
        skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q, cfg.kv_heads,
                       cfg.num_cus, cfg.seg_max, cfg.causal, plan=plan, tok_nseg=tok)
        skv.paged_decode_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens,
                              case.cu_seqlens_q, plan, tok, part_o=part_o, part_lse=part_lse,
                              out=out, out_lse=lse, **kw)
        skv.paged_decode_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens,
                              case.cu_seqlens_q, None, ftok, part_o=part_o, part_lse=part_lse,
                              out=fout, **kw)
        skv.paged_decode_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens,
                              case.cu_seqlens_q, plan, tok, part_o=part_o, part_lse=part_lse,
                              out=cout, **dict(kw, claim_units=True))

    def restore_halves():                 # eager, before every run
        kh.copy_(kh0)
        vh.copy_(vh0)

    def snap():
        return [t.clone() for t in (plan, tok, ftok, out, fout, lse, kh, vh, kp, vp)]

    restore_halves()
    forward()
    torch.cuda.synchronize()
    want = snap()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # warm-up on the capture stream
        restore_halves()
        forward()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    restore_halves()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward()
    names = ["plan", "tok", "ftok", "out", "fout", "lse", "kh", "vh", "kp", "vp"]
    for rep in range(4):
        for t in (plan, tok, ftok, out, fout, lse, kp, vp, cout):   # eager work between replays
            t.zero_()
        restore_halves()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        for n, a, b in zip(names, got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, n)
        d = (cout.float() - want[3].float()).abs().max().item()
        assert d <= (2e-2 if dtype == "fp8" else 1e-2), (rep, d)
    assert np.all(np.isfinite(out.float().cpu().numpy()))
