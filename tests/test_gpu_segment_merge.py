"""The segment kernel alone (skv_segment_attn) and the split reduce
(skv_split_reduce) as separate calls.

* Segment kernel + reduce, called one after the other, give the fused call's
  output and log-sum-exp bit for bit.
* Partials of two calls over disjoint key ranges, placed side by side in one
  buffer with tok_nseg counting both, merge into attention over the whole
  range (the reduce merges whatever partials it is given: [PR, Modifications],
  a token's segment count is all the reduce reads). Sequence i's first p_i
  pages go to call A without a mask (every query sees all of them, p_i pages
  <= L_i - q_i tokens) and the rest to call B with the bottom-right causal
  mask, which on the shorter range is the same mask; the merged result is
  compared with the oracle over the full sequences.
"""
import numpy as np
import pytest
import torch

import split_kv_paged_amd as skv
from gpu_harness import TOL, compare, run_oracle, say
from workloads import configs, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # name, seq_lens, q_lens, Hq, Hkv, dtype, layout
    ("bf16_rows64", [5, 40, 1500, 3333, 700], [4, 4, 3, 2, 4], 32, 2, "bf16", "standard"),
    ("fp8_rows32_shuf", [17, 900, 2049, 4100], [4, 1, 3, 2], 16, 2, "fp8", "shuffled"),
    ("bf16_valu_rows4", [64, 1000, 2500, 33], [1, 1, 1, 1], 8, 2, "bf16", "standard"),
    ("fp16_rows16", [300, 2000, 17, 999], [2, 1, 2, 2], 16, 2, "fp16", "standard"),
]


def _case(name, lens, ql, hq, hkv, dt, layout, causal=1):
    base = configs.FP8_KV if dt == "fp8" else configs.TINY
    cfg = gen.small_config(base, lens, ql, q_heads=hq, kv_heads=hkv, layout=layout,
                           causal=causal, num_cus=64, seg_max=16, seed=11, kv_dtype=dt)
    return gen.make_case(cfg, DEV)


def _kv(case):
    if case.cfg.layout == "shuffled":
        return skv.kv_page_shuffle(case.kv)
    return case.kv, None


def _attn_kw(case):
    cfg = case.cfg
    return dict(kv_heads=cfg.kv_heads, max_q=cfg.max_q, num_cus=cfg.num_cus,
                seg_max=cfg.seg_max, kv_dtype=cfg.kv_dtype, layout=cfg.layout,
                k_scale=case.k_scale, v_scale=case.v_scale, page_size=cfg.page_size)


def _parts(cfg, seg_max):
    rows = cfg.total_q * cfg.q_heads * seg_max
    return (torch.full((rows * cfg.head_dim,), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("spec", CASES, ids=lambda c: c[0])
def test_segment_then_reduce_equals_fused_call(spec):
    say("seg+reduce", spec[0])
    case = _case(*spec)
    cfg = case.cfg
    kv_a, kv_b = _kv(case)
    plan, tok = skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q, cfg.kv_heads,
                               cfg.num_cus, cfg.seg_max, cfg.causal, page_size=cfg.page_size)
    po, pl = _parts(cfg, cfg.seg_max)
    lse_f = torch.empty((cfg.total_q, cfg.q_heads), dtype=torch.float32, device=DEV)
    out_f, _ = skv.paged_decode_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens,
                                     case.cu_seqlens_q, plan, tok, causal=cfg.causal,
                                     part_o=po, part_lse=pl, out_lse=lse_f, **_attn_kw(case))
    po2, pl2 = _parts(cfg, cfg.seg_max)
    skv.segment_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens, case.cu_seqlens_q,
                     plan, tok, causal=cfg.causal, part_o=po2, part_lse=pl2, **_attn_kw(case))
    lse_s = torch.empty_like(lse_f)
    out_s, _ = skv.split_reduce(po2, pl2, tok, total_q=cfg.total_q, q_heads=cfg.q_heads,
                                seg_max=cfg.seg_max, head_dim=cfg.head_dim, out_lse=lse_s,
                                out_dtype="fp16" if cfg.kv_dtype == "fp16" else "bf16")
    torch.cuda.synchronize()
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_f.view(torch.int32), lse_s.view(torch.int32))


@pytest.mark.parametrize("spec", CASES, ids=lambda c: c[0])
def test_partials_of_two_calls_merge(spec):
    say("two-call merge", spec[0])
    case = _case(*spec)
    cfg = case.cfg
    kv_a, kv_b = _kv(case)
    P = cfg.page_size
    lens = np.asarray(cfg.seq_lens)
    ql = np.asarray(cfg.q_lens)
    # call A: each sequence's first p_i pages, all visible to its queries
    full = np.maximum((lens - ql) // P, 0)         # pages every query of sequence i sees
    p = (full + 1) // 2
    table = case.page_table.cpu().numpy()
    stride = table.shape[1]
    spare = int(table[0, -1])
    tab_b = np.full_like(table, spare)
    for i in range(cfg.bs):
        tab_b[i, :stride - p[i]] = table[i, p[i]:]
    lens_a = torch.as_tensor((p * P).astype(np.int32), device=DEV)
    lens_b = torch.as_tensor((lens - p * P).astype(np.int32), device=DEV)
    tb = torch.as_tensor(tab_b, device=DEV)
    kw = _attn_kw(case)
    S = cfg.seg_max
    # A: planned split over the leading pages, no mask
    plan_a, tok_a = skv.plan_build(lens_a, case.cu_seqlens_q, cfg.total_q, cfg.kv_heads,
                                   cfg.num_cus, S, 0, page_size=P)
    po_a, pl_a = _parts(cfg, S)
    skv.segment_attn(case.q, kv_a, kv_b, case.page_table, lens_a, case.cu_seqlens_q, plan_a,
                     tok_a, causal=0, part_o=po_a, part_lse=pl_a, **kw)
    # B: fixed split over the rest, causal
    po_b, pl_b = _parts(cfg, S)
    _, _, tok_b = skv.segment_attn(case.q, kv_a, kv_b, tb, lens_b, case.cu_seqlens_q, None,
                                   None, causal=1, part_o=po_b, part_lse=pl_b, **kw)
    torch.cuda.synchronize()
    # side by side: token t's A partials, then its B partials
    D, H = cfg.head_dim, cfg.q_heads
    a_o, a_l = po_a.view(cfg.total_q, H, S, D), pl_a.view(cfg.total_q, H, S)
    b_o, b_l = po_b.view(cfg.total_q, H, S, D), pl_b.view(cfg.total_q, H, S)
    m_o = torch.zeros((cfg.total_q, H, 2 * S, D), dtype=torch.float32, device=DEV)
    m_l = torch.full((cfg.total_q, H, 2 * S), float("nan"), dtype=torch.float32, device=DEV)
    na, nb = tok_a.cpu().tolist(), tok_b.cpu().tolist()
    for t in range(cfg.total_q):
        m_o[t, :, :na[t]] = a_o[t, :, :na[t]]
        m_l[t, :, :na[t]] = a_l[t, :, :na[t]]
        m_o[t, :, na[t]:na[t] + nb[t]] = b_o[t, :, :nb[t]]
        m_l[t, :, na[t]:na[t] + nb[t]] = b_l[t, :, :nb[t]]
    tok_m = torch.as_tensor(np.asarray(na) + np.asarray(nb), dtype=torch.int32, device=DEV)
    lse = torch.empty((cfg.total_q, H), dtype=torch.float32, device=DEV)
    out, _ = skv.split_reduce(m_o.view(-1), m_l.view(-1), tok_m, total_q=cfg.total_q, q_heads=H,
                              seg_max=2 * S, head_dim=D, out_lse=lse,
                              out_dtype="fp16" if cfg.kv_dtype == "fp16" else "bf16")
    torch.cuda.synchronize()
    assert max(na) > 0 and max(nb) > 0, "both calls hold keys"
    ref_out, ref_lse = run_oracle(case)
    r = compare(out.float().cpu().numpy().astype(np.float64),
                lse.cpu().numpy().astype(np.float64), ref_out, ref_lse, cfg.kv_dtype)
    say(spec[0], r)
    assert r["max_abs"] <= TOL[cfg.kv_dtype], r
    assert r["lse_err"] <= 1e-3, r
