"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs. Imported by tests only."""
import sys

import numpy as np
import torch

import oracle
import split_kv_paged_amd as skv
from workloads import gen

# max-abs on unit-scale inputs; fp16 (more mantissa than bf16) is held to the bf16 bar
TOL = {"bf16": 1e-2, "fp8": 2e-2, "fp16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_hip(case, layout=None, planes=None, poison_ws=True, num_cus=None, seg_max=None,
            causal=None, fixed=False, claim=False):
    """Plan + (optional shuffle) + attention + reduce on cuda:0. Returns a dict of
    host copies (plan, tok_nseg, out as float64, lse) plus the device planes.
    fixed=True runs the fixed split (no plan; the segment kernel writes tok_nseg,
    which starts out holding -7 so an unwritten entry shows). claim=True
    lets fp8 waves claim their units at run time (SKV_ATTN_CLAIM_UNITS);
    the default is the fixed, bit-reproducible order."""
    cfg = case.cfg
    layout = layout or cfg.layout
    num_cus = num_cus or cfg.num_cus
    seg_max = seg_max or cfg.seg_max
    causal = cfg.causal if causal is None else causal
    if fixed:
        plan = None
        tok = torch.full((cfg.total_q,), -7, dtype=torch.int32, device=case.q.device)
    else:
        plan, tok = skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q,
                                   cfg.kv_heads, num_cus, seg_max, causal,
                                   page_size=cfg.page_size)
    if layout == "shuffled" and planes is None:
        planes = skv.kv_page_shuffle(case.kv)
    rows = cfg.total_q * cfg.q_heads * seg_max
    fill = float("nan") if poison_ws else 0.0
    part_o = torch.full((rows * cfg.head_dim,), fill, dtype=torch.float32, device=case.q.device)
    part_lse = torch.full((rows,), fill, dtype=torch.float32, device=case.q.device)
    out_lse = torch.empty((cfg.total_q, cfg.q_heads), dtype=torch.float32, device=case.q.device)
    kv_a, kv_b = (planes if layout == "shuffled" else (case.kv, None))
    out, _ = skv.paged_decode_attn(
        case.q, kv_a, kv_b, case.page_table, case.seq_lens, case.cu_seqlens_q, plan, tok,
        kv_heads=cfg.kv_heads, max_q=cfg.max_q, num_cus=num_cus, seg_max=seg_max,
        kv_dtype=cfg.kv_dtype, layout=layout, k_scale=case.k_scale, v_scale=case.v_scale,
        causal=causal, part_o=part_o, part_lse=part_lse, out_lse=out_lse,
        page_size=cfg.page_size, claim_units=claim)
    torch.cuda.synchronize()
    return dict(plan=None if plan is None else plan.cpu().numpy().tolist(),
                tok=tok.cpu().numpy().tolist(),
                out=out.float().cpu().numpy().astype(np.float64),
                out_bits=gen.raw_u16(out), lse=out_lse.cpu().numpy().astype(np.float64),
                planes=planes)


def run_oracle(case, rows=None, causal=None):
    cfg = case.cfg
    q = oracle.decode_q(gen.raw_u16(case.q), cfg.kv_dtype)
    kv = gen.raw_kv(case)
    return oracle.decode_attention(
        q, kv, cfg.kv_dtype, case.page_table.cpu().numpy(), case.seq_lens.cpu().numpy(),
        case.cu_seqlens_q.cpu().numpy(), cfg.kv_heads, cfg.page_size,
        cfg.causal if causal is None else causal, cfg.k_scale, cfg.v_scale, rows=rows)


def oracle_plan(case, num_cus=None, seg_max=None, causal=None):
    cfg = case.cfg
    return oracle.plan_segments(cfg.seq_lens, case.cu_seqlens_q.cpu().numpy(), cfg.kv_heads,
                                cfg.page_size, num_cus or cfg.num_cus, seg_max or cfg.seg_max,
                                cfg.causal if causal is None else causal)


def compare(hip_out, hip_lse, ref_out, ref_lse, kv_dtype, rows=None):
    """max-abs error (the bar), plus relative RMS per row and lse error (reported)."""
    if rows is not None:
        idx = tuple(np.array(rows).T)
        hip_out, hip_lse = hip_out[idx], hip_lse[idx]
        ref_out, ref_lse = ref_out[idx], ref_lse[idx]
    assert np.all(np.isfinite(hip_out)), "non-finite output"
    err = np.abs(hip_out - ref_out)
    max_abs = float(err.max()) if err.size else 0.0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(hip_lse)), "lse finiteness differs"
    assert np.all(hip_lse[~fin] == -np.inf)
    dead = ~fin
    assert np.all(hip_out[dead] == 0.0), "rows that see no key must be zero"
    lse_err = float(np.abs(hip_lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    num = np.sqrt(((hip_out - ref_out) ** 2).sum(-1))
    den = np.sqrt((ref_out ** 2).sum(-1))
    rel = float((num[fin] / np.maximum(den[fin], 1e-30)).max()) if fin.any() else 0.0
    return dict(max_abs=max_abs, tol=TOL[kv_dtype], lse_err=lse_err, max_rel_rms=rel)
