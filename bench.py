"""Benchmark: paged split-KV decode/verify attention on one MI355X.

One step = one forward of one attention layer over a batch already resident
in HBM: the length-aware plan (plan_build), the segment kernel and the split
reduce. The metric is the attention call (segment + reduce): microseconds per
call and effective KV TB/s = sum_i L_i * kv_heads * 2 * head_dim * bytes / time,
also as a fraction of the 8 TB/s HBM peak. Per-kernel durations come from HIP
events recorded on the stream the kernels run on. For shuffled-page workloads
the standard->shuffled repack runs before the timed steps and is timed on its
own, as is the in-place conversion of the same pool received as byte halves
(and its inverse). A KV pool much smaller than 2 GiB (the fp8 batches) is
timed on several copies of itself used in turn, so that no call is served from
the lines the previous call left in the 256 MB last-level cache.

Prints ONE JSON line (rank 0). Default workload: the uniform verify batch
(bs=16 x 119k tokens, 4 query tokens, 32/2 heads, bf16). `--all` adds the other
workloads to the line under "workloads", among them the uniform and agentic
batches with an fp8 cache, the element type of the split-KV PR's own table.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# A KV pool small next to the 256 MB last-level cache is timed on several
# copies used in turn (together at least this many bytes, at most 8 copies),
# so that no call reads lines the previous call left in that cache.
ROTATE_BYTES = 2 << 30


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The first ~100 launches after the GPU has been idle run up to 40% slower
    # (clock/power ramp); 100 warmup steps put the timed region in steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="uniform_verify")
    ap.add_argument("--all", action="store_true", help="also time the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU-oracle time for the baseline sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


# the sources the segment-attention kernels are compiled from
SEGMENT_SOURCES = ("skv_attn.hip", "skv_attn_mfma.hip", "skv_attn_mfma_priv.hip", "skv_attn_valu.hip",
                   "skv_attn_gd.hip",
                   "skv_attn_common.h", "skv_internal.h")


def _code_only(text):
    """C++ source with comments removed and whitespace collapsed (string and
    character literals kept), so that editing a comment keeps the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the segment kernels' code (comments and layout ignored)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "split_kv_paged_amd", "csrc")
    for f in SEGMENT_SOURCES:
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(cfg_name, src_hash):
    """HBM bytes per segment-kernel launch from committed rocprofv3 PMC
    summaries, only if they were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "segment_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(cfg_name)
    if not e or e.get("kernel_source_hash") != src_hash:
        return None
    return e.get("hbm_bytes_per_launch")


def time_workload(cfg, steps, warmup, torch, skv, gen):
    dev = "cuda:0"
    case = gen.make_case(cfg, dev)
    st = torch.cuda.current_stream()
    res = {}
    kv_a, kv_b = case.kv, None
    if cfg.layout == "shuffled":
        kp, vp = skv.kv_page_shuffle(case.kv)
        for _ in range(max(warmup // 5, 2)):
            skv.kv_page_shuffle(case.kv, kp, vp)
        n = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(n):
            skv.kv_page_shuffle(case.kv, kp, vp)
        e1.record(st)
        torch.cuda.synchronize()
        sh_us = e0.elapsed_time(e1) * 1e3 / n
        moved = 2 * case.kv.numel() * case.kv.element_size()
        res["shuffle_us"] = sh_us
        res["shuffle_gbs"] = moved / sh_us / 1e3
        # in-place conversion of the same pool received as byte halves, and back
        B = case.kv.shape[0]
        flat = case.kv.view(torch.uint8).view(B, -1)
        hb = flat.shape[1] // 2
        x = 16 // case.kv.element_size()
        H, D = cfg.kv_heads, cfg.head_dim
        kh = flat[:, :hb].contiguous().view(case.kv.dtype).view(B, H, D // x, 16, x)
        vh = flat[:, hb:].contiguous().view(case.kv.dtype).view(B, H, 16 // x, D, x)
        for _ in range(max(warmup // 10, 2)):
            skv.kv_page_convert(kh, vh)
            skv.kv_page_convert(kh, vh, direction="to_standard")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        to_s = to_b = 0.0
        for _ in range(n):
            ev[0].record(st)
            skv.kv_page_convert(kh, vh)
            ev[1].record(st)
            skv.kv_page_convert(kh, vh, direction="to_standard")
            ev[2].record(st)
            torch.cuda.synchronize()
            to_s += ev[0].elapsed_time(ev[1]) * 1e3 / n
            to_b += ev[1].elapsed_time(ev[2]) * 1e3 / n
        res["convert_us"] = to_s
        res["convert_gbs"] = moved / to_s / 1e3
        res["convert_back_us"] = to_b
        res["convert_back_gbs"] = moved / to_b / 1e3
        del kh, vh, flat
        # cache writer: one decode step's new token per sequence into the planes
        tab = case.page_table
        last = (case.seq_lens.long() - 1).clamp(min=0)
        slots = tab.gather(1, (last // 16).view(-1, 1).int()).view(-1).long() * 16 + last % 16
        knew = torch.randn((cfg.bs, H, D), device=dev).to(case.kv.dtype)
        vnew = torch.randn((cfg.bs, H, D), device=dev).to(case.kv.dtype)
        for _ in range(5):
            skv.kv_cache_write(knew, vnew, slots, kp, vp)
        ev[0].record(st)
        for _ in range(n):
            skv.kv_cache_write(knew, vnew, slots, kp, vp)
        ev[1].record(st)
        torch.cuda.synchronize()
        res["cache_write_us"] = ev[0].elapsed_time(ev[1]) * 1e3 / n
        res["cache_write_tokens"] = cfg.bs
        # restore the planes for the attention steps
        skv.kv_page_shuffle(case.kv, kp, vp)
        kv_a, kv_b = kp, vp
    pool = sum(t.numel() * t.element_size() for t in (kv_a, kv_b) if t is not None)
    ncopy = max(1, min(8, -(-ROTATE_BYTES // pool)))
    kvs = [(kv_a, kv_b)] + [(kv_a.clone(), None if kv_b is None else kv_b.clone())
                            for _ in range(ncopy - 1)]
    res["kv_copies"] = ncopy
    rows = cfg.total_q * cfg.q_heads * cfg.seg_max
    part_o = torch.empty(rows * cfg.head_dim, dtype=torch.float32, device=dev)
    part_lse = torch.empty(rows, dtype=torch.float32, device=dev)
    out = torch.empty((cfg.total_q, cfg.q_heads, cfg.head_dim), dtype=skv.io_dtype(cfg.kv_dtype),
                      device=dev)
    odt = "fp16" if cfg.kv_dtype == "fp16" else "bf16"
    plan = torch.empty(skv.plan_words(cfg.bs, cfg.kv_heads, cfg.num_cus), dtype=torch.int32,
                       device=dev)
    tok = torch.empty(cfg.total_q, dtype=torch.int32, device=dev)
    kw = dict(kv_heads=cfg.kv_heads, max_q=cfg.max_q, num_cus=cfg.num_cus,
              seg_max=cfg.seg_max, kv_dtype=cfg.kv_dtype, layout=cfg.layout,
              k_scale=case.k_scale, v_scale=case.v_scale, causal=cfg.causal)

    def step(ev=None, i=0):
        kv_a, kv_b = kvs[i % ncopy]
        if ev:
            ev[0].record(st)
        skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q, cfg.kv_heads,
                       cfg.num_cus, cfg.seg_max, cfg.causal, plan=plan, tok_nseg=tok)
        if ev:
            ev[1].record(st)
        skv.segment_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens,
                         case.cu_seqlens_q, plan, tok, part_o=part_o, part_lse=part_lse, **kw)
        if ev:
            ev[2].record(st)
        skv.split_reduce(part_o, part_lse, tok, total_q=cfg.total_q, q_heads=cfg.q_heads,
                         seg_max=cfg.seg_max, head_dim=cfg.head_dim, out=out,
                         out_dtype=odt)
        if ev:
            ev[3].record(st)

    for i in range(warmup):
        step(i=i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i], i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    plan_us = sum(e[0].elapsed_time(e[1]) for e in evs) * 1e3 / steps
    seg_us = sum(e[1].elapsed_time(e[2]) for e in evs) * 1e3 / steps
    red_us = sum(e[2].elapsed_time(e[3]) for e in evs) * 1e3 / steps
    step_us = sum(e[0].elapsed_time(e[3]) for e in evs) * 1e3 / steps
    segs = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in evs)
    kvb = cfg.kv_bytes()
    call_us = seg_us + red_us
    res.update(dict(
        workload=cfg.name, kv_bytes=kvb, plan_us=plan_us, segment_us=seg_us,
        segment_us_p10=segs[len(segs) // 10], segment_us_p90=segs[(9 * len(segs)) // 10],
        segment_us_median=segs[len(segs) // 2],
        reduce_us=red_us, attn_us_per_call=call_us, step_us=step_us, wall_s=wall,
        kv_tb_s=kvb / call_us / 1e6, frac_of_hbm_peak=kvb / call_us / 1e3 / HBM_PEAK_GBS,
        segment_gb_s=kvb / seg_us / 1e3, plan_T=int(plan[0].item())))
    # the same attention call captured once in a HIP graph and replayed, as a
    # serving loop runs decode steps: launch gaps between segment and reduce go
    def attn_call(kv_a, kv_b):
        skv.segment_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens,
                         case.cu_seqlens_q, plan, tok, part_o=part_o, part_lse=part_lse, **kw)
        skv.split_reduce(part_o, part_lse, tok, total_q=cfg.total_q, q_heads=cfg.q_heads,
                         seg_max=cfg.seg_max, head_dim=cfg.head_dim, out=out,
                         out_dtype=odt)

    side = torch.cuda.Stream()
    side.wait_stream(st)
    with torch.cuda.stream(side):
        attn_call(*kvs[0])
    st.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for kv in kvs:                     # one graph per KV copy, replayed in turn
        graphs.append(torch.cuda.CUDAGraph())
        with torch.cuda.graph(graphs[-1]):
            attn_call(*kv)
    for i in range(warmup):
        graphs[i % ncopy].replay()
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        gev[i][0].record(st)
        graphs[i % ncopy].replay()
        gev[i][1].record(st)
    torch.cuda.synchronize()
    res["graph_us_per_call"] = sum(e[0].elapsed_time(e[1]) for e in gev) * 1e3 / steps
    res["graph_kv_tb_s"] = kvb / res["graph_us_per_call"] / 1e6
    del graphs

    # the fixed split on the same batch (no plan; the segment kernel writes the
    # per-token counts): the pages' A/B comparison, on these kernels
    def fixed_call(ev=None, i=0):
        kv_a, kv_b = kvs[i % ncopy]
        if ev:
            ev[0].record(st)
        skv.segment_attn(case.q, kv_a, kv_b, case.page_table, case.seq_lens,
                         case.cu_seqlens_q, None, tok, part_o=part_o, part_lse=part_lse, **kw)
        skv.split_reduce(part_o, part_lse, tok, total_q=cfg.total_q, q_heads=cfg.q_heads,
                         seg_max=cfg.seg_max, head_dim=cfg.head_dim, out=out,
                         out_dtype=odt)
        if ev:
            ev[1].record(st)

    for i in range(warmup):
        fixed_call(i=i)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        fixed_call(fev[i], i)
    torch.cuda.synchronize()
    fixed_us = sum(e[0].elapsed_time(e[1]) for e in fev) * 1e3 / steps
    res.update(fixed_split_us_per_call=fixed_us, fixed_split_kv_tb_s=kvb / fixed_us / 1e6,
               fixed_split_segments=_fixed_segments(cfg))
    del case, part_o, part_lse, out, kvs
    torch.cuda.empty_cache()
    return res


def _fixed_segments(cfg):
    """Segments per sequence of the fixed split: max(1, min(seg_max,
    pow2floor(num_cus / (bs * kv_heads))))."""
    q = cfg.num_cus // (cfg.bs * cfg.kv_heads)
    p = 1
    while p * 2 <= q:
        p *= 2
    return max(1, min(cfg.seg_max, p))


def cpu_baseline(cfg, min_seconds, gen, np):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the workload: all query rows of one sequence at a time, in order (wrapping
    around), until at least `min_seconds` of CPU work (and at most ~3x that)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    # inputs only for the sequences the sample can reach (generation is not timed)
    n_gen = min(cfg.bs, 8)
    sub = gen.small_config(cfg, cfg.seq_lens[:n_gen], cfg.q_lens[:n_gen])
    case = gen.make_case(sub, "cpu")
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    kv = gen.raw_kv(case)
    cu = case.cu_seqlens_q.numpy()
    table, lens = case.page_table.numpy(), case.seq_lens.numpy()
    elapsed, done, kv_bytes = 0.0, 0, 0
    while elapsed < min_seconds and done < 64:
        i = done % n_gen
        rows = [(t, h) for t in range(cu[i], cu[i + 1]) for h in range(cfg.q_heads)]
        t0 = time.perf_counter()
        oracle.decode_attention(q, kv, cfg.kv_dtype, table, lens, cu, cfg.kv_heads,
                                cfg.page_size, cfg.causal, cfg.k_scale, cfg.v_scale, rows=rows)
        elapsed += time.perf_counter() - t0
        kv_bytes += int(lens[i]) * cfg.kv_heads * 2 * cfg.head_dim * cfg.elem_bytes
        done += 1
    return {"value": kv_bytes / elapsed / 1e12, "unit": "TB/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(elapsed, 3),
            "sample": f"{cfg.name}: all query rows of {done} sequences taken in order "
                      f"(first {n_gen} of the batch, wrapping), {kv_bytes} KV bytes, "
                      f"numpy fp64 oracle",
            "host": platform.processor() or platform.machine(),
            "host_cpus": os.cpu_count()}


def main():
    a = _args()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import split_kv_paged_amd as skv
    from workloads import configs, gen

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    skv.load()
    if a.copy_probe:
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 1 << 30, "launches": 5}))
        return
    cfg = configs.BY_NAME[a.config]
    head = time_workload(cfg, a.steps, a.warmup, torch, skv, gen)
    props = torch.cuda.get_device_properties(0)
    src_hash = kernel_source_hash()
    traffic = traffic_from_profiles(cfg.name, src_hash)
    seg_gbs = head["segment_gb_s"]
    line = {
        "metric": "paged decode-attn effective KV TB/s (attention + reduce; us/call and "
                  "fraction of HBM peak alongside)",
        "value": round(head["kv_tb_s"], 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["step_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp16": "fp16", "fp8": "fp8-e4m3fn"}[cfg.kv_dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "bs": cfg.bs,
                   "total_kv_tokens": int(sum(cfg.seq_lens)), "q_heads": cfg.q_heads,
                   "kv_heads": cfg.kv_heads, "head_dim": cfg.head_dim,
                   "page_size": cfg.page_size, "kv_dtype": cfg.kv_dtype,
                   "layout": cfg.layout, "num_cus": cfg.num_cus, "seg_max": cfg.seg_max,
                   "parallelism": "single GPU", "kv_copies": head["kv_copies"]},
        "us_per_call": round(head["attn_us_per_call"], 2),
        "frac_of_hbm_peak": round(head["frac_of_hbm_peak"], 4),
        "breakdown_us": {k: round(head[k], 2) for k in
                         ("plan_us", "segment_us", "segment_us_median", "segment_us_p10",
                          "segment_us_p90", "reduce_us", "step_us")},
        "graph_replay": {"us_per_call": round(head["graph_us_per_call"], 2),
                         "kv_tb_s": round(head["graph_kv_tb_s"], 4)},
        "fixed_split": {"us_per_call": round(head["fixed_split_us_per_call"], 2),
                        "kv_tb_s": round(head["fixed_split_kv_tb_s"], 4),
                        "segments_per_seq": head["fixed_split_segments"]},
        "roofline": {"bound": "hbm", "kernel": "segment attention",
                     "achieved": round(seg_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(seg_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": head["kv_bytes"],
                     "traffic": traffic, "kernel_source_hash": src_hash},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
    }
    repack = {k: round(head[k], 2) for k in ("shuffle_us", "shuffle_gbs", "convert_us",
                                             "convert_gbs", "convert_back_us",
                                             "convert_back_gbs", "cache_write_us",
                                             "cache_write_tokens") if k in head}
    if repack:
        line["repack"] = repack
    if a.all:
        wl = []
        for c in configs.CONFIGS + configs.EXTRA:
            if c.name == cfg.name:
                continue
            r = time_workload(c, a.steps, a.warmup, torch, skv, gen)
            wl.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        line["workloads"] = wl
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, a.cpu_seconds, gen, np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
