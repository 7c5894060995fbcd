"""Benchmark: paged split-KV decode/verify attention on one MI355X.

One step = one forward of one attention layer over a batch already resident
in HBM: the length-aware plan (plan_build), the segment kernel and the split
reduce. The metric is the attention call (segment + reduce): microseconds per
call and effective KV TB/s = sum_i L_i * kv_heads * 2 * head_dim * bytes / time,
also as a fraction of the 8 TB/s HBM peak. Per-kernel durations come from HIP
events recorded on the stream the kernels run on.

Headline (`value`): the skewed agentic verify batch (bs 20, 2.32M tokens,
ragged 1..4 query tokens, 32/2 heads, bf16), the batch shape of the split-KV
PR's agentic rows (Benchmarking and Profiling). Every other workload is timed
the same way, each in a child process of its own started before this one
touches the GPU (so each starts from fresh device memory, as a serving process
that allocates its KV pool at startup), and reported under "workloads" in the
same JSON line (`--only` times the headline alone).

Each workload is timed in four arms: the planned split with an event
between every launch (plan, segment kernel, reduce: the per-kernel times and
the roofline), the planned call alone (segment + reduce between two events,
on the plan the step before built: `value`), the fixed split (no plan; the
PR's A/B baseline and its bs == 1 path) and the planned call replayed from a
HIP graph. An event between the call's two launches lengthens the call by
3-5 us, so only the first arm records one. The arms are interleaved: timed
step i runs all four, in an order rotated by i, so no arm gains or loses from
its position. Before the counted warm-up, the planned call is repeated until
the median duration of its last 20 segment launches is within 1% of the 20
before (at least 100 launches, at most --precondition-s seconds): after the
GPU has been idle, the first ~100 launches run up to 40% slower while clocks
ramp. That phase is reported under "precondition".

Every KV pool is timed on at least two copies used in turn (more when the
pool is small: together at least 4 GiB, at most 8 copies), one copy per call
whatever the arm, so no call reads lines the previous call left in the 256 MB
last-level cache.

For shuffled-page workloads the standard->shuffled repack, the in-place
conversion of the same pool received as byte halves (and its inverse) and a
cache write are timed on their own. "request_conversion" times the in-place
conversion of one received request's pages, layer by layer, at 4k and 16k
context on the geometry of the NixlConnector RFC's estimate.

`--summarize DIR` turns the rocprofv3 outputs of one workload (the kernel
trace and the two HBM counter runs whose commands it prints) into the
summaries under profiles/.

Prints ONE JSON line.
"""
import argparse
import csv
import collections
import glob
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "agentic_skew"
ROTATE_BYTES = 4 << 30          # KV copies used in turn: together at least this
ARMS = ("planned", "call", "fixed", "graph")


def _args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="time the --config workload alone")
    ap.add_argument("--workload-result", action="store_true",
                    help="time the --config workload and print its raw result as JSON "
                         "(the child-process form the default run uses for every workload "
                         "but the headline)")
    ap.add_argument("--precondition-s", type=float, default=3.0,
                    help="cap (seconds) of the clock pre-conditioning phase; 0 skips it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU-oracle time for the baseline sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write profiles/ summaries from the rocprofv3 outputs in DIR")
    return ap.parse_args(argv)


# the sources the segment-attention kernels are compiled from: the dispatch and
# the shared code, and one file per kernel family (by kernel-name prefix)
SEGMENT_COMMON = ("skv_attn.hip", "skv_attn_common.h", "skv_internal.h")
SEGMENT_KERNEL_FILES = (("seg_mfma_priv", "skv_attn_mfma_priv.hip"),
                        ("seg_mfma", "skv_attn_mfma.hip"),
                        ("seg_valu", "skv_attn_valu.hip"),
                        ("seg_gd", "skv_attn_gd.hip"))


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


def kernel_source_hash(kernel=None):
    """Hash of the code (comments and layout ignored) of the shared segment
    sources and of the file that defines `kernel` (a kernel name as the
    profiler prints it), or of every segment source when kernel is None."""
    files = list(SEGMENT_COMMON)
    for prefix, f in SEGMENT_KERNEL_FILES:
        if kernel is None:
            files.append(f)
        elif kernel.startswith(prefix):
            files.append(f)
            break
    h = hashlib.sha256()
    d = os.path.join(ROOT, "split_kv_paged_amd", "csrc")
    for f in files:
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(cfg_name):
    """(HBM bytes per segment-kernel launch, kernel, its source hash) from the
    committed rocprofv3 PMC summaries; the bytes are None unless they were
    taken on the current sources of the kernel that produced them."""
    p = os.path.join(ROOT, "profiles", "segment_traffic.json")
    if not os.path.exists(p):
        return None, None, kernel_source_hash()
    with open(p) as f:
        d = json.load(f)
    e = d.get(cfg_name)
    if not e:
        return None, None, kernel_source_hash()
    h = kernel_source_hash(e["kernel"])
    return (e.get("hbm_bytes_per_launch") if e.get("kernel_source_hash") == h else None,
            e["kernel"], h)


def _stats(xs):
    s = sorted(xs)
    n = len(s)
    return {"mean": sum(s) / n, "median": s[n // 2], "p10": s[n // 10], "p90": s[(9 * n) // 10]}


def _repack_timings(cfg, case, warmup, torch, skv, dev):
    """Shuffle, in-place conversion (and back) and one decode step's cache
    write on the workload's own pool; returns (timings, k_plane, v_plane)."""
    st = torch.cuda.current_stream()
    res = {}
    kp, vp = skv.kv_page_shuffle(case.kv)
    for _ in range(max(warmup, 2)):
        skv.kv_page_shuffle(case.kv, kp, vp)
    n = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(n):
        skv.kv_page_shuffle(case.kv, kp, vp)
    e1.record(st)
    torch.cuda.synchronize()
    moved = 2 * case.kv.numel() * case.kv.element_size()
    res["shuffle_us"] = e0.elapsed_time(e1) * 1e3 / n
    res["shuffle_gbs"] = moved / res["shuffle_us"] / 1e3
    B = case.kv.shape[0]
    flat = case.kv.view(torch.uint8).view(B, -1)
    hb = flat.shape[1] // 2
    x = 16 // case.kv.element_size()
    H, D, P = cfg.kv_heads, cfg.head_dim, cfg.page_size
    kh = flat[:, :hb].contiguous().view(case.kv.dtype).view(B, H, D // x, P, x)
    vh = flat[:, hb:].contiguous().view(case.kv.dtype).view(B, H, P // x, D, x)
    for _ in range(max(warmup, 2)):
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
    res.update(convert_us=to_s, convert_gbs=moved / to_s / 1e3, convert_back_us=to_b,
               convert_back_gbs=moved / to_b / 1e3)
    del kh, vh, flat
    tab = case.page_table
    last = (case.seq_lens.long() - 1).clamp(min=0)
    slots = tab.gather(1, (last // P).view(-1, 1).int()).view(-1).long() * P + last % P
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
    skv.kv_page_shuffle(case.kv, kp, vp)     # restore the planes for attention
    return res, kp, vp


# One request's pages converted on arrival, on the geometry of the NixlConnector
# RFC's estimate (Proposed Change, 4. Convert: a Qwen3-8B request carries 0.6 GB
# of bf16 KV at 4k context and 2.4 GB at 16k; generic torch ops would take
# roughly 1-2.5 ms and 3-10 ms): 36 layers of 8 kv heads, head dim 128, 16-token
# pages, one in-place conversion call per layer over the request's received
# blocks, which lie scattered in a layer pool twice their number.
REQUEST_GEOMETRY = {"layers": 36, "kv_heads": 8, "head_dim": 128, "page_size": 16}
RFC_TORCH_ESTIMATE_MS = {4096: [1.0, 2.5], 16384: [3.0, 10.0]}


def time_request_conversion(ctx, torch, skv, reps=10):
    dev = "cuda:0"
    st = torch.cuda.current_stream()
    L, H, D, P = (REQUEST_GEOMETRY[k] for k in ("layers", "kv_heads", "head_dim", "page_size"))
    x = 8                                    # bf16: 16-byte chunks of 8 elements
    nb = -(-ctx // P)
    pool = 2 * nb
    g = torch.Generator(device=dev)
    g.manual_seed(ctx)
    layers = []
    for _ in range(L):
        kp = torch.randint(-32768, 32768, (pool, H, D // x, P, x), dtype=torch.int16,
                           device=dev, generator=g).view(torch.bfloat16)
        vp = torch.randint(-32768, 32768, (pool, H, P // x, D, x), dtype=torch.int16,
                           device=dev, generator=g).view(torch.bfloat16)
        ids = torch.randperm(pool, device=dev, generator=g)[:nb].to(torch.int32)
        layers.append((kp, vp, ids))

    def request(direction):
        for kp, vp, ids in layers:
            skv.kv_page_convert(kp, vp, block_ids=ids, direction=direction)

    for _ in range(2):
        request("to_shuffled")
        request("to_standard")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(reps):
        e0.record(st)
        request("to_shuffled")
        e1.record(st)
        request("to_standard")               # untimed: the next pass reads fresh halves
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    kv_bytes = nb * L * 2 * H * P * D * 2    # the request's K and V, all layers
    mean = sum(ms) / len(ms)
    return {"context_tokens": ctx, **REQUEST_GEOMETRY, "kv_bytes": kv_bytes,
            "ms_per_request": mean, "us_per_layer": mean * 1e3 / L,
            "read_write_tb_s": 2 * kv_bytes / (mean * 1e-3) / 1e12,
            "rfc_torch_estimate_ms": RFC_TORCH_ESTIMATE_MS.get(ctx)}


def time_workload(cfg, a, torch, skv, gen, with_schedule=False):
    dev = "cuda:0"
    st = torch.cuda.current_stream()
    case = gen.make_case(cfg, dev)
    res = {"workload": cfg.name, "note": cfg.note}
    kv_a, kv_b = case.kv, None
    if cfg.layout == "shuffled":
        rp, kv_a, kv_b = _repack_timings(cfg, case, a.warmup, torch, skv, dev)
        res["repack"] = rp
        case.kv = None                       # the standard pool is not read by attention
    pool = sum(t.numel() * t.element_size() for t in (kv_a, kv_b) if t is not None)
    ncopy = max(2, min(8, -(-ROTATE_BYTES // pool)))
    kvs = [(kv_a, kv_b)] + [(kv_a.clone(), None if kv_b is None else kv_b.clone())
                            for _ in range(ncopy - 1)]
    res["kv_copies"] = ncopy
    rows = cfg.total_q * cfg.q_heads * cfg.seg_max
    part_o = torch.empty(rows * cfg.head_dim, dtype=torch.float32, device=dev)
    part_lse = torch.empty(rows, dtype=torch.float32, device=dev)
    iot = skv.io_dtype(cfg.kv_dtype)
    out = torch.empty((cfg.total_q, cfg.q_heads, cfg.head_dim), dtype=iot, device=dev)
    fout = torch.empty_like(out)
    odt = "fp16" if cfg.kv_dtype == "fp16" else "bf16"
    plan = torch.empty(skv.plan_words(cfg.bs, cfg.kv_heads, cfg.num_cus), dtype=torch.int32,
                       device=dev)
    tok = torch.empty(cfg.total_q, dtype=torch.int32, device=dev)
    ftok = torch.empty(cfg.total_q, dtype=torch.int32, device=dev)
    kw = dict(kv_heads=cfg.kv_heads, max_q=cfg.max_q, num_cus=cfg.num_cus,
              seg_max=cfg.seg_max, kv_dtype=cfg.kv_dtype, layout=cfg.layout,
              k_scale=case.k_scale, v_scale=case.v_scale, causal=cfg.causal,
              page_size=cfg.page_size)
    red = dict(total_q=cfg.total_q, q_heads=cfg.q_heads, seg_max=cfg.seg_max,
               head_dim=cfg.head_dim, out_dtype=odt)
    calls = [0]                              # KV copy used by the next call, any arm
    schedule = []

    def log(phase, arm):
        if schedule and schedule[-1][0] == phase and schedule[-1][1] == arm:
            schedule[-1][2] += 1
        else:
            schedule.append([phase, arm, 1])

    def next_kv():
        kv = kvs[calls[0] % ncopy]
        calls[0] += 1
        return kv

    def seg_reduce(kv, p, t, o):
        skv.segment_attn(case.q, kv[0], kv[1], case.page_table, case.seq_lens,
                         case.cu_seqlens_q, p, t, part_o=part_o, part_lse=part_lse, **kw)
        skv.split_reduce(part_o, part_lse, t, out=o, **red)

    def planned(ev=None):
        kv = next_kv()
        if ev:
            ev[0].record(st)
        skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q, cfg.kv_heads,
                       cfg.num_cus, cfg.seg_max, cfg.causal, plan=plan, tok_nseg=tok,
                       page_size=cfg.page_size)
        if ev:
            ev[1].record(st)
        skv.segment_attn(case.q, kv[0], kv[1], case.page_table, case.seq_lens,
                         case.cu_seqlens_q, plan, tok, part_o=part_o, part_lse=part_lse, **kw)
        if ev:
            ev[2].record(st)
        skv.split_reduce(part_o, part_lse, tok, out=out, **red)
        if ev:
            ev[3].record(st)

    def call(ev=None):
        kv = next_kv()
        if ev:
            ev[0].record(st)
        seg_reduce(kv, plan, tok, out)
        if ev:
            ev[1].record(st)

    def fixed(ev=None):
        kv = next_kv()
        if ev:
            ev[0].record(st)
        skv.segment_attn(case.q, kv[0], kv[1], case.page_table, case.seq_lens,
                         case.cu_seqlens_q, None, ftok, part_o=part_o, part_lse=part_lse,
                         **kw)
        skv.split_reduce(part_o, part_lse, ftok, out=fout, **red)
        if ev:
            ev[1].record(st)

    # the planned call (segment + reduce, plan built beforehand) captured once
    # per KV copy and replayed, as a serving loop runs decode steps
    planned()
    log("plan for capture", "planned")
    side = torch.cuda.Stream()
    side.wait_stream(st)
    with torch.cuda.stream(side):
        seg_reduce(kvs[0], plan, tok, out)
    log("capture warm-up", "graph")
    st.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for kv in kvs:
        graphs.append(torch.cuda.CUDAGraph())
        with torch.cuda.graph(graphs[-1]):
            seg_reduce(kv, plan, tok, out)

    def graph(ev=None):
        i = calls[0] % ncopy
        calls[0] += 1
        if ev:
            ev[0].record(st)
        graphs[i].replay()
        if ev:
            ev[1].record(st)

    run = {"planned": planned, "call": call, "fixed": fixed, "graph": graph}
    nev = {"planned": 4, "call": 2, "fixed": 2, "graph": 2}

    # clock pre-conditioning: the planned call until its segment-kernel time settles
    t0 = time.perf_counter()
    pre, meds, converged = [], [], False
    while a.precondition_s > 0:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(20)]
        for e in evs:
            planned(e)
            log("precondition", "planned")
        torch.cuda.synchronize()
        pre += [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
        meds.append(sorted(pre[-20:])[10])
        if len(pre) >= 100 and abs(meds[-1] - meds[-2]) <= 0.01 * meds[-2]:
            converged = True
            break
        if time.perf_counter() - t0 > a.precondition_s:
            break
    res["precondition"] = {"launches": len(pre), "seconds": round(time.perf_counter() - t0, 3),
                           "converged": converged,
                           "segment_us_first20_median": round(meds[0], 2) if meds else None,
                           "segment_us_last20_median": round(meds[-1], 2) if meds else None}

    def order(i):
        return ARMS[i % len(ARMS):] + ARMS[:i % len(ARMS)]

    for i in range(a.warmup):
        for arm in order(i):
            run[arm]()
            log("warm-up", arm)
    torch.cuda.synchronize()
    evs = {arm: [] for arm in ARMS}
    t0 = time.perf_counter()
    for i in range(a.steps):
        for arm in order(i):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(nev[arm])]
            run[arm](e)
            evs[arm].append(e)
            log("timed", arm)
    torch.cuda.synchronize()
    res["wall_s"] = time.perf_counter() - t0
    us = lambda e, i, j: e[i].elapsed_time(e[j]) * 1e3
    kvb = cfg.kv_bytes()
    pl = evs["planned"]
    p_call = [us(e, 1, 3) for e in pl]
    p_seg = [us(e, 1, 2) for e in pl]
    c_call = [us(e, 0, 1) for e in evs["call"]]
    f_call = [us(e, 0, 1) for e in evs["fixed"]]
    g_call = [us(e, 0, 1) for e in evs["graph"]]
    call = sum(c_call) / len(c_call)
    seg = sum(p_seg) / len(p_seg)
    res.update(
        kv_bytes=kvb, us_per_call=call, kv_tb_s=kvb / call / 1e6,
        frac_of_hbm_peak=kvb / call / 1e3 / HBM_PEAK_GBS, segment_us=seg,
        segment_gb_s=kvb / seg / 1e3, plan_T=int(plan[0].item()),
        call={"call_us": _stats(c_call), "kv_tb_s": kvb / call / 1e6},
        planned={"call_us": _stats(p_call), "segment_us": _stats(p_seg),
                 "plan_us": sum(us(e, 0, 1) for e in pl) / len(pl),
                 "reduce_us": sum(us(e, 2, 3) for e in pl) / len(pl),
                 "step_us": sum(us(e, 0, 3) for e in pl) / len(pl)},
        fixed={"call_us": _stats(f_call), "segments_per_seq": _fixed_segments(cfg),
               "kv_tb_s": kvb / (sum(f_call) / len(f_call)) / 1e6},
        graph={"call_us": _stats(g_call), "kv_tb_s": kvb / (sum(g_call) / len(g_call)) / 1e6})
    # the planned and the fixed split on the same inputs: the PR's accuracy
    # check (they differ only by the fp32 summation order across segments)
    planned()
    log("accuracy check", "planned")
    fixed()
    log("accuracy check", "fixed")
    torch.cuda.synchronize()
    res["plan_vs_fixed_max_abs"] = float((out.float() - fout.float()).abs().max().item())
    if with_schedule:
        res["segment_launch_schedule"] = schedule
    del graphs, case, part_o, part_lse, out, fout, kvs
    torch.cuda.empty_cache()
    return res


def _child_workload(name, a):
    """One workload timed by a child process (a fresh device memory state)."""
    cmd = [sys.executable, os.path.abspath(__file__), "--workload-result", "--config", name,
           "--steps", str(a.steps), "--warmup", str(a.warmup),
           "--precondition-s", str(a.precondition_s)]
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if p.returncode != 0:
        raise RuntimeError(f"workload {name} failed ({p.returncode}): {p.stderr[-2000:]}")
    return json.loads([l for l in p.stdout.splitlines() if l.startswith("{")][-1])


def _device_clocks():
    """Peak engine and memory clocks (MHz) as the HIP runtime reports them."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return {}
    out = {}
    # hipDeviceAttributeClockRate = 5, hipDeviceAttributeMemoryClockRate = 60 (kHz)
    for name, attr in (("engine_clock_mhz", 5), ("memory_clock_mhz", 60)):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0:
            out[name] = v.value // 1000
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


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
    q = oracle.decode_q(gen.raw_u16(case.q), cfg.kv_dtype)
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
            "host": _cpu_model(), "host_cpus": os.cpu_count()}


def _round(x):
    if isinstance(x, float):
        return round(x, 4)
    if isinstance(x, dict):
        return {k: _round(v) for k, v in x.items()}
    if isinstance(x, list):
        return [_round(v) for v in x]
    return x


# ---- profile summaries (rocprofv3 outputs -> profiles/) ----------------------

def _short(name):
    return name.replace("skv::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def _one(d, pat):
    got = glob.glob(os.path.join(d, pat))
    if not got:
        raise FileNotFoundError(os.path.join(d, pat))
    return got[0]


def _bench_line(path):
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                return json.loads(line)
    raise ValueError(f"no bench JSON line in {path}")


def _arm_of_segment_launches(line):
    """(phase, arm) of every segment-kernel launch, in launch order, from the
    schedule the profiled bench run printed."""
    sched = line.get("segment_launch_schedule")
    if sched is None:
        raise ValueError("the profiled run must use --only (it prints the launch schedule)")
    return [(ph, arm) for ph, arm, n in sched for _ in range(n)]


def _counter_per_dispatch(path):
    out = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            out[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: [v for _, v in sorted(vs)] for k, vs in out.items()}


PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o trace -- "
             "python3 bench.py --only --config {wl} --no-cpu-baseline > {d}/trace.json",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o fetch -- "
             "python3 bench.py --only --config {wl} --steps 3 --warmup 1 --precondition-s 0 "
             "--no-cpu-baseline > {d}/fetch.json",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o write -- "
             "python3 bench.py --only --config {wl} --steps 3 --warmup 1 --precondition-s 0 "
             "--no-cpu-baseline > {d}/write.json",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {c}/fetch -o cf -- "
                  "python3 bench.py --copy-probe",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {c}/write -o cw -- "
                  "python3 bench.py --copy-probe",
}


def summarize(d, copy_dir=None, out_dir=None):
    """Kernel-trace and HBM-counter summaries of one profiled workload.

    d holds trace/, fetch/, write/ and the bench lines trace.json, fetch.json,
    write.json written by the PROFILE_CMDS commands; copy_dir (default: the
    sibling p_copy/) the two counter runs of the plain 1 GiB copy used to
    scale the counters. Writes <workload>_kernel_trace.md and
    <workload>_pmc.md and updates segment_traffic.json in out_dir (default
    profiles/)."""
    d = d.rstrip("/")
    copy_dir = copy_dir or os.path.join(os.path.dirname(d), "p_copy")
    tline = _bench_line(os.path.join(d, "trace.json"))
    wl = tline["config"]["workload"].split(":")[0]
    rel = lambda p: os.path.relpath(p, ROOT)
    fmt = dict(d=rel(d), wl=wl, c=rel(copy_dir))
    prof = out_dir or os.path.join(ROOT, "profiles")
    # kernel trace, per arm and phase
    with open(_one(os.path.join(d, "trace"), "*kernel_trace.csv")) as f:
        kt = [r for r in csv.DictReader(f) if "skv::" in r["Kernel_Name"]]
    kt.sort(key=lambda r: int(r["Start_Timestamp"]))
    seg = [r for r in kt if "seg_" in _short(r["Kernel_Name"])]
    seg_kernel = _short(seg[0]["Kernel_Name"]) if seg else None
    # the sources of the segment kernel that ran, as they are now (the
    # summary is made right after the profiled run, from the same tree)
    src_hash = kernel_source_hash(seg_kernel)
    arms = _arm_of_segment_launches(tline)
    if len(arms) != len(seg):
        raise ValueError(f"{len(seg)} segment launches traced, schedule lists {len(arms)}")
    groups = collections.defaultdict(list)
    for (ph, arm), r in zip(arms, seg):
        groups[(ph, arm)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    # the reduce follows its segment launch; the plan precedes planned launches
    by_name = collections.defaultdict(list)
    for r in kt:
        by_name[_short(r["Kernel_Name"])].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    L = [f"# Kernel trace: {wl}", "",
         "Command (repository root, one MI355X; the bench line it prints is the source of the",
         "launch schedule used below):", "", "```", PROFILE_CMDS["trace"].format(**fmt), "```",
         "", f"Bench line of this run: {tline['us_per_call']} us per call, "
             f"{tline['value']} TB/s (the call arm, events); kernel sources hash {src_hash}.", "",
         "Segment kernel, per arm (the timed steps interleave the arms in rotated order):",
         "", "| phase | arm | launches | avg us | median us | p10 us | p90 us | KV TB/s (avg) |",
         "|---|---|---|---|---|---|---|---|"]
    kvb = tline["roofline"]["algorithmic_bytes_per_launch"]
    for (ph, arm), v in groups.items():
        s = _stats(v)
        L.append(f"| {ph} | {arm} | {len(v)} | {s['mean']:.1f} | {s['median']:.1f} | "
                 f"{s['p10']:.1f} | {s['p90']:.1f} | {kvb / s['mean'] / 1e6:.3f} |")
    L += ["", "Every launch of every library kernel (all phases):", "",
          "| kernel | launches | avg us | min us | max us |", "|---|---|---|---|---|"]
    for k, v in by_name.items():
        L.append(f"| {k} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    timed = groups.get(("timed", "planned"))
    if timed:
        L += ["", f"Timed planned launches: segment kernel {sum(timed) / len(timed):.1f} us = "
                  f"{kvb / (sum(timed) / len(timed)) / 1e3:.1f} GB/s = "
                  f"{kvb / (sum(timed) / len(timed)) / 1e3 / HBM_PEAK_GBS:.3f} of the 8 TB/s peak "
                  f"({kvb} algorithmic KV bytes per launch)."]
    os.makedirs(prof, exist_ok=True)
    with open(os.path.join(prof, f"{wl}_kernel_trace.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    # HBM counters, scaled by what they read for a plain 1 GiB copy
    copy_kib = (1 << 30) / 1024
    cf = _counter_per_dispatch(_one(os.path.join(copy_dir, "fetch"), "*counter_collection.csv"))
    cw = _counter_per_dispatch(_one(os.path.join(copy_dir, "write"), "*counter_collection.csv"))
    cfv = [v for k, vs in cf.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs]
    cwv = [v for k, vs in cw.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs]
    f_scale = copy_kib / (sum(cfv) / len(cfv))
    w_scale = copy_kib / (sum(cwv) / len(cwv))
    fline = _bench_line(os.path.join(d, "fetch.json"))
    fc = _counter_per_dispatch(_one(os.path.join(d, "fetch"), "*counter_collection.csv"))
    wc = _counter_per_dispatch(_one(os.path.join(d, "write"), "*counter_collection.csv"))
    farms = _arm_of_segment_launches(fline)
    L = [f"# HBM traffic per launch: {wl}", "",
         "Commands (repository root; one counter per run, then the calibration copy):", "",
         "```"] + [PROFILE_CMDS[k].format(**fmt) for k in ("fetch", "write", "copy_fetch",
                                                            "copy_write")] + [
         f"python3 bench.py --summarize {fmt['d']}", "```", "",
         f"Calibration (plain 1 GiB device copy): FETCH_SIZE reads {sum(cfv) / len(cfv):.0f} KiB "
         f"for 1048576 KiB (scale {f_scale:.4f}); WRITE_SIZE reads {sum(cwv) / len(cwv):.0f} KiB "
         f"(scale {w_scale:.4f}).", f"Kernel sources hash {src_hash}.", "",
         "Per dispatch, averaged; the segment kernel over its planned-arm dispatches only.", "",
         "| kernel | dispatches | FETCH_SIZE raw KiB | WRITE_SIZE raw KiB | read bytes (scaled) | "
         "written bytes (scaled) | (read + written) / algorithmic KV bytes |",
         "|---|---|---|---|---|---|---|"]
    traffic = {}
    for k in fc:
        if "skv::" not in k:
            continue
        name = _short(k)
        fk, wk = fc[k], wc.get(k, [0.0])
        if name.startswith("seg_"):
            if len(fk) != len(farms) or len(wk) != len(farms):
                raise ValueError(f"{name}: {len(fk)}/{len(wk)} dispatches, "
                                 f"schedule lists {len(farms)}")
            fk = [v for v, (ph, arm) in zip(fk, farms) if arm == "planned"]
            wk = [v for v, (ph, arm) in zip(wk, farms) if arm == "planned"]
        fr, wr = sum(fk) / len(fk), sum(wk) / len(wk)
        rb, wb = fr * 1024 * f_scale, wr * 1024 * w_scale
        ratio = f"{(rb + wb) / kvb:.4f}" if name.startswith("seg_") else "-"
        L.append(f"| {name} | {len(fk)} | {fr:.1f} | {wr:.1f} | {rb:.4e} | {wb:.4e} | {ratio} |")
        if name.startswith("seg_"):
            traffic[wl] = {"kernel": name, "kernel_source_hash": src_hash,
                           "hbm_bytes_per_launch": round(rb + wb), "read_bytes": round(rb),
                           "write_bytes": round(wb), "algorithmic_bytes_per_launch": kvb,
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                           "source": f"profiles/{wl}_pmc.md"}
    with open(os.path.join(prof, f"{wl}_pmc.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    tj = os.path.join(prof, "segment_traffic.json")
    old = {}
    if os.path.exists(tj):
        with open(tj) as f:
            old = json.load(f)
    old.update(traffic)
    with open(tj, "w") as f:
        json.dump(old, f, indent=1, sort_keys=True)
        f.write("\n")
    return traffic


def main(argv=None):
    a = _args(argv)
    if a.summarize:
        print(json.dumps(summarize(a.summarize)))
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU (the kernel on one GPU's share); "
                                   "--gpus must be 1", "n_gpus": a.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import split_kv_paged_amd as skv
    from workloads import configs, gen

    # every workload but the headline in a child process of its own, started
    # before this process touches the GPU: within one process, a workload
    # timed after others ran 3-4% slower (device memory handed out after
    # earlier pools were freed), while a serving process allocates its KV pool
    # once, at startup
    others = []
    if not (a.only or a.workload_result or a.copy_probe):
        for c in configs.CONFIGS + configs.EXTRA + configs.BS1:
            if c.name == a.config:
                continue
            r = _child_workload(c.name, a)
            others.append(r)
            print(f"timed {c.name}: {r['us_per_call']:.1f} us per call", file=sys.stderr,
                  flush=True)

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
    if a.workload_result:
        print(json.dumps(_round(time_workload(cfg, a, torch, skv, gen))), flush=True)
        return
    head = time_workload(cfg, a, torch, skv, gen, with_schedule=a.only)
    props = torch.cuda.get_device_properties(0)
    traffic, traffic_kernel, src_hash = traffic_from_profiles(cfg.name)
    seg_gbs = head["segment_gb_s"]
    line = {
        "metric": "paged decode-attn effective KV TB/s (attention + reduce; us/call and "
                  "fraction of HBM peak alongside)",
        "value": round(head["kv_tb_s"], 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["planned"]["step_us"] / 1e3, 5),
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
        "us_per_call": round(head["us_per_call"], 2),
        "frac_of_hbm_peak": round(head["frac_of_hbm_peak"], 4),
        "arms": _round({k: head[k] for k in ARMS}),
        "plan_vs_fixed_max_abs": head["plan_vs_fixed_max_abs"],
        "precondition": head["precondition"],
        "roofline": {"bound": "hbm", "kernel": "segment attention",
                     "achieved": round(seg_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(seg_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": head["kv_bytes"],
                     "traffic": traffic, "traffic_kernel": traffic_kernel,
                     "kernel_source_hash": src_hash},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""), **_device_clocks()},
    }
    if "segment_launch_schedule" in head:
        line["segment_launch_schedule"] = head["segment_launch_schedule"]
    if not a.only:
        keep = ("workload", "note", "kv_bytes", "us_per_call", "kv_tb_s", "frac_of_hbm_peak",
                "segment_us", "segment_gb_s", "plan_T", "planned", "call", "fixed", "graph",
                "plan_vs_fixed_max_abs", "precondition", "kv_copies", "repack")
        wl = [_round({k: r[k] for k in keep if k in r}) for r in others]
        line["workloads"] = wl
        line["request_conversion"] = [_round(time_request_conversion(c, torch, skv))
                                      for c in sorted(RFC_TORCH_ESTIMATE_MS)]
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, a.cpu_seconds, gen, np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
