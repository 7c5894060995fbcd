"""GPU parity (through the C ABI) of the cache writer into shuffled pages:
bit-exact against the CPU oracle, and a decode step that writes the newest
tokens and then attends over them."""
import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_amd as skv
from gpu_harness import TOL, compare, run_oracle, say
from workloads import configs, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128
PAGE = 16            # attention pages


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skv.load()
    yield
    torch.cuda.synchronize()


def _dev(a, e):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if e == 2 else
                            np.ascontiguousarray(a)).to(DEV)


def _host(t, e):
    a = t.cpu().numpy()
    return a.view(np.uint16) if e == 2 else a


@pytest.mark.parametrize("e,H,N,D", [(2, 1, 16, D), (2, 2, 16, D), (2, 8, 16, D), (1, 2, 16, D),
                                     (1, 8, 16, D), (2, 3, 32, D), (1, 4, 32, D),
                                     (2, 2, 16, 64), (1, 3, 32, 64), (2, 3, 16, 256),
                                     (1, 2, 32, 256)])
def test_cache_write_bit_exact(e, H, N, D):
    """Bit-exact against the oracle, with padding slots (-1) and slots at or
    past the end of the cache (skipped) mixed in."""
    say("cache write", e, H, N, D)
    rng = np.random.default_rng(40 + 3 * H + e + D)
    dt = np.uint16 if e == 2 else np.uint8
    x = 16 // e
    B, T = 9, 70
    pad = 3 * x                                            # strided token rows
    kfull = rng.integers(0, 1 << (8 * e), size=(T, H * D + pad)).astype(dt)
    vfull = rng.integers(0, 1 << (8 * e), size=(T, H * D + pad)).astype(dt)
    slots = rng.choice(B * N, size=T, replace=False).astype(np.int64)
    slots[[0, 11, 40]] = -1                                # padding tokens
    slots[[5, 23, 61]] = [B * N, B * N + 7, 1 << 40]       # past the cache: skipped
    kp0 = rng.integers(0, 1 << (8 * e), size=(B, H, D // x, N, x)).astype(dt)
    vp0 = rng.integers(0, 1 << (8 * e), size=(B, H, N // x, D, x)).astype(dt)
    kp, vp = _dev(kp0, e), _dev(vp0, e)
    kd, vd = _dev(kfull, e), _dev(vfull, e)
    key = kd[:, :H * D].view(T, H, D)
    val = vd[:, :H * D].view(T, H, D)
    skv.kv_cache_write(key, val, torch.as_tensor(slots, device=DEV), kp, vp)
    torch.cuda.synchronize()
    wk, wv = oracle.write_tokens_shuffled(kp0, vp0, kfull[:, :H * D].reshape(T, H, D),
                                          vfull[:, :H * D].reshape(T, H, D), slots)
    assert np.array_equal(_host(kp, e), wk)
    assert np.array_equal(_host(vp, e), wv)


@pytest.mark.parametrize("P", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_step_writes_then_attends(dtype, P):
    """A verify step: each sequence's last q tokens are written into the
    shuffled cache through their slots, then attention reads them. Against the
    oracle writing the same tokens into standard pages."""
    say("write+attend", dtype, P)
    base = configs.FP8_KV if dtype == "fp8" else configs.TINY
    lens, ql = [40, 300, 17, 1000, 2], [2, 4, 1, 3, 1]
    cfg = gen.small_config(base, lens, ql, q_heads=16, kv_heads=2, layout="shuffled",
                           num_cus=64, seg_max=16, seed=21, page_size=P)
    case = gen.make_case(cfg, DEV)
    e = 2 if dtype == "bf16" else 1
    H = cfg.kv_heads
    table = case.page_table.cpu().numpy()
    slots = []
    for i, (L, q) in enumerate(zip(lens, ql)):
        for pos in range(L - q, L):
            slots.append(int(table[i, pos // P]) * P + pos % P)
    slots = np.array(slots, dtype=np.int64)
    T = len(slots)
    # new K/V codes: copies of other real tokens' rows (unit-scale values of the
    # batch's own distribution), so the step changes what attention sees
    rng = np.random.default_rng(8)
    std0 = gen.raw_kv(case)
    real = [(i, p) for i, L in enumerate(lens) for p in range(L)]
    pick = rng.choice(len(real), size=(2, T))
    kv_new = np.empty((2, T, H, D), dtype=std0.dtype)
    for w in range(2):
        for t in range(T):
            i, pos = real[pick[w, t]]
            row = std0[int(table[i, pos // P]), :, pos % P]
            kv_new[w, t] = row[:, :D] if w == 0 else row[:, D:]
    kp, vp = skv.kv_page_shuffle(case.kv)
    key = _dev(kv_new[0], e).view(T, H, D)
    val = _dev(kv_new[1], e).view(T, H, D)
    if dtype == "bf16":
        key, val = key.view(torch.bfloat16), val.view(torch.bfloat16)
    skv.kv_cache_write(key, val, torch.as_tensor(slots, device=DEV), kp, vp)
    plan, tok = skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q, H,
                               cfg.num_cus, cfg.seg_max, cfg.causal, page_size=P)
    out_lse = torch.empty((cfg.total_q, cfg.q_heads), dtype=torch.float32, device=DEV)
    out, _ = skv.paged_decode_attn(case.q, kp, vp, case.page_table, case.seq_lens,
                                   case.cu_seqlens_q, plan, tok, kv_heads=H, max_q=cfg.max_q,
                                   num_cus=cfg.num_cus, seg_max=cfg.seg_max,
                                   kv_dtype=dtype, layout="shuffled", k_scale=case.k_scale,
                                   v_scale=case.v_scale, out_lse=out_lse, page_size=P)
    torch.cuda.synchronize()
    # oracle: the same tokens written into the standard pages
    std = oracle.write_tokens_standard(std0, kv_new[0], kv_new[1], slots)
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    ref_out, ref_lse = oracle.decode_attention(
        q, std, dtype, table, case.seq_lens.cpu().numpy(), case.cu_seqlens_q.cpu().numpy(),
        H, P, cfg.causal, cfg.k_scale, cfg.v_scale)
    r = compare(out.float().cpu().numpy().astype(np.float64),
                out_lse.cpu().numpy().astype(np.float64), ref_out, ref_lse, dtype)
    say("write+attend", dtype, P, r)
    assert r["max_abs"] <= TOL[dtype], r
    assert r["lse_err"] <= 1e-3, r


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("H,N,D", [(1, 16, D), (2, 16, D), (8, 16, D), (3, 32, D), (2, 16, 64),
                                   (3, 32, 256)])
def test_cache_write_quantises_bit_exact(H, N, D):
    """bf16 rows into an fp8 cache with per-tensor scales: every code equals the
    oracle's nearest-even e4m3fn code of value / scale (fp32 division),
    saturated at 448."""
    say("cache write quantise", H, N, D)
    rng = np.random.default_rng(70 + H + N + D)
    B, T = 7, 50
    ks, vs = 0.0173, 0.0211
    k = rng.normal(0, 1, size=(T, H, D)) * rng.choice([0.01, 1, 5, 50], size=(T, H, 1))
    v = rng.normal(0, 1, size=(T, H, D)) * rng.choice([0.01, 1, 5, 50], size=(T, H, 1))
    k[0, 0, :4] = [1e6, -1e6, 0.0, -0.0]                   # saturation, signed zero
    kb, vb = _bf16_bits(k), _bf16_bits(v)
    slots = rng.choice(B * N, size=T, replace=False).astype(np.int64)
    slots[[2, 9]] = -1
    slots[[4, 30]] = [B * N, 10 ** 12]                     # past the cache: skipped
    kp0 = rng.integers(0, 256, size=(B, H, D // 16, N, 16)).astype(np.uint8)
    vp0 = rng.integers(0, 256, size=(B, H, N // 16, D, 16)).astype(np.uint8)
    kp, vp = _dev(kp0, 1), _dev(vp0, 1)
    key = torch.from_numpy(kb.view(np.int16)).to(DEV).view(torch.bfloat16)
    val = torch.from_numpy(vb.view(np.int16)).to(DEV).view(torch.bfloat16)
    ksc = torch.tensor([ks], dtype=torch.float32, device=DEV)
    vsc = torch.tensor([vs], dtype=torch.float32, device=DEV)
    skv.kv_cache_write(key, val, torch.as_tensor(slots, device=DEV), kp, vp, ksc, vsc)
    torch.cuda.synchronize()
    kq = oracle.quantize_e4m3fn(kb, ks)
    vq = oracle.quantize_e4m3fn(vb, vs)
    wk, wv = oracle.write_tokens_shuffled(kp0, vp0, kq, vq, slots)
    assert np.array_equal(_host(kp, 1), wk)
    assert np.array_equal(_host(vp, 1), wv)


def test_cache_write_quantises_nan_to_nan():
    H, N, B = 1, 16, 2
    k = np.ones((1, H, D), dtype=np.float32)
    k[0, 0, 5] = np.nan
    kb = _bf16_bits(k)
    kp = torch.zeros((B, H, D // 16, N, 16), dtype=torch.uint8, device=DEV)
    vp = torch.zeros((B, H, N // 16, D, 16), dtype=torch.uint8, device=DEV)
    key = torch.from_numpy(kb.view(np.int16)).to(DEV).view(torch.bfloat16)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    skv.kv_cache_write(key, key, torch.tensor([3], dtype=torch.int64, device=DEV), kp, vp,
                       one, one)
    torch.cuda.synchronize()
    got = kp.cpu().numpy()[0, 0, 0, 3]                      # channels 0..15 of row 3
    vals = oracle.decode_e4m3fn(got)
    assert np.isnan(vals[5]) and np.all(vals[np.arange(16) != 5] == 1.0)


def test_fp8_decode_step_quantises_then_attends():
    """A verify step on an fp8 cache: the newest tokens arrive in bf16, are
    quantised by the writer with the cache's scales, and attention reads them.
    Against the oracle quantising the same values into standard pages."""
    say("quantise+attend")
    lens, ql = [40, 300, 17, 1000, 2], [2, 4, 1, 3, 1]
    cfg = gen.small_config(configs.FP8_KV, lens, ql, q_heads=16, kv_heads=2, layout="shuffled",
                           num_cus=64, seg_max=16, seed=23)
    case = gen.make_case(cfg, DEV)
    H = cfg.kv_heads
    table = case.page_table.cpu().numpy()
    slots = np.array([int(table[i, pos // PAGE]) * PAGE + pos % PAGE
                      for i, (L, q) in enumerate(zip(lens, ql)) for pos in range(L - q, L)],
                     dtype=np.int64)
    T = len(slots)
    rng = np.random.default_rng(31)
    kb = _bf16_bits(rng.normal(0, 1, size=(T, H, D)))
    vb = _bf16_bits(rng.normal(0, 1, size=(T, H, D)))
    kp, vp = skv.kv_page_shuffle(case.kv)
    key = torch.from_numpy(kb.view(np.int16)).to(DEV).view(torch.bfloat16)
    val = torch.from_numpy(vb.view(np.int16)).to(DEV).view(torch.bfloat16)
    skv.kv_cache_write(key, val, torch.as_tensor(slots, device=DEV), kp, vp,
                       case.k_scale, case.v_scale)
    plan, tok = skv.plan_build(case.seq_lens, case.cu_seqlens_q, cfg.total_q, H,
                               cfg.num_cus, cfg.seg_max, cfg.causal)
    out_lse = torch.empty((cfg.total_q, cfg.q_heads), dtype=torch.float32, device=DEV)
    out, _ = skv.paged_decode_attn(case.q, kp, vp, case.page_table, case.seq_lens,
                                   case.cu_seqlens_q, plan, tok, kv_heads=H, max_q=cfg.max_q,
                                   num_cus=cfg.num_cus, seg_max=cfg.seg_max, kv_dtype="fp8",
                                   layout="shuffled", k_scale=case.k_scale,
                                   v_scale=case.v_scale, out_lse=out_lse)
    torch.cuda.synchronize()
    std = oracle.write_tokens_standard(gen.raw_kv(case), oracle.quantize_e4m3fn(kb, cfg.k_scale),
                                       oracle.quantize_e4m3fn(vb, cfg.v_scale), slots)
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    ref_out, ref_lse = oracle.decode_attention(
        q, std, "fp8", table, case.seq_lens.cpu().numpy(), case.cu_seqlens_q.cpu().numpy(),
        H, PAGE, cfg.causal, cfg.k_scale, cfg.v_scale)
    r = compare(out.float().cpu().numpy().astype(np.float64),
                out_lse.cpu().numpy().astype(np.float64), ref_out, ref_lse, "fp8")
    say("quantise+attend", r)
    assert r["max_abs"] <= TOL["fp8"], r
    assert r["lse_err"] <= 1e-3, r
