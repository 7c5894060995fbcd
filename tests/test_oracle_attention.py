"""Pins for the oracle's gather, attention and LSE merge (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import configs, gen


def _case(seq_lens, q_lens, q_heads=8, kv_heads=2, kv_dtype="bf16", seed=7, **kw):
    base = configs.FP8_KV if kv_dtype == "fp8" else configs.TINY
    cfg = gen.small_config(base, seq_lens, q_lens, q_heads=q_heads, kv_heads=kv_heads,
                           seed=seed, kv_dtype=kv_dtype, **kw)
    return cfg, gen.make_case(cfg, "cpu")


def _oracle(cfg, case, planes=None, rows=None, causal=None):
    q = oracle.decode_q(gen.raw_u16(case.q), cfg.kv_dtype)
    kv = None if planes is not None else gen.raw_kv(case)
    return oracle.decode_attention(
        q, kv, cfg.kv_dtype, case.page_table.numpy(), case.seq_lens.numpy(),
        case.cu_seqlens_q.numpy(), cfg.kv_heads, cfg.page_size,
        cfg.causal if causal is None else causal, cfg.k_scale, cfg.v_scale,
        planes=planes, rows=rows)


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(128)
    K = rng.standard_normal((1, 128))
    V = rng.standard_normal((1, 128))
    o, lse = oracle.attend_one(q, K, V)
    assert np.array_equal(o, V[0])
    assert lse == pytest.approx(float(K[0] @ q) / math.sqrt(128), rel=1e-15)


def test_equal_keys_give_mean_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(128)
    K = np.tile(rng.standard_normal(128), (37, 1))
    V = rng.standard_normal((37, 128))
    o, lse = oracle.attend_one(q, K, V)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=0, atol=1e-14)
    assert lse == pytest.approx(float(K[0] @ q) / math.sqrt(128) + math.log(37), rel=1e-14)


def test_zero_query_gives_mean_and_log_count():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((20, 128))
    V = rng.standard_normal((20, 128))
    o, lse = oracle.attend_one(np.zeros(128), K, V)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14)
    assert lse == pytest.approx(math.log(20), rel=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128)
    K = rng.standard_normal((50, 128)) * 0.01
    K[17] = q * 10.0                        # score ~ 10*|q|^2/sqrt(D) >> others
    V = rng.standard_normal((50, 128))
    o, _ = oracle.attend_one(q, K, V)
    np.testing.assert_allclose(o, V[17], atol=1e-9)


def test_no_visible_key_is_zero_and_neg_inf():
    o, lse = oracle.attend_one(np.ones(128), np.zeros((0, 128)), np.zeros((0, 128)))
    assert np.array_equal(o, np.zeros(128)) and lse == -math.inf


def test_scale_and_sign_against_exp_loops():
    """Brute force with math.exp on a tiny row (no numpy reductions)."""
    rng = np.random.default_rng(5)
    D = 128
    q = rng.standard_normal(D)
    K = rng.standard_normal((9, D))
    V = rng.standard_normal((9, D))
    s = [sum(q[d] * K[n][d] for d in range(D)) / math.sqrt(D) for n in range(9)]
    m = max(s)
    w = [math.exp(v - m) for v in s]
    tot = sum(w)
    want = [sum(w[n] * V[n][d] for n in range(9)) / tot for d in range(D)]
    o, lse = oracle.attend_one(q, K, V)
    np.testing.assert_allclose(o, want, atol=1e-13)
    assert lse == pytest.approx(m + math.log(tot), rel=1e-14)


@pytest.mark.parametrize("head_dim", [128, 64, 256])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "fp16"])
def test_batch_matches_torch_sdpa_fp64(kv_dtype, head_dim):
    """Independent library routine: torch SDPA in float64 on gathered tensors,
    with the bottom-right causal mask and grouped heads expanded by hand (its
    default scale 1/sqrt(D) pins the oracle's at every head dim)."""
    lens, ql = [37, 100, 16, 1, 5], [1, 4, 3, 2, 4]
    cfg, case = _case(lens, ql, q_heads=8, kv_heads=2, kv_dtype=kv_dtype, head_dim=head_dim)
    out, lse = _oracle(cfg, case)
    q = torch.from_numpy(gen.raw_u16(case.q).view(np.int16)).view(
        torch.float16 if kv_dtype == "fp16" else torch.bfloat16).double().numpy()
    kv = gen.raw_kv(case)
    G = cfg.q_heads // cfg.kv_heads
    cu = case.cu_seqlens_q.numpy()
    for i, L in enumerate(lens):
        Kr, Vr = oracle.gather_standard(kv, case.page_table.numpy()[i], L, 16)
        K = oracle.decode_kv(Kr, kv_dtype, cfg.k_scale)
        V = oracle.decode_kv(Vr, kv_dtype, cfg.v_scale)
        qi = q[cu[i]:cu[i + 1]]                                  # [qn, Hq, D]
        qn = qi.shape[0]
        mask = np.zeros((qn, L), dtype=bool)
        for j in range(qn):
            mask[j, : max(0, L - qn + j + 1)] = True
        Kt = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2)  # [Hq, L, D]
        Vt = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2)
        Qt = torch.from_numpy(qi).permute(1, 0, 2)                        # [Hq, qn, D]
        ok = mask.any(axis=1)
        if not ok.any():
            continue
        ref = torch.nn.functional.scaled_dot_product_attention(
            Qt[:, ok], Kt, Vt, attn_mask=torch.from_numpy(mask[ok]))
        np.testing.assert_allclose(out[cu[i]:cu[i + 1]][ok],
                                   ref.permute(1, 0, 2).numpy(), atol=1e-12)
        for j in np.nonzero(~ok)[0]:
            assert np.all(out[cu[i] + j] == 0) and np.all(lse[cu[i] + j] == -np.inf)


def test_page_relabelling_invariance():
    cfg, case = _case([70, 33], [2, 1])
    out, lse = _oracle(cfg, case)
    kv = gen.raw_kv(case)
    perm = np.random.default_rng(9).permutation(kv.shape[0])
    kv2 = np.empty_like(kv)
    kv2[perm] = kv                                      # block b moves to perm[b]
    table2 = perm[case.page_table.numpy()]
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    out2, lse2 = oracle.decode_attention(q, kv2, "bf16", table2, case.seq_lens.numpy(),
                                         case.cu_seqlens_q.numpy(), 2, 16, 1)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_standard_and_shuffled_layouts_agree(kv_dtype):
    cfg, case = _case([70, 33, 1], [2, 1, 3], kv_dtype=kv_dtype)
    out, lse = _oracle(cfg, case)
    planes = oracle.shuffle_blocks(gen.raw_kv(case))
    out2, lse2 = _oracle(cfg, case, planes=planes)
    # same gathered values; only BLAS summation order may differ with memory layout
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-15)


def test_causal_token_equals_truncated_single_query():
    cfg, case = _case([53], [4], q_heads=4, kv_heads=1)
    out, _ = _oracle(cfg, case)
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    kv = gen.raw_kv(case)
    for j in range(4):
        Lj = 53 - 4 + j + 1
        o1, _ = oracle.decode_attention(q[j:j + 1], kv, "bf16", case.page_table.numpy(),
                                        [Lj], [0, 1], 1, 16, 1)
        assert np.array_equal(o1[0], out[j])


def test_equal_queries_in_a_group_give_equal_rows():
    cfg, case = _case([45], [1], q_heads=8, kv_heads=2)
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    q[0, 1] = q[0, 0]
    q[0, 5] = q[0, 0]
    out, _ = oracle.decode_attention(q, gen.raw_kv(case), "bf16", case.page_table.numpy(),
                                     [45], [0, 1], 2, 16, 1)
    assert np.array_equal(out[0, 1], out[0, 0])
    assert not np.array_equal(out[0, 5], out[0, 0])     # other kv head, other keys


def test_sampled_rows_equal_full_rows():
    cfg, case = _case([70, 33], [2, 3])
    out, lse = _oracle(cfg, case)
    rows = [(0, 3), (4, 7), (2, 0)]
    o2, l2 = _oracle(cfg, case, rows=rows)
    for t, h in rows:
        assert np.array_equal(o2[t, h], out[t, h]) and l2[t, h] == lse[t, h]


@pytest.mark.parametrize("poison", ["finite", "nan"])
def test_poison_never_reaches_the_result(poison):
    cfg = gen.small_config(configs.TINY, [37, 100, 5], [1, 2, 4], seed=3)
    a = gen.make_case(cfg, "cpu", poison="none")
    b = gen.make_case(cfg, "cpu", poison=poison)
    oa, la = _oracle(cfg, a)
    ob, lb = _oracle(cfg, b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    assert not np.array_equal(gen.raw_kv(a), gen.raw_kv(b))


# ---- log-sum-exp merge -------------------------------------------------------

def test_merge_single_partial_is_identity():
    o = np.arange(128.0)
    out, lse = oracle.lse_merge([o], [1.25])
    assert np.array_equal(out, o) and lse == 1.25


def test_merge_order_independent_and_empty():
    rng = np.random.default_rng(6)
    outs = rng.standard_normal((5, 128))
    lses = rng.standard_normal(5) * 3
    a = oracle.lse_merge(outs, lses)
    p = rng.permutation(5)
    b = oracle.lse_merge(outs[p], lses[p])
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    assert a[1] == pytest.approx(b[1], rel=1e-14)
    o, l = oracle.lse_merge(np.zeros((0, 128)), [])
    assert l == -math.inf


def test_merge_keyless_partials_drop_out():
    """A partial with lse -inf (no key) changes nothing: merging it in equals
    merging the others alone, bit for bit; only such partials merge like none."""
    rng = np.random.default_rng(9)
    outs = rng.standard_normal((4, 64))
    lses = rng.standard_normal(4) * 2
    base = oracle.lse_merge(outs, lses)
    with_empty = oracle.lse_merge(np.vstack([outs[:2], np.zeros((1, 64)), outs[2:]]),
                                  np.concatenate([lses[:2], [-math.inf], lses[2:]]))
    assert np.array_equal(base[0], with_empty[0]) and base[1] == with_empty[1]
    o, l = oracle.lse_merge(np.zeros((3, 64)), [-math.inf] * 3)
    assert l == -math.inf and np.array_equal(o, np.zeros(64))


@pytest.mark.parametrize("pages_per_seg", [1, 2, 3, 7])
def test_split_equals_unsplit(pages_per_seg):
    cfg, case = _case([37, 100, 16, 1, 0, 65], [1, 4, 3, 2, 1, 4])
    out, lse = _oracle(cfg, case)
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    so, sl, nseg = oracle.split_decode_attention(
        q, gen.raw_kv(case), "bf16", case.page_table.numpy(), case.seq_lens.numpy(),
        case.cu_seqlens_q.numpy(), 2, 16, pages_per_seg, 1)
    np.testing.assert_allclose(so, out, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(sl[fin], lse[fin], rtol=1e-12)
    assert np.all(sl[~fin] == -np.inf)


def test_planned_split_equals_unsplit_and_counts_match_planner():
    cfg, case = _case([37, 100, 16, 1, 0, 65], [1, 4, 3, 2, 1, 4], num_cus=12)
    plan, tok = oracle.plan_segments(cfg.seq_lens, case.cu_seqlens_q.numpy(),
                                     cfg.kv_heads, 16, cfg.num_cus, cfg.seg_max, 1)
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    so, _, nseg = oracle.split_decode_attention(
        q, gen.raw_kv(case), "bf16", case.page_table.numpy(), case.seq_lens.numpy(),
        case.cu_seqlens_q.numpy(), 2, 16, plan[0], 1)
    assert list(nseg) == tok
    out, _ = _oracle(cfg, case)
    np.testing.assert_allclose(so, out, rtol=1e-12, atol=1e-13)


def test_fixed_split_equals_unsplit_and_counts_match():
    """The fixed split (per-sequence segment lengths) merges to the unsplit
    result, and the per-token counts are the number of non-empty segments."""
    cfg, case = _case([37, 100, 16, 1, 0, 65], [1, 4, 3, 2, 1, 4], num_cus=64)
    S, seg_pages, tok = oracle.fixed_split_plan(cfg.seq_lens, case.cu_seqlens_q.numpy(),
                                                cfg.kv_heads, 16, cfg.num_cus, cfg.seg_max, 1)
    assert S == 4 and seg_pages == [1, 2, 1, 1, 0, 2]
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    so, _, nseg = oracle.split_decode_attention(
        q, gen.raw_kv(case), "bf16", case.page_table.numpy(), case.seq_lens.numpy(),
        case.cu_seqlens_q.numpy(), 2, 16, seg_pages, 1)
    assert list(nseg) == tok
    out, _ = _oracle(cfg, case)
    np.testing.assert_allclose(so, out, rtol=1e-12, atol=1e-13)


def _as_32_token_pages(case16, cfg16):
    """The same tokens re-stored in 32-token pages: page j of sequence i holds
    its tokens 32j .. 32j + 31, taken from the 16-token pages 2j and 2j + 1;
    blocks are numbered in order, the slots past a sequence's end hold zeros."""
    raw = gen.raw_kv(case16)
    table16 = case16.page_table.numpy()
    lens = case16.seq_lens.numpy()
    H, D2 = raw.shape[1], raw.shape[3]
    n32 = [-(-int(L) // 32) for L in lens]
    pool = sum(n32) + 1
    kv32 = np.zeros((pool, H, 32, D2), dtype=raw.dtype)
    table32 = np.full((len(lens), max(max(n32), 1)), pool - 1, dtype=np.int32)
    b = 0
    for i, L in enumerate(lens):
        for j in range(n32[i]):
            for half in range(2):
                p16 = 2 * j + half
                if 16 * p16 < L:
                    kv32[b, :, 16 * half:16 * half + 16] = raw[table16[i, p16]]
            table32[i, j] = b
            b += 1
    return kv32, table32


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_32_token_pages_equal_16_token_pages(kv_dtype):
    """Attention over a 32-token-page cache, standard and shuffled, equals
    attention over the same tokens in 16-token pages: the gathered K and V rows
    are the same values (the standard gather bit for bit)."""
    cfg, case = _case([0, 1, 15, 16, 17, 31, 32, 33, 100, 257], [1, 2, 1, 3, 4, 1, 2, 4, 3, 2],
                      kv_dtype=kv_dtype, seed=21)
    want_o, want_l = _oracle(cfg, case)
    kv32, table32 = _as_32_token_pages(case, cfg)
    q = oracle.decode_bf16(gen.raw_u16(case.q))
    args = (case.seq_lens.numpy(), case.cu_seqlens_q.numpy(), cfg.kv_heads, 32, cfg.causal,
            cfg.k_scale, cfg.v_scale)
    o, l = oracle.decode_attention(q, kv32, cfg.kv_dtype, table32, *args)
    assert np.array_equal(o, want_o) and np.array_equal(l, want_l)
    planes = oracle.shuffle_blocks(kv32)
    assert planes[0].shape[-2:] == (32, 16 // (2 if kv_dtype == "bf16" else 1))
    o2, l2 = oracle.decode_attention(q, None, cfg.kv_dtype, table32, *args, planes=planes)
    # same gathered values; only BLAS summation order may differ with memory layout
    np.testing.assert_allclose(o2, want_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, want_l, rtol=1e-15)
