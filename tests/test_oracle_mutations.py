"""The oracle's pins have teeth: plant a plausible mistake in the oracle (on the
CPU, via monkeypatch) and check that at least one pin then fails.

Each mutation is applied to the oracle only; the pins are the functions of
tests/test_oracle_*.py, called directly.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.contract as contract
import oracle.fp8 as fp8
import oracle.merge as merge
import oracle.planner as planner
import oracle.shuffle as shuffle
import test_oracle_attention as TA
import test_oracle_cache_write as TW
import test_oracle_contract as TK
import test_oracle_convert as TC
import test_oracle_fp8 as TF
import test_oracle_planner as TP
import test_oracle_shuffle as TS
from conftest import load_golden


def _pins():
    """(name, callable) for every pin, parametrized ones expanded."""
    pins = []
    for mod in (TA, TC, TF, TP, TK, TS, TW):
        for name in dir(mod):
            if not name.startswith("test_"):
                continue
            fn = getattr(mod, name)
            marks = getattr(fn, "pytestmark", [])
            params = [m for m in marks if m.name == "parametrize"]
            if not params:
                pins.append((name, fn))
                continue
            axes = []                      # one list of keyword dicts per parametrize mark
            for m in params:
                argnames, values = m.args[0], m.args[1]
                names = ([a.strip() for a in argnames.split(",")]
                         if isinstance(argnames, str) else list(argnames))
                axes.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in values])
            for combo in itertools.product(*axes):
                kw = {k: v for d in combo for k, v in d.items()}
                pins.append((f"{name}[{kw}]", (lambda f=fn, k=kw: f(**k))))
    return pins


def _failing(pins):
    bad = []
    for name, fn in pins:
        try:
            fn()
        except Exception:
            bad.append(name)
    return bad


def test_unmutated_oracle_passes_every_pin():
    assert _failing(_pins()) == []


def _wrong_scale(qvec, K, V):
    qvec = np.asarray(qvec, dtype=np.float64)
    D = qvec.shape[-1]
    if K.shape[0] == 0:
        return np.zeros(D), -math.inf
    s = (K @ qvec) / D                                   # 1/D instead of 1/sqrt(D)
    m = s.max()
    w = np.exp(s - m)
    return (w @ V) / w.sum(), m + math.log(w.sum())


def _no_normalize(qvec, K, V):
    qvec = np.asarray(qvec, dtype=np.float64)
    D = qvec.shape[-1]
    if K.shape[0] == 0:
        return np.zeros(D), -math.inf
    s = (K @ qvec) / math.sqrt(D)
    m = s.max()
    w = np.exp(s - m)
    return (w @ V), m + math.log(w.sum())               # dropped division by the sum


def _causal_off_by_one(L, q, j, causal):
    if not causal:
        return int(L)
    return int(min(max(L - q + j, 0), L))                # misses the token itself


def _swap_kv(kv, table_row, L, page_size):
    Kr, Vr = TRUE_GATHER(kv, table_row, L, page_size)
    return Vr, Kr


def _head_mod(q, kv, kv_dtype, table, seq_lens, cu, kv_heads, page_size, causal=1,
              k_scale=None, v_scale=None, planes=None, rows=None):
    # q head h reads kv head h % Hkv instead of h // G
    q = np.asarray(q, dtype=np.float64)
    total_q, Hq, D = q.shape
    out = np.full((total_q, Hq, D), np.nan)
    lse = np.full((total_q, Hq), np.nan)
    for i, L in enumerate(seq_lens):
        K, V = att.sequence_kv(kv, kv_dtype, k_scale, v_scale, table[i], int(L), page_size,
                               planes)
        qn = int(cu[i + 1] - cu[i])
        for j in range(qn):
            t = int(cu[i]) + j
            vis = att.visible_keys(int(L), qn, j, causal)
            for h in range(Hq):
                out[t, h], lse[t, h] = att.attend_one(q[t, h], K[:vis, h % kv_heads],
                                                      V[:vis, h % kv_heads])
    return out, lse


def _fp8_bias8(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -7
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)


def _merge_log2(outs, lses, dim=None):
    if len(lses) == 0:
        return np.zeros(0 if dim is None else dim), -math.inf
    lses = np.asarray(lses, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    if np.all(lses == -math.inf):
        return np.zeros(outs.shape[1] if dim is None else dim), -math.inf
    M = lses.max()
    tot = np.exp(lses - M).sum()
    lse = M + math.log2(tot)                             # wrong log base
    w = np.exp(lses - lse)
    return (w[:, None] * outs).sum(axis=0), lse


def _plan_plus_one(seq_lens, cu, kv_heads, page_size, num_cus, seg_max, causal=1):
    plan, tok = TRUE_PLAN(seq_lens, cu, kv_heads, page_size, num_cus, seg_max, causal)
    T = plan[0] + 1                                      # not the smallest feasible T
    return TRUE_PLAN_WITH_T(seq_lens, cu, kv_heads, page_size, num_cus, T, causal,
                            len(plan) - 1)


def _plan_segment_major(seq_lens, cu, kv_heads, page_size, num_cus, seg_max, causal=1):
    plan, tok = TRUE_PLAN(seq_lens, cu, kv_heads, page_size, num_cus, seg_max, causal)
    items = [w for w in plan[1:] if w != -1]
    items.sort(key=lambda w: (w & 0xFFFF, w >> 16))       # segment-major order
    return [plan[0]] + items + [-1] * (len(plan) - 1 - len(items)), tok


def _plan_seq_count(seq_lens, cu, kv_heads, page_size, num_cus, seg_max, causal=1):
    plan, tok = TRUE_PLAN(seq_lens, cu, kv_heads, page_size, num_cus, seg_max, causal)
    T = plan[0]
    tok2 = []
    for i, L in enumerate(seq_lens):                     # sequence's count, not the token's
        n = -(-int(L) // page_size)
        for _ in range(int(cu[i + 1]) - int(cu[i])):
            tok2.append(-(-n // T))
    return plan, tok2


def _shuffle_transposed(std, block_ids=None, elem_bytes=None):
    kp, vp = TRUE_SHUFFLE(std, block_ids, elem_bytes)
    B, H, C, N, x = kp.shape
    kp2 = kp.reshape(B, H, C * N * x).reshape(B, H, N, C, x).transpose(0, 1, 3, 2, 4).copy()
    return kp2.reshape(kp.shape), vp


def _halves_swapped(std, block_ids=None, k_plane=None, v_plane=None, elem_bytes=None):
    kp, vp = TRUE_HALVES(std, block_ids, k_plane, v_plane, elem_bytes)
    std = np.asarray(std)
    B, H, N, D2 = std.shape
    half = H * N * (D2 // 2)
    for b in (range(B) if block_ids is None else block_ids):
        flat = std[b].reshape(-1)                        # second half into the K plane
        kp[b] = flat[half:].reshape(kp.shape[1:])
        vp[b] = flat[:half].reshape(vp.shape[1:])
    return kp, vp


def _fixed_floor(seq_lens, cu, kv_heads, page_size, num_cus=256, seg_max=64, causal=1):
    S, seg_pages, tok = TRUE_FIXED(seq_lens, cu, kv_heads, page_size, num_cus, seg_max, causal)
    pages = [-(-int(L) // page_size) for L in seq_lens]
    return S, [max(n // S, 1) if n else 0 for n in pages], tok     # floor, not ceil


def _write_k_transposed(k_plane, v_plane, key, value, slot_mapping):
    kp, vp = TRUE_WRITE(k_plane, v_plane, key, value, slot_mapping)
    B, H, Dx, N, x = kp.shape
    c = np.arange(Dx * x)
    for t, slot in enumerate(slot_mapping):
        if slot < 0:
            continue
        b, n = divmod(int(slot), N)
        for h in range(H):
            kp[b, h, c % Dx, n, c // Dx] = key[t, h]          # channel split the wrong way
    return kp, vp


def _write_wraps(k_plane, v_plane, key, value, slot_mapping):
    B, N = k_plane.shape[0], k_plane.shape[3]
    wrapped = [s % (B * N) if s >= 0 else s for s in np.asarray(slot_mapping, np.int64)]
    return TRUE_WRITE(k_plane, v_plane, key, value, wrapped)


def _write_std_wraps(std, key, value, slot_mapping):
    B, N = std.shape[0], std.shape[2]
    wrapped = [s % (B * N) if s >= 0 else s for s in np.asarray(slot_mapping, np.int64)]
    return TRUE_WRITE_STD(std, key, value, wrapped)


TRUE_CHECK = contract.check_inputs


def _check_reads_one_more(page_table, seq_lens, cu_seqlens_q, total_q, max_q, page_size,
                          num_blocks):
    # reads floor(L / P) + 1 entries instead of ceil(L / P): one too many when
    # L is a whole number of pages
    table = np.asarray(page_table)
    lens = [int(v) for v in seq_lens]
    mask, first = TRUE_CHECK(table, lens, cu_seqlens_q, total_q, max_q, page_size, num_blocks)
    for i, L in enumerate(lens):
        if L > 0 and L % page_size == 0 and L // page_size < table.shape[1]:
            if not (0 <= int(table[i][L // page_size]) < num_blocks):
                mask |= contract.BAD_PAGE_ID
                first = i if first < 0 else min(first, i)
    return mask, first


def _encode_ties_up(values):
    v = np.asarray(values, dtype=np.float64)
    pos = fp8._E4M3FN[:0x7F]
    out = np.empty(v.shape, dtype=np.uint8)
    for idx, x in np.ndenumerate(v):
        sign = 0x80 if math.copysign(1.0, x) < 0 else 0
        a = min(abs(x), 448.0)
        hi = int(np.searchsorted(pos, a))
        lo = max(hi - 1, 0)
        code = hi if pos[hi] - a <= a - pos[lo] else lo       # ties away from zero
        out[idx] = sign | code
    return out


TRUE_WRITE = shuffle.write_tokens_shuffled
TRUE_WRITE_STD = shuffle.write_tokens_standard
TRUE_FIXED = planner.fixed_split_plan
TRUE_HALVES = shuffle.halves_from_standard
TRUE_GATHER = att.gather_standard
TRUE_PLAN = planner.plan_segments
TRUE_SHUFFLE = shuffle.shuffle_blocks


def TRUE_PLAN_WITH_T(seq_lens, cu, kv_heads, page_size, num_cus, T, causal, width):
    items = []
    for i, L in enumerate(seq_lens):
        n = -(-int(L) // page_size)
        items += [(i << 16) | s for s in range(-(-n // T))]
    tok = []
    for i, L in enumerate(seq_lens):
        qn = int(cu[i + 1]) - int(cu[i])
        for j in range(qn):
            vis = att.visible_keys(int(L), qn, j, causal)
            tok.append(-(-vis // (T * page_size)))
    return [T] + items + [-1] * (width - len(items)), tok


MUTATIONS = [
    ("score scale 1/D", [(att, "attend_one", _wrong_scale), (merge, "attend_one", _wrong_scale)]),
    ("softmax not normalized", [(att, "attend_one", _no_normalize),
                                (merge, "attend_one", _no_normalize)]),
    ("causal off by one", [(att, "visible_keys", _causal_off_by_one),
                           (planner, "visible_keys", _causal_off_by_one),
                           (merge, "visible_keys", _causal_off_by_one)]),
    ("K and V swapped", [(att, "gather_standard", _swap_kv)]),
    ("head mapping h % Hkv", [(att, "decode_attention", _head_mod),
                              (oracle, "decode_attention", _head_mod)]),
    ("e4m3 bias 8", [(fp8, "e4m3fn_value", _fp8_bias8),
                     (fp8, "_E4M3FN", np.array([_fp8_bias8(c) for c in range(256)])),
                     (oracle, "e4m3fn_value", _fp8_bias8)]),
    ("lse in log2", [(merge, "lse_merge", _merge_log2), (oracle, "lse_merge", _merge_log2)]),
    ("T not smallest", [(planner, "plan_segments", _plan_plus_one),
                        (oracle, "plan_segments", _plan_plus_one)]),
    ("segment-major work list", [(planner, "plan_segments", _plan_segment_major),
                                 (oracle, "plan_segments", _plan_segment_major)]),
    ("per-sequence instead of per-token counts", [(planner, "plan_segments", _plan_seq_count),
                                                  (oracle, "plan_segments", _plan_seq_count)]),
    ("K plane transposed", [(shuffle, "shuffle_blocks", _shuffle_transposed),
                            (oracle, "shuffle_blocks", _shuffle_transposed)]),
    ("fixed split floors the segment length", [(planner, "fixed_split_plan", _fixed_floor),
                                               (oracle, "fixed_split_plan", _fixed_floor)]),
    ("e4m3 encode ties away from zero", [(fp8, "encode_e4m3fn", _encode_ties_up),
                                         (oracle, "encode_e4m3fn", _encode_ties_up)]),
    ("cache writer K channel split transposed",
     [(shuffle, "write_tokens_shuffled", _write_k_transposed),
      (oracle, "write_tokens_shuffled", _write_k_transposed)]),
    ("cache writer wraps slots past the cache",
     [(shuffle, "write_tokens_shuffled", _write_wraps),
      (oracle, "write_tokens_shuffled", _write_wraps),
      (shuffle, "write_tokens_standard", _write_std_wraps),
      (oracle, "write_tokens_standard", _write_std_wraps)]),
    ("byte halves swapped", [(shuffle, "halves_from_standard", _halves_swapped),
                             (oracle, "halves_from_standard", _halves_swapped)]),
    ("contract checker reads one page-table entry too many",
     [(contract, "check_inputs", _check_reads_one_more),
      (oracle, "check_inputs", _check_reads_one_more)]),
]


@pytest.mark.parametrize("name,patches", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, patches, monkeypatch):
    for mod, attr, value in patches:
        monkeypatch.setattr(mod, attr, value)
    bad = _failing(_pins())
    assert bad, f"no pin caught the planted mistake: {name}"
