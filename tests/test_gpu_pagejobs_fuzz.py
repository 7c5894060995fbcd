"""Randomised page jobs, bit-exact against the oracle: each seeded case draws
the element size (bf16/fp16 bits or fp8 bytes), page size, head dim, kv heads
(up to the conversion's 128 KiB block bound), pool size and a listed subset of
blocks in random order, and runs every page job on it: the repack into
shuffled planes, the unshuffle, the in-place conversion of received byte
halves and back, and the cache writer with padding and past-the-end slots.
Unlisted blocks must come through untouched."""
import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_amd as skv
from gpu_harness import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 48
MAX_BLOCK_BYTES = 128 * 1024


def _dev(a, e):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if e == 2 else
                            np.ascontiguousarray(a)).to(DEV)


def _host(t, e):
    a = t.cpu().numpy()
    return a.view(np.uint16) if e == 2 else a


def _codes(rng, shape, e):
    return rng.integers(0, 1 << (8 * e), size=shape).astype(np.uint16 if e == 2 else np.uint8)


def _draw(seed):
    rng = np.random.default_rng(20_000 + seed)
    e = int(rng.choice([1, 2]))
    N = int(rng.choice([16, 32]))
    D = int(rng.choice([64, 128, 256]))
    hmax = MAX_BLOCK_BYTES // (2 * N * D * e)
    H = int(rng.integers(1, min(hmax, 16) + 1))
    B = int(rng.integers(1, 40))
    listed = None
    if rng.random() < 0.6:
        listed = rng.permutation(B)[:int(rng.integers(1, B + 1))].astype(np.int32)
    return rng, e, N, D, H, B, listed


@pytest.mark.parametrize("seed", range(N_CASES), ids=lambda s: f"jobs{s}")
def test_random_page_jobs_match_oracle(seed):
    rng, e, N, D, H, B, listed = _draw(seed)
    say("page jobs", seed, dict(e=e, N=N, D=D, H=H, B=B,
                                listed=None if listed is None else len(listed)))
    x = 16 // e
    ids = None if listed is None else torch.as_tensor(listed, device=DEV)
    in_list = (np.ones(B, bool) if listed is None else np.isin(np.arange(B), listed))
    std = _codes(rng, (B, H, N, 2 * D), e)

    # repack into planes that already hold other data
    k_old = _codes(rng, (B, H, D // x, N, x), e)
    v_old = _codes(rng, (B, H, N // x, D, x), e)
    kp, vp = _dev(k_old, e), _dev(v_old, e)
    skv.kv_page_shuffle(_dev(std, e), kp, vp, block_ids=ids)
    torch.cuda.synchronize()
    wk, wv = oracle.shuffle_blocks(std, elem_bytes=e)
    gk, gv = _host(kp, e), _host(vp, e)
    for b in range(B):
        if in_list[b]:
            assert np.array_equal(gk[b], wk[b]) and np.array_equal(gv[b], wv[b]), b
        else:
            assert np.array_equal(gk[b], k_old[b]) and np.array_equal(gv[b], v_old[b]), b

    # unshuffle the listed blocks back into a pool holding other data
    fill = _codes(rng, std.shape, e)
    out = _dev(fill, e)
    skv.kv_page_unshuffle(_dev(wk, e), _dev(wv, e), out, block_ids=ids)
    torch.cuda.synchronize()
    got = _host(out, e)
    for b in range(B):
        assert np.array_equal(got[b], std[b] if in_list[b] else fill[b]), b

    # the received byte halves, converted in place and back
    kh, vh = oracle.halves_from_standard(std, listed, k_old, v_old, elem_bytes=e)
    kp, vp = _dev(kh, e), _dev(vh, e)
    skv.kv_page_convert(kp, vp, block_ids=ids, direction="to_shuffled")
    torch.cuda.synchronize()
    ck, cv = oracle.convert_halves(kh, vh, listed, elem_bytes=e)
    assert np.array_equal(_host(kp, e), ck) and np.array_equal(_host(vp, e), cv)
    skv.kv_page_convert(kp, vp, block_ids=ids, direction="to_standard")
    torch.cuda.synchronize()
    assert np.array_equal(_host(kp, e), kh) and np.array_equal(_host(vp, e), vh)

    # new tokens written at their slots, padding and past-the-end slots mixed in
    T = int(rng.integers(1, 2 * N + 2))
    slots = rng.choice(B * N, size=min(T, B * N), replace=False).astype(np.int64)
    T = len(slots)
    bad = rng.random(T)
    slots[bad < 0.1] = -1
    slots[(bad >= 0.1) & (bad < 0.2)] = B * N + rng.integers(0, 1000)
    key = _codes(rng, (T, H, D), e)
    val = _codes(rng, (T, H, D), e)
    kp, vp = _dev(k_old, e), _dev(v_old, e)
    skv.kv_cache_write(_dev(key, e), _dev(val, e), torch.as_tensor(slots, device=DEV), kp, vp)
    torch.cuda.synchronize()
    ok, ov = oracle.write_tokens_shuffled(k_old, v_old, key, val, slots)
    assert np.array_equal(_host(kp, e), ok) and np.array_equal(_host(vp, e), ov)
