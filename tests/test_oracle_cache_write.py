"""Pins for the oracle's cache writer (new tokens at their slots; CPU only)."""
import numpy as np
import pytest

import oracle

N, D = 16, 128


def test_hand_derived_slot():
    """Slot 37 is block 2, row 5. bf16 (x = 8): K channel 19 lands at
    k_plane[2, h, 2, 5, 3]; V channel 19 at v_plane[2, h, 0, 19, 5]."""
    B, H = 4, 2
    kp = np.zeros((B, H, D // 8, N, 8), np.uint32)
    vp = np.zeros((B, H, N // 8, D, 8), np.uint32)
    key = np.arange(H * D, dtype=np.uint32).reshape(1, H, D) + 1000
    val = np.arange(H * D, dtype=np.uint32).reshape(1, H, D) + 5000
    kp2, vp2 = oracle.write_tokens_shuffled(kp, vp, key, val, [37])
    assert kp2[2, 1, 2, 5, 3] == 1000 + 128 + 19
    assert vp2[2, 1, 0, 19, 5] == 5000 + 128 + 19
    assert np.count_nonzero(kp2) == H * D and np.count_nonzero(vp2) == H * D


@pytest.mark.parametrize("N", [16, 32])
@pytest.mark.parametrize("H,e", [(1, 2), (2, 2), (3, 2), (8, 2), (1, 1), (4, 1)])
def test_equals_standard_write_then_shuffle(H, e, N):
    """Writing into shuffled planes equals writing into standard pages and then
    shuffling, on a cache that already holds data (untouched rows keep it);
    padding slots (-1) change nothing."""
    rng = np.random.default_rng(H * 3 + e)
    B = 6
    dt = np.uint16 if e == 2 else np.uint8
    std0 = rng.integers(0, 1 << (8 * e), size=(B, H, N, 2 * D)).astype(dt)
    T = 40
    slots = rng.choice(B * N, size=T, replace=False).astype(np.int64)
    slots[[3, 17, 29]] = -1
    key = rng.integers(0, 1 << (8 * e), size=(T, H, D)).astype(dt)
    val = rng.integers(0, 1 << (8 * e), size=(T, H, D)).astype(dt)
    kp0, vp0 = oracle.shuffle_blocks(std0)
    kp1, vp1 = oracle.write_tokens_shuffled(kp0, vp0, key, val, slots)
    std1 = oracle.write_tokens_standard(std0, key, val, slots)
    ks, vs = oracle.shuffle_blocks(std1)
    assert np.array_equal(kp1, ks) and np.array_equal(vp1, vs)
    # the standard write is the definition itself: rows at live slots, nothing else
    live = {int(s): t for t, s in enumerate(slots) if s >= 0}
    for b in range(B):
        for n in range(N):
            t = live.get(b * N + n)
            want = std0[b, :, n] if t is None else np.concatenate([key[t], val[t]], axis=-1)
            assert np.array_equal(std1[b, :, n], want)
