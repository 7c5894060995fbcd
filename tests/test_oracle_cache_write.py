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


@pytest.mark.parametrize("D,e,ch,kidx,vidx", [
    (256, 2, 201, (25, 5, 1), (0, 201, 5)),      # x = 8: 201 = 25*8 + 1
    (64, 1, 50, (3, 5, 2), (0, 50, 5)),          # x = 16: 50 = 3*16 + 2
    (64, 2, 63, (7, 5, 7), (0, 63, 5))])         # x = 8: 63 = 7*8 + 7
def test_hand_derived_slot_other_head_dims(D, e, ch, kidx, vidx):
    """Slot 37 is block 2, row 5 (16-token pages) at head dims 64 and 256 too:
    K channel ch = c1*x + i lands at k_plane[2, h, c1, 5, i] and V channel ch at
    v_plane[2, h, 5 // x, ch, 5 % x]."""
    B, H, x = 4, 2, 16 // e
    kp = np.zeros((B, H, D // x, N, x), np.uint32)
    vp = np.zeros((B, H, N // x, D, x), np.uint32)
    key = np.arange(H * D, dtype=np.uint32).reshape(1, H, D) + 1000
    val = np.arange(H * D, dtype=np.uint32).reshape(1, H, D) + 5000
    kp2, vp2 = oracle.write_tokens_shuffled(kp, vp, key, val, [37])
    assert kp2[(2, 1) + kidx] == 1000 + D + ch
    assert vp2[(2, 1) + vidx] == 5000 + D + ch
    assert np.count_nonzero(kp2) == H * D and np.count_nonzero(vp2) == H * D


@pytest.mark.parametrize("D", [128, 64, 256])
@pytest.mark.parametrize("N", [16, 32])
@pytest.mark.parametrize("H,e", [(1, 2), (2, 2), (3, 2), (8, 2), (1, 1), (4, 1)])
def test_equals_standard_write_then_shuffle(H, e, N, D):
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


@pytest.mark.parametrize("writer", ["standard", "shuffled"])
def test_slots_past_the_cache_are_skipped(writer):
    """Hand case for the reading that a slot at or past num_blocks * N names no
    row of the cache and is skipped like padding. B = 2 blocks of N = 16 rows:
    slot 31 is block 1, row 15 (the last row) and is written; slots 32 (one
    past the end), 47 and 10**9 change nothing, nor does -1."""
    B, H = 2, 1
    std0 = np.full((B, H, N, 2 * D), 7, np.uint16)
    key = np.arange(5 * H * D, dtype=np.uint16).reshape(5, H, D) + 100
    val = key + 1000
    slots = np.array([32, 31, 47, 10**9, -1], np.int64)
    if writer == "standard":
        got = oracle.write_tokens_standard(std0, key, val, slots)
    else:
        kp, vp = oracle.write_tokens_shuffled(*oracle.shuffle_blocks(std0), key, val, slots)
        got = oracle.unshuffle_blocks(kp, vp)
    want = std0.copy()
    want[1, 0, 15, :D] = key[1, 0]                       # token 1 -> block 1, row 15
    want[1, 0, 15, D:] = val[1, 0]
    assert np.array_equal(got, want)
    # exactly one row changed: nothing wrapped to block 0 or clamped to the end
    assert np.count_nonzero(got != 7) == 2 * D
