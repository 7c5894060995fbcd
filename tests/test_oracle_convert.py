"""Pins for the oracle's in-place conversion of received byte halves (CPU)."""
import numpy as np
import pytest

import oracle
from conftest import load_golden

N, D = 16, 128


def _ids(B, H, D=D):
    return np.arange(B * H * N * 2 * D, dtype=np.uint32).reshape(B, H, N, 2 * D)


@pytest.mark.parametrize("case", load_golden("byte_halves_offsets.json")["cases"],
                         ids=lambda c: f'H{c["heads"]}e{c["elem_bytes"]}D{c.get("head_dim", D)}'
                                       f'{c["after"]}{c["after_flat"]}')
def test_hand_derived_offsets(case):
    H, e = case["heads"], case["elem_bytes"]
    std = _ids(1, H, case.get("head_dim", D))
    assert std.reshape(-1)[case["std_flat"]] == case["std_flat"]
    kp0, vp0 = oracle.halves_from_standard(std, elem_bytes=e)
    before = kp0 if case["before"] == "K" else vp0
    assert before[0].reshape(-1)[case["before_flat"]] == case["std_flat"]
    kp1, vp1 = oracle.convert_halves(kp0, vp0)
    after = kp1 if case["after"] == "K" else vp1
    assert after[0].reshape(-1)[case["after_flat"]] == case["std_flat"]


@pytest.mark.parametrize("H", [1, 2, 3, 5])
def test_halves_are_the_byte_halves(H):
    """The element-level split equals the split of the block's raw bytes
    (little-endian element codes)."""
    rng = np.random.default_rng(H)
    std = rng.integers(0, 1 << 16, size=(2, H, N, 2 * D), dtype=np.uint16)
    kp, vp = oracle.halves_from_standard(std)
    for b in range(2):
        raw = std[b].tobytes()
        assert kp[b].tobytes() == raw[:len(raw) // 2]
        assert vp[b].tobytes() == raw[len(raw) // 2:]


@pytest.mark.parametrize("D", [128, 64, 256])
@pytest.mark.parametrize("N", [16, 32])
@pytest.mark.parametrize("H,e", [(1, 2), (2, 2), (3, 2), (8, 2), (1, 1), (3, 1), (4, 1)])
def test_matches_out_of_place_shuffle_and_round_trips(H, e, N, D):
    B = 5
    std = np.arange(B * H * N * 2 * D, dtype=np.uint32).reshape(B, H, N, 2 * D)
    listed = [3, 0, 4]
    rng = np.random.default_rng(7)
    x = 16 // e
    k_old = rng.integers(0, 1 << 30, size=(B, H, D // x, N, x)).astype(np.uint32)
    v_old = rng.integers(0, 1 << 30, size=(B, H, N // x, D, x)).astype(np.uint32)
    kp0, vp0 = oracle.halves_from_standard(std, listed, k_old, v_old, elem_bytes=e)
    kp1, vp1 = oracle.convert_halves(kp0, vp0, listed)
    ks, vs = oracle.shuffle_blocks(std, elem_bytes=e)
    for b in range(B):
        if b in listed:
            assert np.array_equal(kp1[b], ks[b]) and np.array_equal(vp1[b], vs[b])
            both = np.sort(np.concatenate([kp1[b].ravel(), vp1[b].ravel()]))
            assert np.array_equal(both, std[b].ravel())        # a permutation
        else:
            assert np.array_equal(kp1[b], k_old[b]) and np.array_equal(vp1[b], v_old[b])
    kp2, vp2 = oracle.revert_to_halves(kp1, vp1, listed)
    assert np.array_equal(kp2, kp0) and np.array_equal(vp2, vp0)


def test_single_head_planes_hold_token_halves():
    """With one head, the K plane receives token rows 0..7 and the V plane rows
    8..15, each row with both its K and V channels."""
    std = _ids(1, 1)
    kp, vp = oracle.halves_from_standard(std, elem_bytes=2)
    assert np.array_equal(kp[0].reshape(8, 2 * D), std[0, 0, :8])
    assert np.array_equal(vp[0].reshape(8, 2 * D), std[0, 0, 8:])
