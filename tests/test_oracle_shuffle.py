"""Pins for the oracle's page shuffle (CPU only)."""
import numpy as np
import pytest

import oracle
from conftest import load_golden


@pytest.mark.parametrize("case", load_golden("shuffle_offsets.json")["cases"],
                         ids=lambda c: f'{c["plane"]}{c["elem_bytes"]}N{c.get("page_size", 16)}')
def test_hand_derived_offsets(case):
    e = case["elem_bytes"]
    N, D = case.get("page_size", 16), 128
    std = np.zeros((1, 1, N, 2 * D), dtype=np.uint32)
    std.reshape(-1)[:] = np.arange(N * 2 * D)           # unique ids
    kp, vp = oracle.shuffle_blocks(std.astype(np.uint32), elem_bytes=e)
    plane = kp if case["plane"] == "K" else vp
    assert plane.reshape(-1)[case["plane_flat"]] == case["std_flat"]
    ch = case["channel"] + (D if case["plane"] == "V" else 0)
    assert case["token"] * 2 * D + ch == case["std_flat"]


@pytest.mark.parametrize("D", [128, 64, 256])
@pytest.mark.parametrize("N", [16, 32])
@pytest.mark.parametrize("H,e", [(1, 2), (2, 2), (3, 2), (8, 2), (1, 1), (3, 1)])
def test_bijection_and_inverse(H, e, N, D):
    B = 3
    std = np.arange(B * H * N * 2 * D, dtype=np.uint32).reshape(B, H, N, 2 * D)
    kp, vp = oracle.shuffle_blocks(std, elem_bytes=e)
    x = 16 // e
    assert kp.shape == (B, H, D // x, N, x) and vp.shape == (B, H, N // x, D, x)
    allv = np.concatenate([kp.reshape(-1), vp.reshape(-1)])
    assert np.array_equal(np.sort(allv), std.reshape(-1))   # every element once
    back = oracle.unshuffle_blocks(kp, vp, elem_bytes=e)
    assert np.array_equal(back, std)
    kp2, vp2 = oracle.shuffle_blocks(oracle.unshuffle_blocks(kp, vp, elem_bytes=e),
                                     elem_bytes=e)
    assert np.array_equal(kp2, kp) and np.array_equal(vp2, vp)


def test_chunk_structure():
    """A 16-byte K chunk of the plane is a 16-byte chunk of one standard token
    row; a 16-byte V chunk holds x consecutive tokens of one channel."""
    N, D, H = 16, 128, 2
    std = np.arange(H * N * 2 * D, dtype=np.uint16).reshape(1, H, N, 2 * D)
    kp, vp = oracle.shuffle_blocks(std)
    x = 8
    for h in range(H):
        for c in range(D // x):
            for n in range(N):
                assert np.array_equal(kp[0, h, c, n], std[0, h, n, c * x:(c + 1) * x])
        for g in range(N // x):
            for d in range(D):
                assert np.array_equal(vp[0, h, g, d], std[0, h, g * x:(g + 1) * x, D + d])


def test_listed_blocks_only():
    std = np.arange(4 * 2 * 16 * 256, dtype=np.uint16).reshape(4, 2, 16, 256)
    kp, vp = oracle.shuffle_blocks(std, block_ids=[2, 0])
    full_k, full_v = oracle.shuffle_blocks(std)
    for b in (0, 2):
        assert np.array_equal(kp[b], full_k[b]) and np.array_equal(vp[b], full_v[b])
    for b in (1, 3):
        assert not kp[b].any() and not vp[b].any()
