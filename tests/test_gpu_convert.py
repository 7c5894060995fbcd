"""GPU parity (through the C ABI) of the in-place conversion of received byte
halves, its inverse and the out-of-place unshuffle: bit-exact against the CPU
oracle."""
import numpy as np
import pytest
import torch

import oracle
import split_kv_paged_amd as skv
from gpu_harness import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skv.load()
    yield
    torch.cuda.synchronize()


def _np_dtype(e):
    return np.uint16 if e == 2 else np.uint8


def _torch_dtype(e):
    return torch.int16 if e == 2 else torch.uint8


def _to_dev(a, e):
    return torch.from_numpy(a.view(np.int16) if e == 2 else a).to(DEV)


def _to_host(t, e):
    a = t.cpu().numpy()
    return a.view(np.uint16) if e == 2 else a


def _random_codes(rng, shape, e):
    return rng.integers(0, 1 << (8 * e), size=shape).astype(_np_dtype(e))


CONVERT_CASES = [(2, 1, 16), (2, 2, 16), (2, 3, 16), (2, 8, 16), (2, 16, 16), (1, 1, 16),
                 (1, 3, 16), (1, 8, 16), (1, 32, 16),
                 (2, 1, 32), (2, 3, 32), (2, 8, 32), (1, 5, 32), (1, 16, 32)]


@pytest.mark.parametrize("subset", [False, True])
@pytest.mark.parametrize("e,H,N", CONVERT_CASES)
def test_convert_in_place_and_back(e, H, N, subset):
    say("convert", e, H, N, subset)
    rng = np.random.default_rng(100 * H + e)
    B = 23
    x = 16 // e
    std = _random_codes(rng, (B, H, N, 2 * D), e)
    k_old = _random_codes(rng, (B, H, D // x, N, x), e)
    v_old = _random_codes(rng, (B, H, N // x, D, x), e)
    listed = None
    if subset:
        listed = rng.choice(B, size=9, replace=False).astype(np.int32)
    kp0, vp0 = oracle.halves_from_standard(std, listed, k_old, v_old, elem_bytes=e)
    kp, vp = _to_dev(kp0, e), _to_dev(vp0, e)
    ids = None if listed is None else torch.as_tensor(listed, device=DEV)

    skv.kv_page_convert(kp, vp, block_ids=ids, direction="to_shuffled")
    torch.cuda.synchronize()
    wk, wv = oracle.convert_halves(kp0, vp0, listed)
    assert np.array_equal(_to_host(kp, e), wk)
    assert np.array_equal(_to_host(vp, e), wv)

    skv.kv_page_convert(kp, vp, block_ids=ids, direction="to_standard")
    torch.cuda.synchronize()
    assert np.array_equal(_to_host(kp, e), kp0)
    assert np.array_equal(_to_host(vp, e), vp0)


@pytest.mark.parametrize("subset", [False, True])
@pytest.mark.parametrize("e,H,N", [(2, 1, 16), (2, 3, 16), (2, 8, 16), (1, 2, 16), (1, 5, 16),
                                   (2, 3, 32), (1, 2, 32)])
def test_unshuffle_bit_exact(e, H, N, subset):
    say("unshuffle", e, H, N, subset)
    rng = np.random.default_rng(7 * H + e)
    B = 19
    std = _random_codes(rng, (B, H, N, 2 * D), e)
    kp0, vp0 = oracle.shuffle_blocks(std, elem_bytes=e)
    listed = None if not subset else rng.choice(B, size=6, replace=False).astype(np.int32)
    ids = None if listed is None else torch.as_tensor(listed, device=DEV)
    fill = _random_codes(rng, std.shape, e)
    out = _to_dev(fill, e)
    skv.kv_page_unshuffle(_to_dev(kp0, e), _to_dev(vp0, e), out, block_ids=ids)
    torch.cuda.synchronize()
    got = _to_host(out, e)
    want = oracle.unshuffle_blocks(kp0, vp0, elem_bytes=e)
    for b in range(B):
        if listed is None or b in listed:
            assert np.array_equal(got[b], want[b]), b
            assert np.array_equal(got[b], std[b]), b
        else:
            assert np.array_equal(got[b], fill[b]), f"unlisted block {b} written"


@pytest.mark.parametrize("N", [16, 32])
def test_convert_agrees_with_out_of_place_shuffle(N):
    """Same standard blocks, two routes on the GPU: the out-of-place repack and
    the in-place conversion of the byte halves write identical planes."""
    say("convert vs shuffle", N)
    rng = np.random.default_rng(5)
    B, H, e = 64, 8, 2
    std = _random_codes(rng, (B, H, N, 2 * D), e)
    kp0, vp0 = oracle.halves_from_standard(std, elem_bytes=e)
    kp, vp = _to_dev(kp0, e), _to_dev(vp0, e)
    skv.kv_page_convert(kp, vp)
    ks, vs = skv.kv_page_shuffle(_to_dev(std, e))
    torch.cuda.synchronize()
    assert torch.equal(kp, ks) and torch.equal(vp, vs)
