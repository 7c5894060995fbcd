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


CONVERT_CASES = [(2, 1, 16, D), (2, 2, 16, D), (2, 3, 16, D), (2, 8, 16, D), (2, 16, 16, D),
                 (1, 1, 16, D), (1, 3, 16, D), (1, 8, 16, D), (1, 32, 16, D),
                 (2, 1, 32, D), (2, 3, 32, D), (2, 8, 32, D), (1, 5, 32, D), (1, 16, 32, D),
                 # head dims 64 and 256, up to the 128 KiB block bound
                 (2, 1, 16, 64), (2, 3, 16, 64), (2, 32, 16, 64), (1, 64, 16, 64),
                 (1, 3, 32, 64), (2, 5, 32, 64),
                 (2, 1, 16, 256), (2, 3, 16, 256), (2, 8, 16, 256), (1, 1, 16, 256),
                 (1, 5, 32, 256), (2, 4, 32, 256)]


@pytest.mark.parametrize("subset", [False, True])
@pytest.mark.parametrize("e,H,N,D", CONVERT_CASES)
def test_convert_in_place_and_back(e, H, N, D, subset):
    say("convert", e, H, N, D, subset)
    rng = np.random.default_rng(100 * H + e + D)
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
@pytest.mark.parametrize("e,H,N,D", [(2, 1, 16, D), (2, 3, 16, D), (2, 8, 16, D), (1, 2, 16, D),
                                     (1, 5, 16, D), (2, 3, 32, D), (1, 2, 32, D),
                                     (2, 3, 16, 64), (1, 5, 32, 64), (2, 2, 32, 256),
                                     (1, 3, 16, 256)])
def test_unshuffle_bit_exact(e, H, N, D, subset):
    say("unshuffle", e, H, N, D, subset)
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


@pytest.mark.parametrize("N,D", [(16, D), (32, D), (16, 64), (16, 256)])
def test_convert_agrees_with_out_of_place_shuffle(N, D):
    """Same standard blocks, two routes on the GPU: the out-of-place repack and
    the in-place conversion of the byte halves write identical planes."""
    say("convert vs shuffle", N, D)
    rng = np.random.default_rng(5)
    B, H, e = 64, (4 if D == 256 and N == 32 else 8), 2
    std = _random_codes(rng, (B, H, N, 2 * D), e)
    kp0, vp0 = oracle.halves_from_standard(std, elem_bytes=e)
    kp, vp = _to_dev(kp0, e), _to_dev(vp0, e)
    skv.kv_page_convert(kp, vp)
    ks, vs = skv.kv_page_shuffle(_to_dev(std, e))
    torch.cuda.synchronize()
    assert torch.equal(kp, ks) and torch.equal(vp, vs)
