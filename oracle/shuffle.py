"""Standard <-> shuffled KV page repack (test infrastructure; see
oracle/__init__.py).

[RFC, Background and Proposed Change §4]: a standard block holds, per head,
N token rows of 2D channels (K then V). The shuffled layout keeps K and V in
separate planes with x = 16 // element_size elements grouped per 16 bytes:
  K plane block [H, D/x, N, x]: element (c, n, i) is token n's K channel c*x + i;
  V plane block [H, N/x, D, x]: element (g, d, i) is token g*x + i's V channel d.
Written here as explicit destination <- source index maps; the inverse reads
the same maps backwards. Pure data movement: bit-exact on element codes.
"""
import numpy as np


def _maps(H, N, D, x):
    """Source coordinates (h, n, ch) in the standard block for every element
    of the K plane [H, D/x, N, x] and of the V plane [H, N/x, D, x]."""
    h, c, n, i = np.meshgrid(np.arange(H), np.arange(D // x), np.arange(N),
                             np.arange(x), indexing="ij")
    k_src = (h, n, c * x + i)
    h2, g, d, i2 = np.meshgrid(np.arange(H), np.arange(N // x), np.arange(D),
                               np.arange(x), indexing="ij")
    v_src = (h2, g * x + i2, D + d)
    return k_src, v_src


def shuffle_blocks(std, block_ids=None, elem_bytes=None):
    """std [B, H, N, 2D] element codes -> (k_plane [B, H, D/x, N, x],
    v_plane [B, H, N/x, D, x]) for the listed blocks (all when None).

    Blocks not listed are left as zeros in the returned planes; callers compare
    only the listed ones.
    """
    std = np.asarray(std)
    B, H, N, D2 = std.shape
    D = D2 // 2
    e = std.dtype.itemsize if elem_bytes is None else elem_bytes
    x = 16 // e
    kp = np.zeros((B, H, D // x, N, x), dtype=std.dtype)
    vp = np.zeros((B, H, N // x, D, x), dtype=std.dtype)
    k_src, v_src = _maps(H, N, D, x)
    ids = range(B) if block_ids is None else [int(b) for b in block_ids]
    for b in ids:
        kp[b] = std[b][k_src]
        vp[b] = std[b][v_src]
    return kp, vp


def unshuffle_blocks(k_plane, v_plane, elem_bytes=None):
    """Inverse of shuffle_blocks: planes -> standard [B, H, N, 2D]."""
    k_plane = np.asarray(k_plane)
    v_plane = np.asarray(v_plane)
    B, H, Dx, N, x = k_plane.shape
    D = Dx * x
    std = np.zeros((B, H, N, 2 * D), dtype=k_plane.dtype)
    k_src, v_src = _maps(H, N, D, x)
    for b in range(B):
        std[b][k_src] = k_plane[b]
        std[b][v_src] = v_plane[b]
    return std


# --- In-place conversion of received byte halves -----------------------------
#
# [RFC, Proposed Change §3 Descriptors and §4 Convert]: a decoder with separate
# K and V planes receives a remote standard block as two virtual regions of half
# a block each, so after the transfer the local K-plane block holds the standard
# block's first byte half and the V-plane block its second half (not K and V).
# The converter then rewrites each received block into the shuffled K and V
# planes. A block's halves split at byte H*N*D*e, which is a whole number of
# elements, so the split is taken here on element codes in the standard
# [H, N, 2D] order. With an odd head count one head straddles the two halves; a
# single head has its first N/2 token rows in the K plane and the rest in the V
# plane.


def halves_from_standard(std, block_ids=None, k_plane=None, v_plane=None, elem_bytes=None):
    """What the transfer leaves in the planes: for each listed block b of std
    [B, H, N, 2D], the first H*N*D element codes (standard order) go to K-plane
    block b and the rest to V-plane block b. Planes have the shuffled shapes
    [B, H, D/x, N, x] and [B, H, N/x, D, x] (x from the dtype); blocks not
    listed keep what the given planes held (zeros when none are given)."""
    std = np.asarray(std)
    B, H, N, D2 = std.shape
    D = D2 // 2
    x = 16 // (std.dtype.itemsize if elem_bytes is None else elem_bytes)
    kp = np.zeros((B, H, D // x, N, x), std.dtype) if k_plane is None else np.array(k_plane)
    vp = np.zeros((B, H, N // x, D, x), std.dtype) if v_plane is None else np.array(v_plane)
    half = H * N * D
    ids = range(B) if block_ids is None else [int(b) for b in block_ids]
    for b in ids:
        flat = std[b].reshape(-1)
        kp[b] = flat[:half].reshape(kp.shape[1:])
        vp[b] = flat[half:].reshape(vp.shape[1:])
    return kp, vp


def convert_halves(k_plane, v_plane, block_ids=None, elem_bytes=None):
    """Planes holding received byte halves -> planes holding the shuffled K and
    V of the listed blocks (all when None); other blocks are unchanged. Returns
    new arrays."""
    kp = np.array(k_plane)
    vp = np.array(v_plane)
    B, H, Dx, N, x = kp.shape
    D = Dx * x
    k_src, v_src = _maps(H, N, D, x)
    ids = range(B) if block_ids is None else [int(b) for b in block_ids]
    for b in ids:
        std = np.concatenate([kp[b].reshape(-1), vp[b].reshape(-1)]).reshape(H, N, 2 * D)
        kp[b] = std[k_src]
        vp[b] = std[v_src]
    return kp, vp


def revert_to_halves(k_plane, v_plane, block_ids=None, elem_bytes=None):
    """Inverse of convert_halves: shuffled planes -> the byte halves of each
    listed block's standard form; other blocks are unchanged."""
    kp = np.array(k_plane)
    vp = np.array(v_plane)
    B, H, Dx, N, x = kp.shape
    D = Dx * x
    half = H * N * D
    k_src, v_src = _maps(H, N, D, x)
    ids = range(B) if block_ids is None else [int(b) for b in block_ids]
    for b in ids:
        std = np.zeros((H, N, 2 * D), dtype=kp.dtype)
        std[k_src] = kp[b]
        std[v_src] = vp[b]
        flat = std.reshape(-1)
        kp[b] = flat[:half].reshape(kp.shape[1:])
        vp[b] = flat[half:].reshape(vp.shape[1:])
    return kp, vp


# --- Writing new tokens into the cache ----------------------------------------
#
# [RFC, Proposed Change §4]: the backend's cache writer places each new token's
# K and V at the slot its slot mapping names (block = slot // N, row = slot % N),
# straight into the shuffled planes; negative slots mark padding tokens and are
# skipped. Standard pages take the same token as one row of K then V channels.
# The pages never index past the cache; a slot at or past num_blocks * N names
# no row of it and is skipped like padding (reading taken: the write would land
# outside the cache, so it is dropped rather than wrapped or clamped).


def write_tokens_standard(std, key, value, slot_mapping):
    """std [B, H, N, 2D] with key/value [T, H, D] written at their slots
    (slots < 0 or >= B * N skipped); returns a new array."""
    std = np.array(std)
    B, H, N, D2 = std.shape
    D = D2 // 2
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= B * N:
            continue
        b, n = divmod(int(slot), N)
        std[b, :, n, :D] = key[t]
        std[b, :, n, D:] = value[t]
    return std


def write_tokens_shuffled(k_plane, v_plane, key, value, slot_mapping):
    """Planes [B, H, D/x, N, x] and [B, H, N/x, D, x] with key/value [T, H, D]
    written at their slots: token n of block b puts K channel c = c1*x + i at
    k_plane[b, h, c1, n, i] and V channel d at v_plane[b, h, n // x, d, n % x].
    Slots < 0 or >= B * N are skipped. Returns new arrays."""
    kp = np.array(k_plane)
    vp = np.array(v_plane)
    B, H, Dx, N, x = kp.shape
    D = Dx * x
    c = np.arange(D)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= B * N:
            continue
        b, n = divmod(int(slot), N)
        for h in range(H):
            kp[b, h, c // x, n, c % x] = key[t, h]
            vp[b, h, n // x, c, n % x] = value[t, h]
    return kp, vp
