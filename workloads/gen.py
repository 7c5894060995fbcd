"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only draws and lays out inputs (lengths, page tables, element codes
and poison); it holds none of the attention, planning, merging or shuffling
arithmetic. Both sides receive the same raw element codes (bf16 bit patterns
or OCP e4m3fn bytes) and decode them on their own.

Recipe (per config, seed = config.seed):
  * metadata from numpy PCG64 default_rng(seed), drawn in this order: physical
    block permutation of a pool of sum(ceil(L_i/P)) + extra_blocks blocks;
  * values from a torch.Generator seeded with `seed` on the target device:
    Q ~ N(0,1) rounded to bf16 (RNE; fp16 with an fp16 cache); K and V ~ N(0,1),
    rounded to bf16 or fp16, or divided by the per-tensor scale and rounded to
    e4m3fn with saturation to +-448 for fp8;
  * page-tail slots (token slots >= L_i mod P of a sequence's last page), the
    unused pool blocks and page-table entries past a sequence's last page hold
    poison (a large finite value by default, NaN in strict mode); the latter
    point at an unused, poisoned block so an out-of-range read changes results
    but never leaves the pool.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import Config

POISON_BF16 = {"finite": 0x46EA, "nan": 0x7FC0}   # 29952.0 and a quiet NaN
POISON_FP16 = {"finite": 0x7800, "nan": 0x7E00}   # 32768.0 and a quiet NaN
POISON_FP8 = {"finite": 0x7E, "nan": 0x7F}        # 448.0 and the e4m3fn NaN


@dataclass
class Case:
    cfg: Config
    seq_lens: torch.Tensor        # int32 [bs]
    cu_seqlens_q: torch.Tensor    # int32 [bs+1]
    page_table: torch.Tensor      # int32 [bs, pt_stride]
    q: torch.Tensor               # bf16 [total_q, Hq, D]
    kv: torch.Tensor              # bf16 or uint8 [pool, Hkv, P, 2D] (standard pages)
    k_scale: Optional[torch.Tensor]   # fp32 [1] or None
    v_scale: Optional[torch.Tensor]
    num_pool_blocks: int

    @property
    def pt_stride(self):
        return int(self.page_table.shape[1])


def layout_metadata(cfg: Config):
    """Host-side metadata: lengths, cu_seqlens_q, page table, pool size, poison slots."""
    rng = np.random.default_rng(cfg.seed)
    P = cfg.page_size
    L = np.asarray(cfg.seq_lens, dtype=np.int64)
    qn = np.asarray(cfg.q_lens, dtype=np.int64)
    n = (L + P - 1) // P
    used = int(n.sum())
    pool = used + cfg.extra_blocks
    perm = rng.permutation(pool).astype(np.int64)
    stride = max(int(n.max()) if len(n) else 1, 1)
    spare = int(perm[-1])  # an unused block (extra_blocks >= 1)
    table = np.full((len(L), stride), spare, dtype=np.int32)
    off = 0
    tails = []
    for i in range(len(L)):
        table[i, : n[i]] = perm[off: off + n[i]]
        off += int(n[i])
        r = int(L[i] % P)
        if r:
            tails.append((int(table[i, n[i] - 1]), r))
    cu = np.zeros(len(L) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(qn)
    unused = perm[used:]
    return dict(seq_lens=L.astype(np.int32), cu=cu, table=table, pool=pool,
                unused=unused, tails=tails)


def _fill_values(shape, gen, device, dtype, scale, chunk_rows=2048):
    out = torch.empty(shape, dtype={"bf16": torch.bfloat16, "fp16": torch.float16}.get(
        dtype, torch.uint8), device=device)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        if dtype in ("bf16", "fp16"):
            out[s:e] = x.to(out.dtype)
        else:
            y = (x / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
            out[s:e] = y.view(torch.uint8)
    return out


def make_case(cfg: Config, device="cpu", poison="finite") -> Case:
    meta = layout_metadata(cfg)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    D, P, Hkv = cfg.head_dim, cfg.page_size, cfg.kv_heads
    qdt = torch.float16 if cfg.kv_dtype == "fp16" else torch.bfloat16
    q = torch.randn((cfg.total_q, cfg.q_heads, D), generator=gen, device=device,
                    dtype=torch.float32).to(qdt)
    shape = (meta["pool"], Hkv, P, 2 * D)
    if cfg.kv_dtype in ("bf16", "fp16"):
        kv = _fill_values(shape, gen, device, cfg.kv_dtype, None)
    else:
        # K and V share one draw stream but use their own per-tensor scale
        kv = torch.empty(shape, dtype=torch.uint8, device=device)
        kv[..., :D] = _fill_values(shape[:-1] + (D,), gen, device, "fp8", cfg.k_scale)
        kv[..., D:] = _fill_values(shape[:-1] + (D,), gen, device, "fp8", cfg.v_scale)
    if poison != "none":
        raw = kv.view(torch.int16) if cfg.kv_dtype != "fp8" else kv
        pv = {"bf16": POISON_BF16, "fp16": POISON_FP16, "fp8": POISON_FP8}[cfg.kv_dtype][poison]
        if pv >= 0x8000:
            pv -= 0x10000
        if len(meta["unused"]):
            idx = torch.as_tensor(meta["unused"], device=device)
            raw[idx] = pv
        for blk, r in meta["tails"]:
            raw[blk, :, r:, :] = pv
    ks = vs = None
    if cfg.kv_dtype == "fp8":
        ks = torch.tensor([cfg.k_scale], dtype=torch.float32, device=device)
        vs = torch.tensor([cfg.v_scale], dtype=torch.float32, device=device)
    return Case(cfg=cfg,
                seq_lens=torch.as_tensor(meta["seq_lens"], device=device),
                cu_seqlens_q=torch.as_tensor(meta["cu"], device=device),
                page_table=torch.as_tensor(meta["table"], device=device),
                q=q, kv=kv, k_scale=ks, v_scale=vs, num_pool_blocks=meta["pool"])


def small_config(base: Config, seq_lens, q_lens, **kw) -> Config:
    """A copy of `base` with other lengths (parity sweeps and edge cases)."""
    d = dict(base.__dict__)
    d.update(seq_lens=list(seq_lens), q_lens=list(q_lens))
    d.update(kw)
    return Config(**d)


def raw_u16(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as its uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def raw_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def raw_kv(case: Case) -> np.ndarray:
    return raw_u8(case.kv) if case.cfg.kv_dtype == "fp8" else raw_u16(case.kv)
