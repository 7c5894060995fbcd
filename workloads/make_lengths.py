"""Recipe that produced the literal length / query-count lists in configs.py.

Run `python -m workloads.make_lengths` to print them again; configs.py holds the
committed output so every consumer sees the same lists without re-drawing.

The skewed batches stand in for the "agentic length distribution" the split-KV
PR (sglang #39172, "[AMD] gfx950 assembly attention: length-aware split-KV for
dynamic workload", Benchmarking and Profiling table) measures from a trace replay
that is not available here: heavy-tailed lognormal lengths, with the tiny
sequences (0/1/5/17 tokens) and the single 248k request that its Accuracy Tests
section names.
"""
import numpy as np


def skew_lengths(seed=3, total=2_320_000, fixed=(0, 1, 5, 17, 248_000), n_draw=15):
    """bs=20: fixed lengths plus 15 lognormal(0,1) draws water-filled to `total`.

    Water-filling: find c with sum(min(cap, c*z_i)) == remaining, cap one below
    the long request so it stays the longest; round down and hand the remainder
    out one token at a time to the largest fractional parts (ties by index).
    """
    rng = np.random.default_rng(seed)
    z = rng.lognormal(0.0, 1.0, n_draw)
    remaining = total - sum(fixed)
    cap = max(fixed) - 1
    lo, hi = 0.0, float(remaining) / z.min() + 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(cap, mid * z).sum() < remaining:
            lo = mid
        else:
            hi = mid
    x = np.minimum(cap, hi * z)
    base = np.floor(x).astype(np.int64)
    rest = remaining - int(base.sum())
    frac = x - base
    order = sorted(range(n_draw), key=lambda i: (-frac[i], i))
    for i in order:
        if rest <= 0:
            break
        if base[i] < cap:
            base[i] += 1
            rest -= 1
    assert rest == 0 and int(base.sum()) == remaining
    lens = list(fixed[:4]) + [int(v) for v in base] + [fixed[4]]
    q = [int(v) for v in rng.integers(1, 5, size=len(lens))]
    return lens, q


def fp8_lengths(seed=4, bs=64, median=8192, max_len=131072):
    """bs=64: L = clamp(round(median * exp(s*z)), 1, max_len), s = ln(max/median)/max z."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(bs)
    s = np.log(max_len / median) / z.max()
    lens = np.clip(np.rint(median * np.exp(s * z)), 1, max_len).astype(np.int64)
    q = rng.integers(1, 5, size=bs)
    return [int(v) for v in lens], [int(v) for v in q]


def skew16_lengths():
    """bs=16, 1.85M tokens: the same recipe with 11 lognormal draws (the PR's
    "verify bs16, agentic length distribution, 1.85M tokens" row)."""
    lens, _ = skew_lengths(seed=15, total=1_850_000, n_draw=11)
    return lens


if __name__ == "__main__":
    l16 = skew16_lengths()
    print("SKEW16_LENS =", l16)
    print("sum", sum(l16))
    l3, q3 = skew_lengths()
    print("SKEW_LENS =", l3)
    print("SKEW_Q =", q3)
    print("sum", sum(l3))
    l4, q4 = fp8_lengths()
    print("FP8_LENS =", l4)
    print("FP8_Q =", q4)
    print("sum", sum(l4), "median", sorted(l4)[32], "max", max(l4))
