"""The five synthetic workloads: tiny correctness case, uniform long verify,
skewed agentic verify, fp8 KV, and shuffled-page decode.

Shapes follow the split-KV PR (sglang #39172, "[AMD] gfx950 assembly attention:
length-aware split-KV for dynamic workload", Accuracy Tests and Benchmarking and
Profiling) and, for the shuffled-page decode, the page-conversion RFC (vLLM
#59111, "NixlConnector: convert standard KV pages to ROCm AITER shuffled pages
on the decode side", Decode section: batch 64-128, 8k context, 16-token pages).

Length lists are literals written by `workloads/make_lengths.py`.
"""
from dataclasses import dataclass, field
from typing import List, Optional

# written by make_lengths.skew_lengths(): bs=20, sum 2,320,000
SKEW_LENS = [0, 1, 5, 17, 247999, 14719, 247999, 107452, 120562, 152813, 25149,
             150337, 79806, 247999, 237602, 133244, 143097, 97199, 66000, 248000]
SKEW_Q = [4, 4, 4, 2, 2, 3, 3, 3, 4, 2, 4, 1, 1, 4, 4, 2, 1, 2, 1, 4]

# written by make_lengths.skew16_lengths(): bs=16, sum 1,850,000
SKEW16_LENS = [0, 1, 5, 17, 28268, 46342, 175306, 70001, 199979, 247999, 27912, 247999, 65166,
               247999, 245006, 248000]

# written by make_lengths.fp8_lengths(): bs=64, median 8140, max 131072
FP8_LENS = [3673, 6607, 63486, 18438, 1087, 8140, 3803, 9836, 1132, 11031, 10945,
            56962, 12096, 15356, 1304, 131072, 775, 31792, 5458, 2771, 3653, 3583,
            13080, 7154, 50798, 862, 8161, 2733, 21287, 604, 5366, 10610, 1318,
            27543, 10207, 28286, 26674, 2453, 3069, 6378, 20568, 23348, 3420, 3880,
            3069, 3991, 6112, 6965, 103154, 4392, 5742, 14405, 2535, 5204, 8327,
            21241, 1622, 44306, 5309, 10091, 23237, 18475, 30169, 10138]
FP8_Q = [4, 4, 1, 4, 2, 1, 4, 1, 1, 4, 1, 3, 2, 1, 2, 3, 1, 1, 4, 3, 2, 3, 4, 3,
         3, 1, 1, 3, 3, 2, 3, 2, 4, 2, 3, 3, 3, 3, 3, 3, 1, 1, 2, 1, 4, 1, 3, 2,
         4, 2, 1, 1, 4, 3, 4, 2, 3, 3, 3, 3, 1, 4, 3, 3]


@dataclass
class Config:
    name: str
    seq_lens: List[int]
    q_lens: List[int]
    q_heads: int
    kv_heads: int
    head_dim: int = 128
    page_size: int = 16
    kv_dtype: str = "bf16"          # "bf16", "fp16" or "fp8" (OCP e4m3fn codes)
    layout: str = "standard"        # "standard" [H,N,2D] or "shuffled" planes
    num_cus: int = 256
    seg_max: int = 64
    causal: int = 1
    k_scale: Optional[float] = None
    v_scale: Optional[float] = None
    seed: int = 0
    extra_blocks: int = 8           # unused pool blocks, poison-filled
    note: str = field(default="", compare=False)

    @property
    def bs(self):
        return len(self.seq_lens)

    @property
    def total_q(self):
        return int(sum(self.q_lens))

    @property
    def max_q(self):
        return int(max(self.q_lens)) if self.q_lens else 1

    @property
    def elem_bytes(self):
        return 1 if self.kv_dtype == "fp8" else 2

    def kv_bytes(self):
        """Bytes of K and V the sequences hold: sum(L) * kv_heads * 2 * D * e."""
        return int(sum(self.seq_lens)) * self.kv_heads * 2 * self.head_dim * self.elem_bytes


TINY = Config("tiny", [37, 100], [1, 1], 8, 2, seed=1,
              note="bs=2, L={37,100}, q=1, 8/2 heads, bf16, random page table")
UNIFORM_VERIFY = Config("uniform_verify", [119_000] * 16, [4] * 16, 32, 2, seed=2,
                        note="bs=16 x 119k, q=4, 32/2 heads (GQA 16), bf16, permuted page table")
AGENTIC_SKEW = Config("agentic_skew", SKEW_LENS, SKEW_Q, 32, 2, seed=3,
                      note="bs=20, 2.32M tokens, lognormal + {0,1,5,17,248k}, q 1..4, bf16")
FP8_KV = Config("fp8_kv", FP8_LENS, FP8_Q, 16, 2, kv_dtype="fp8",
                k_scale=0.0173, v_scale=0.0211, seed=4,
                note="bs=64 lognormal (median 8k, max 128k), q 1..4, 16/2 heads, e4m3fn KV")
SHUFFLED_DECODE = Config("shuffled_decode", [8192] * 128, [1] * 128, 32, 8,
                         layout="shuffled", seed=5,
                         note="bs=128 x 8k, q=1, 32/8 heads, bf16, standard pages repacked")

CONFIGS = [TINY, UNIFORM_VERIFY, AGENTIC_SKEW, FP8_KV, SHUFFLED_DECODE]

# The split-KV PR's own MI355X kernel table (Benchmarking and Profiling: the
# 16 x 119k uniform verify and the bs 20 / 2.32M-token agentic verify) counts
# one byte per KV element, i.e. an fp8 cache. The same two batches with e4m3fn
# KV (the fp8 workload's scales) give like-for-like figures beside that table.
UNIFORM_VERIFY_FP8 = Config("uniform_verify_fp8", [119_000] * 16, [4] * 16, 32, 2,
                            kv_dtype="fp8", k_scale=0.0173, v_scale=0.0211, seed=6,
                            note="bs=16 x 119k, q=4, 32/2 heads (GQA 16), e4m3fn KV")
AGENTIC_SKEW_FP8 = Config("agentic_skew_fp8", SKEW_LENS, SKEW_Q, 32, 2, kv_dtype="fp8",
                          k_scale=0.0173, v_scale=0.0211, seed=7,
                          note="bs=20, 2.32M tokens, lognormal + {0,1,5,17,248k}, q 1..4, "
                               "e4m3fn KV")
# the uniform verify batch with an fp16 cache and fp16 queries (the RFC's
# decoder scope is BF16/FP16)
UNIFORM_VERIFY_FP16 = Config("uniform_verify_fp16", [119_000] * 16, [4] * 16, 32, 2,
                             kv_dtype="fp16", seed=8,
                             note="bs=16 x 119k, q=4, 32/2 heads (GQA 16), fp16 Q and KV")
# the uniform verify batch at head dims 64 and 256 (the generic-width kernel)
UNIFORM_VERIFY_D64 = Config("uniform_verify_d64", [119_000] * 16, [4] * 16, 32, 2,
                            head_dim=64, seed=9,
                            note="bs=16 x 119k, q=4, 32/2 heads (GQA 16), head dim 64, bf16")
UNIFORM_VERIFY_D256 = Config("uniform_verify_d256", [119_000] * 16, [4] * 16, 32, 2,
                             head_dim=256, seed=10,
                             note="bs=16 x 119k, q=4, 32/2 heads (GQA 16), head dim 256, bf16")
# The PR's two verify rows on agentic length distributions (4 query tokens per
# sequence, e4m3fn KV): bs 20 / 2.32M tokens (the skew lengths above) and
# bs 16 / 1.85M tokens
AGENTIC_VERIFY_FP8 = Config("agentic_verify_fp8", SKEW_LENS, [4] * 20, 32, 2, kv_dtype="fp8",
                            k_scale=0.0173, v_scale=0.0211, seed=16,
                            note="bs=20, 2.32M tokens, q=4, 32/2 heads, e4m3fn KV")
AGENTIC16_VERIFY_FP8 = Config("agentic16_verify_fp8", SKEW16_LENS, [4] * 16, 32, 2,
                              kv_dtype="fp8", k_scale=0.0173, v_scale=0.0211, seed=17,
                              note="bs=16, 1.85M tokens, q=4, 32/2 heads, e4m3fn KV")
# a grouped-query shape with fewer query heads per KV head (32/4 heads, GQA 8:
# 8-32 rows per work item, the 16-bit private-ring kernel) on the bs-16 agentic
# lengths with ragged 1..4 query tokens, bf16. (With 4 KV heads the plan's
# budget is 256 / 4 = 64 segments, so a batch of 64 or more sequences could
# not be split at all.)
SKEW_GQA8 = Config("skew_gqa8", SKEW16_LENS, SKEW_Q[:16], 32, 4, seed=18,
                   note="bs=16, 1.85M tokens, q 1..4, 32/4 heads (GQA 8), bf16")
EXTRA = [UNIFORM_VERIFY_FP8, AGENTIC_SKEW_FP8, AGENTIC_VERIFY_FP8, AGENTIC16_VERIFY_FP8,
         UNIFORM_VERIFY_FP16, UNIFORM_VERIFY_D64, UNIFORM_VERIFY_D256, SKEW_GQA8]
BY_NAME = {c.name: c for c in CONFIGS + EXTRA}

# The split-KV PR's single-sequence rows (Benchmarking and Profiling: "bs1
# 110k / 248k", run on the fixed split, which the planner bypasses at bs 1):
# one verify sequence of 110,000 or 248,000 tokens, 4 query tokens, 32/2
# heads, with an e4m3fn cache (the PR's table counts one byte per element)
# and with bf16.
BS1_110K_FP8 = Config("bs1_110k_fp8", [110_000], [4], 32, 2, kv_dtype="fp8",
                      k_scale=0.0173, v_scale=0.0211, seed=11,
                      note="bs=1 x 110k, q=4, 32/2 heads, e4m3fn KV")
BS1_248K_FP8 = Config("bs1_248k_fp8", [248_000], [4], 32, 2, kv_dtype="fp8",
                      k_scale=0.0173, v_scale=0.0211, seed=12,
                      note="bs=1 x 248k, q=4, 32/2 heads, e4m3fn KV")
BS1_110K = Config("bs1_110k", [110_000], [4], 32, 2, seed=13,
                  note="bs=1 x 110k, q=4, 32/2 heads, bf16")
BS1_248K = Config("bs1_248k", [248_000], [4], 32, 2, seed=14,
                  note="bs=1 x 248k, q=4, 32/2 heads, bf16")
BS1 = [BS1_110K_FP8, BS1_248K_FP8, BS1_110K, BS1_248K]
BY_NAME.update({c.name: c for c in BS1})
