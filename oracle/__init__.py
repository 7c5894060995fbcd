"""CPU oracle for paged split-KV decode/verify attention — TEST INFRASTRUCTURE.

Plain, slow, obviously-correct numpy code (fp64 for all floating point) that the
tests, the smoke check and the benchmark's CPU baseline compare the HIP path
against. Only `tests/`, `__graft_entry__.smoke()` and `bench.py`'s CPU-baseline
leg may import it; the product package never does, and this package imports
nothing from the product (it shares no code with it). Inputs come as the raw
element codes produced by `workloads.gen`, which both sides decode on their own.

Sources, cited by page title and section throughout:
  [RFC]  vLLM RFC #59111, "NixlConnector: convert standard KV pages to ROCm
         AITER shuffled pages on the decode side" — defines the standard
         [H, N, 2D] page and the shuffled K [H, D/x, N, x] / V [H, N/x, D, x]
         planes (Background; Proposed Change §4 "Convert").
  [PR]   sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware
         split-KV for dynamic workload" — the fixed split it replaces
         (Motivation), the length-aware planner, work list, per-token segment
         count, segment kernel and split reduce (Modifications), accuracy
         checks (Accuracy Tests).
  [OCP]  the OCP 8-bit floating point specification (E4M3 encoding), for the
         fp8 KV codes the RFC names in Proposed Change ("e4m3fn").
  [IEEE] IEEE 754 binary16, for the FP16 pages in the RFC's scope.

Modules:
  fp8        element decode (bf16 and fp16 bits, e4m3fn codes) and
             the rounding of values to e4m3fn codes             -- pinned
  attention  page gather + unsplit fp64 attention               -- pinned
  planner    length-aware segment planner, fixed split          -- pinned
  merge      per-segment partials and log-sum-exp merge         -- pinned
  shuffle    standard <-> shuffled page repack, the in-place
             conversion of received byte halves (+ inverse), and
             the cache writer (new tokens at their slots)       -- pinned
  contract   the plan and attention calls' device-data contract,
             checked input by input                             -- pinned
Every function is pinned by tests under tests/test_oracle_*.py against values
the pages print, closed forms, invariants, brute force or an independent
library routine; none is "parity unpinned".
"""
from .fp8 import (decode_bf16, decode_fp16, decode_q, fp16_value, decode_e4m3fn,
                  e4m3fn_value, decode_kv, encode_e4m3fn, quantize_e4m3fn)
from .attention import (gather_standard, gather_shuffled, visible_keys,
                        attend_one, decode_attention)
from .planner import plan_segments, fixed_split_segments, fixed_split_plan, pow2floor
from .merge import segment_partials, lse_merge, split_decode_attention
from .shuffle import (shuffle_blocks, unshuffle_blocks, halves_from_standard,
                      convert_halves, revert_to_halves, write_tokens_standard,
                      write_tokens_shuffled)
from .contract import check_inputs

__all__ = [
    "decode_bf16", "decode_fp16", "decode_q", "fp16_value", "decode_e4m3fn",
    "e4m3fn_value", "decode_kv", "encode_e4m3fn", "quantize_e4m3fn",
    "gather_standard", "gather_shuffled", "visible_keys", "attend_one",
    "decode_attention", "plan_segments", "fixed_split_segments", "fixed_split_plan",
    "pow2floor",
    "segment_partials", "lse_merge", "split_decode_attention",
    "shuffle_blocks", "unshuffle_blocks", "halves_from_standard", "convert_halves",
    "revert_to_halves", "write_tokens_standard", "write_tokens_shuffled",
    "check_inputs",
]
