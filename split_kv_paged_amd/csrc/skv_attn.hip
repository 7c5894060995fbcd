// Segment-attention launcher: picks the matrix-core or the vector-ALU kernel
// from the number of query rows a work-group carries (GQA group x max query
// tokens) and launches a 1-D grid over the work list x kv heads (planned
// split) or over sequences x segments x kv heads (fixed split, no plan).
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Modifications: the attention kernel is launched as
// a 1-D grid over the work list; padding entries (-1) exit at once.
#include "skv_attn_common.h"
#include "skv.h"

namespace skv {

int launch_segments_mfma(const SegParams& sp, int e, bool shuf, int max_rows, int grid,
                         hipStream_t st);
int launch_segments_valu(const SegParams& sp, bool shuf, int grid, hipStream_t st);
int launch_segments_mfma_priv(const SegParams& sp, bool shuf, int max_rows, int grid,
                              hipStream_t st);

// bf16 KV with at most this many rows goes to the vector-ALU kernel; the rest
// to 16-row matrix-core tiles. Measured on MI355X (balanced 32 x 60k batches):
// at 1-4 bf16 rows both kernels stream at 5.6-6.0 TB/s; at 5-8 rows the
// vector ALU's rows x 128 fp32 FMAs per token, and for fp8 at any row count the
// widening of every K and V element, make it compute-bound (1.7-3.4 TB/s)
// where a partly filled MFMA tile still streams at 5.3-5.9 TB/s.
constexpr int kValuMaxRows = 4;

int launch_segments(const AttnArgs& a, void* stream) {
  SegParams sp;
  sp.q = static_cast<const uint16_t*>(a.q);
  sp.kv_a = static_cast<const uint8_t*>(a.kv_a);
  sp.kv_b = static_cast<const uint8_t*>(a.kv_b);
  sp.page_table = a.page_table;
  sp.seq_lens = a.seq_lens;
  sp.cu_q = a.cu_seqlens_q;
  sp.plan = a.plan;
  sp.k_scale = a.k_scale;
  sp.v_scale = a.v_scale;
  sp.part_o = a.part_o;
  sp.part_lse = a.part_lse;
  sp.pt_stride = a.pt_stride;
  sp.bs = a.bs;
  sp.Hq = a.q_heads;
  sp.Hkv = a.kv_heads;
  sp.G = a.q_heads / a.kv_heads;
  sp.seg_max = a.seg_max;
  sp.causal = a.causal;
  sp.tok_out = nullptr;
  sp.fixed_S = 0;
  long long grid;
  if (a.plan) {
    grid = static_cast<long long>(plan_width(a.bs, a.kv_heads, a.num_cus)) * a.kv_heads;
  } else {
    // fixed split: one work-group per (sequence, segment, kv head)
    sp.fixed_S = fixed_split_count(a.bs, a.kv_heads, a.num_cus, a.seg_max);
    sp.tok_out = a.tok_nseg;
    grid = static_cast<long long>(sp.fixed_S) * a.bs * a.kv_heads;
  }
  if (grid > 0x7fffffffLL) return SKV_EUNSUPPORTED;
  const int e = a.kv_dtype == SKV_KV_FP8_E4M3FN ? 1 : 2;
  const bool shuf = a.layout == SKV_LAYOUT_SHUFFLED;
  const int rows = sp.G * a.max_q;
  auto st = static_cast<hipStream_t>(stream);
  if (e == 2 && rows <= kValuMaxRows)
    return launch_segments_valu(sp, shuf, static_cast<int>(grid), st);
  if (e == 1)       // fp8: private per-wave rings, K and V widened once per block
    return launch_segments_mfma_priv(sp, shuf, rows, static_cast<int>(grid), st);
  return launch_segments_mfma(sp, e, shuf, rows, static_cast<int>(grid), st);
}

}  // namespace skv
