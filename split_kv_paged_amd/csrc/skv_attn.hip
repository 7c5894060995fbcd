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

int launch_segments_mfma(const SegParams& sp, bool shuf, bool f16, int grid, hipStream_t st);
int launch_segments_valu(const SegParams& sp, bool shuf, bool f16, bool dual, int grid,
                         hipStream_t st);
int launch_segments_mfma_priv(const SegParams& sp, int e, bool f16, bool shuf, int max_rows,
                              int grid,
                              hipStream_t st);
int launch_segments_gd(const SegParams& sp, int head_dim, int e, bool f16, bool shuf, int grid,
                       hipStream_t st);

// Which kernel runs, by element type and query rows (GQA group x max query
// tokens); measured on MI355X:
//  * bf16, <= 4 rows: the vector-ALU kernel (5.6-6.0 TB/s; at 5+ rows its
//    rows x 128 fp32 FMAs per token make it compute-bound);
//  * bf16, 5-32 rows, and fp8 at any row count: matrix cores on private
//    per-wave rings (no barrier in the loop; fp8 K/V widened once), which a
//    single work-group streams ~35-42 GB/s through a CU against ~24-30 GB/s
//    for a shared ring: that is what skewed batches, with part of the CUs
//    idle, need;
//  * bf16, 33-64 rows: matrix cores on a ring shared by 8 waves (four row
//    tiles per block do not fit two waves per SIMD in private form).
// fp16 KV (with fp16 Q) takes the bf16 routes with the fp16 instructions.
// Head dims 64 and 256 run on the generic-width kernel at every row count.
// When at most half the CUs would be busy, more than 32 rows are split over
// two work-groups (below), which then take the 32-row routes.
constexpr int kValuMaxRows = 4;
constexpr int kPrivMaxRowsBf16 = 32;

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
  sp.page_shift = page_shift_of(a.page_size);
  sp.claim = (a.flags & SKV_ATTN_CLAIM_UNITS) ? 1 : 0;
  long long grid, busy;        // work-groups, and how many of them can carry work
  if (a.plan) {
    const long long w = plan_width(a.bs, a.kv_heads, a.num_cus);
    grid = w * a.kv_heads;
    // the work list is packed: at most seg_max segments per sequence, then -1
    const long long most = static_cast<long long>(a.bs) * a.seg_max;
    busy = (most < w ? most : w) * a.kv_heads;
  } else {
    // fixed split: one work-group per (sequence, segment, kv head)
    sp.fixed_S = fixed_split_count(a.bs, a.kv_heads, a.num_cus, a.seg_max);
    sp.tok_out = a.tok_nseg;
    grid = static_cast<long long>(sp.fixed_S) * a.bs * a.kv_heads;
    busy = grid;
  }
  if (grid > 0x7fffffffLL) return SKV_EUNSUPPORTED;
  const int e = a.kv_dtype == SKV_KV_FP8_E4M3FN ? 1 : 2;
  const bool f16 = a.kv_dtype == SKV_KV_FP16;      // fp16 Q and KV (else bf16 Q)
  const bool shuf = a.layout == SKV_LAYOUT_SHUFFLED;
  int rows = sp.G * a.max_q;
  auto st = static_cast<hipStream_t>(stream);
  // Fewer busy work-groups than half the CUs (single-sequence batches): one
  // work-group with more than 32 query rows is bound by what a single CU
  // computes and streams, not by HBM, so two work-groups share each item, 32
  // rows each, on the same XCD (so that the second reader of each page can
  // find it in that XCD's L2). For fp8 every row's arithmetic is unchanged, so the results
  // are the same bit for bit; 16-bit KV moves from the shared-ring kernel to
  // the private-ring one (the same sums in another order).
  sp.row_split = 1;
  sp.items = static_cast<int>(grid);
  if (a.head_dim == kHeadDim && rows > 32 && 2 * busy <= a.num_cus) {
    sp.row_split = 2;
    sp.items = static_cast<int>(busy);
    grid = (busy + 7) / 8 * 16;
    rows = 32;
  }
  // more work-groups than CUs: the shuffled vector-ALU kernel (one wave per
  // SIMD) runs two work-groups per CU with half-size rings, so that one's
  // prologue and merge overlap the other's streaming instead of leaving the
  // CU idle between consecutive work-groups (the 8-wave kernels gain nothing)
  const bool dual = grid > a.num_cus;
  if (a.head_dim != kHeadDim)             // 64 or 256: the generic-width kernel
    return launch_segments_gd(sp, a.head_dim, e, f16, shuf, static_cast<int>(grid), st);
  if (e == 2 && rows <= kValuMaxRows)
    return launch_segments_valu(sp, shuf, f16, dual, static_cast<int>(grid), st);
  if (e == 1 || rows <= kPrivMaxRowsBf16)
    return launch_segments_mfma_priv(sp, e, f16, shuf, rows, static_cast<int>(grid), st);
  return launch_segments_mfma(sp, shuf, f16, static_cast<int>(grid), st);
}

}  // namespace skv
