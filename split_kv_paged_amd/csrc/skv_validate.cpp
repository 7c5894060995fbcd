// Host-only argument checks for the C ABI. Pure C++ (no HIP headers) so the
// error conventions documented in include/skv.h are testable without a GPU.
#include "skv_internal.h"

#include "skv.h"

namespace skv {

int check_plan_args(const void* seq_lens, const void* cu_seqlens_q, int bs,
                    int total_q, int kv_heads, int page_size, int num_cus,
                    int seg_max, const void* plan, const void* tok_nseg) {
  if (!seq_lens || !cu_seqlens_q || !plan || !tok_nseg) return SKV_EINVAL;
  if (bs < 1 || bs > kMaxBs || total_q < 1 || kv_heads < 1 || num_cus < 1)
    return SKV_EINVAL;
  if (seg_max < 1 || seg_max > kMaxSegMax) return SKV_EINVAL;
  if (!repack_page_size_ok(page_size)) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

int check_inputs_args(const void* page_table, int pt_stride, const void* seq_lens,
                      const void* cu_seqlens_q, int bs, int total_q, int max_q,
                      int page_size, int num_blocks, const void* result) {
  if (!page_table || !seq_lens || !cu_seqlens_q || !result) return SKV_EINVAL;
  if (bs < 1 || bs > kMaxBs || total_q < 1 || max_q < 1 || pt_stride < 1 || num_blocks < 1)
    return SKV_EINVAL;
  if (!repack_page_size_ok(page_size)) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

int check_attn_args(const void* q, const void* kv_a, const void* kv_b,
                    int layout, int kv_dtype, const void* page_table,
                    int pt_stride, const void* seq_lens,
                    const void* cu_seqlens_q, int bs, int total_q, int max_q,
                    int q_heads, int kv_heads, int head_dim, int page_size,
                    const void* k_scale, const void* v_scale,
                    const void* plan, const void* tok_nseg, int num_cus,
                    int seg_max, const void* part_o, const void* part_lse,
                    const void* out, int flags) {
  if (flags & ~(SKV_ATTN_DETERMINISTIC | SKV_ATTN_CLAIM_UNITS)) return SKV_EINVAL;
  if ((flags & SKV_ATTN_DETERMINISTIC) && (flags & SKV_ATTN_CLAIM_UNITS)) return SKV_EINVAL;
  (void)plan;   // NULL selects the fixed split
  if (!q || !kv_a || !page_table || !seq_lens || !cu_seqlens_q || !tok_nseg ||
      !part_o || !part_lse || !out)
    return SKV_EINVAL;
  if (layout != SKV_LAYOUT_STANDARD && layout != SKV_LAYOUT_SHUFFLED)
    return SKV_EINVAL;
  if (kv_dtype != SKV_KV_BF16 && kv_dtype != SKV_KV_FP8_E4M3FN && kv_dtype != SKV_KV_FP16)
    return SKV_EINVAL;
  if ((layout == SKV_LAYOUT_SHUFFLED) != (kv_b != nullptr)) return SKV_EINVAL;
  const bool fp8 = kv_dtype == SKV_KV_FP8_E4M3FN;
  if (fp8 && (!k_scale || !v_scale)) return SKV_EINVAL;
  if (!fp8 && (k_scale || v_scale)) return SKV_EINVAL;
  if (bs < 1 || bs > kMaxBs || total_q < 1 || q_heads < 1 || kv_heads < 1 ||
      num_cus < 1 || pt_stride < 1 || head_dim < 1 || page_size < 1)
    return SKV_EINVAL;
  if (q_heads % kv_heads != 0) return SKV_EINVAL;
  if (seg_max < 1 || seg_max > kMaxSegMax) return SKV_EINVAL;
  if (max_q < 1) return SKV_EINVAL;
  if (!head_dim_ok(head_dim) || !repack_page_size_ok(page_size)) return SKV_EUNSUPPORTED;
  if (max_q > kMaxQ) return SKV_EUNSUPPORTED;
  if ((q_heads / kv_heads) * max_q > kMaxRows) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

int check_reduce_args(const void* part_o, const void* part_lse,
                      const void* tok_nseg, int total_q, int q_heads,
                      int head_dim, int seg_max, int out_dtype, const void* out) {
  if (!part_o || !part_lse || !tok_nseg || !out) return SKV_EINVAL;
  if (out_dtype != SKV_KV_BF16 && out_dtype != SKV_KV_FP16) return SKV_EINVAL;
  if (total_q < 1 || q_heads < 1 || head_dim < 1) return SKV_EINVAL;
  if (seg_max < 1 || seg_max > kMaxSegMax) return SKV_EINVAL;
  if (!head_dim_ok(head_dim)) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

int check_shuffle_args(const void* std_cache, const void* k_plane,
                       const void* v_plane, int num_blocks, int kv_heads,
                       int page_size, int head_dim, int elem_bytes) {
  if (!std_cache || !k_plane || !v_plane) return SKV_EINVAL;
  if (num_blocks < 1 || kv_heads < 1 || page_size < 1 || head_dim < 1)
    return SKV_EINVAL;
  if (!head_dim_ok(head_dim) || !repack_page_size_ok(page_size)) return SKV_EUNSUPPORTED;
  if (elem_bytes != 1 && elem_bytes != 2) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

int check_convert_args(const void* k_plane, const void* v_plane, int num_blocks,
                       int kv_heads, int page_size, int head_dim,
                       int elem_bytes, int direction) {
  if (!k_plane || !v_plane) return SKV_EINVAL;
  if (num_blocks < 1 || kv_heads < 1 || page_size < 1 || head_dim < 1)
    return SKV_EINVAL;
  if (direction != SKV_TO_SHUFFLED && direction != SKV_TO_STANDARD)
    return SKV_EINVAL;
  if (!head_dim_ok(head_dim) || !repack_page_size_ok(page_size)) return SKV_EUNSUPPORTED;
  if (elem_bytes != 1 && elem_bytes != 2) return SKV_EUNSUPPORTED;
  const long long block = 2LL * kv_heads * page_size * head_dim * elem_bytes;
  if (block > kMaxConvertBytes) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

int check_cache_write_args(const void* key, const void* value, const void* slots,
                           int num_tokens, long long key_stride,
                           long long value_stride, const void* k_plane,
                           const void* v_plane, int num_blocks, int kv_heads,
                           int page_size, int head_dim, int elem_bytes,
                           const void* k_scale, const void* v_scale) {
  if (!key || !value || !slots || !k_plane || !v_plane) return SKV_EINVAL;
  if ((k_scale == nullptr) != (v_scale == nullptr)) return SKV_EINVAL;
  if (k_scale && elem_bytes != 1) return SKV_EINVAL;   // quantising needs an fp8 cache
  if (num_tokens < 1 || num_blocks < 1 || kv_heads < 1 || page_size < 1 ||
      head_dim < 1)
    return SKV_EINVAL;
  if (!head_dim_ok(head_dim) || !repack_page_size_ok(page_size)) return SKV_EUNSUPPORTED;
  if (elem_bytes != 1 && elem_bytes != 2) return SKV_EUNSUPPORTED;
  const long long row = static_cast<long long>(kv_heads) * head_dim;
  const int x = 16 / (k_scale ? 2 : elem_bytes);       // input rows: bf16 when quantising
  if (key_stride < row || value_stride < row) return SKV_EINVAL;
  if (key_stride % x != 0 || value_stride % x != 0) return SKV_EINVAL;
  return SKV_OK;
}

}  // namespace skv
