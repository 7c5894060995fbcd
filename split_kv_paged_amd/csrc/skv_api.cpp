// The C ABI declared in include/skv.h: argument checks, then kernel launches.
// Nothing here allocates, frees or synchronizes.
#include "skv.h"

#include "skv_internal.h"

namespace {

skv::AttnArgs make_attn_args(const void* q, const void* kv_a, const void* kv_b, int layout,
                             int kv_dtype, const int32_t* page_table, int pt_stride,
                             const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                             int total_q, int max_q, int q_heads, int kv_heads,
                             int head_dim, int page_size, const float* k_scale,
                             const float* v_scale,
                             int causal,
                             const int32_t* plan, int32_t* tok_nseg, int num_cus,
                             int seg_max, float* part_o, float* part_lse, int flags) {
  skv::AttnArgs a;
  a.flags = flags;
  a.q = q;
  a.kv_a = kv_a;
  a.kv_b = kv_b;
  a.layout = layout;
  a.kv_dtype = kv_dtype;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.bs = bs;
  a.total_q = total_q;
  a.max_q = max_q;
  a.head_dim = head_dim;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.page_size = page_size;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.causal = causal ? 1 : 0;
  a.plan = plan;
  a.tok_nseg = tok_nseg;
  a.num_cus = num_cus;
  a.seg_max = seg_max;
  a.part_o = part_o;
  a.part_lse = part_lse;
  return a;
}

}  // namespace

extern "C" {

size_t skv_plan_words(int bs, int kv_heads, int num_cus) {
  if (bs < 1 || kv_heads < 1 || num_cus < 1) return 0;
  return 1 + static_cast<size_t>(skv::plan_width(bs, kv_heads, num_cus));
}

size_t skv_workspace_bytes(int total_q, int q_heads, int head_dim, int seg_max) {
  if (total_q < 1 || q_heads < 1 || head_dim < 1 || seg_max < 1) return 0;
  const size_t rows = static_cast<size_t>(total_q) * q_heads * seg_max;
  return rows * head_dim * sizeof(float) + rows * sizeof(float);
}

int skv_plan_build(const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                   int total_q, int kv_heads, int page_size, int num_cus,
                   int seg_max, int causal, int32_t* plan, int32_t* tok_nseg,
                   void* stream) {
  int st = skv::check_plan_args(seq_lens, cu_seqlens_q, bs, total_q, kv_heads,
                                page_size, num_cus, seg_max, plan, tok_nseg);
  if (st != SKV_OK) return st;
  return skv::launch_plan(seq_lens, cu_seqlens_q, bs, total_q, kv_heads, page_size,
                          num_cus, seg_max, causal ? 1 : 0, plan, tok_nseg,
                          stream);
}

int skv_segment_attn(const void* q, const void* kv_a, const void* kv_b, int layout,
                     int kv_dtype, const int32_t* page_table, int pt_stride,
                     const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                     int total_q, int max_q, int q_heads, int kv_heads, int head_dim,
                     int page_size, const float* k_scale, const float* v_scale,
                     int causal, const int32_t* plan, int32_t* tok_nseg,
                     int num_cus, int seg_max, float* part_o, float* part_lse,
                     int flags, void* stream) {
  // `out` is not used by this call; pass a non-NULL stand-in to the shared check
  int st = skv::check_attn_args(q, kv_a, kv_b, layout, kv_dtype, page_table,
                                pt_stride, seq_lens, cu_seqlens_q, bs, total_q,
                                max_q, q_heads, kv_heads, head_dim, page_size,
                                k_scale, v_scale, plan, tok_nseg, num_cus,
                                seg_max, part_o, part_lse, part_o, flags);
  if (st != SKV_OK) return st;
  return skv::launch_segments(make_attn_args(q, kv_a, kv_b, layout, kv_dtype, page_table,
                                             pt_stride, seq_lens, cu_seqlens_q, bs, total_q,
                                             max_q, q_heads, kv_heads, head_dim, page_size, k_scale, v_scale,
                                             causal, plan, tok_nseg, num_cus, seg_max,
                                             part_o, part_lse, flags),
                              stream);
}

int skv_paged_decode_attn(const void* q, const void* kv_a, const void* kv_b,
                          int layout, int kv_dtype, const int32_t* page_table,
                          int pt_stride, const int32_t* seq_lens,
                          const int32_t* cu_seqlens_q, int bs, int total_q,
                          int max_q, int q_heads, int kv_heads, int head_dim,
                          int page_size, const float* k_scale,
                          const float* v_scale, int causal, const int32_t* plan,
                          int32_t* tok_nseg, int num_cus, int seg_max,
                          float* part_o, float* part_lse, void* out,
                          float* out_lse, int flags, void* stream) {
  int st = skv::check_attn_args(q, kv_a, kv_b, layout, kv_dtype, page_table,
                                pt_stride, seq_lens, cu_seqlens_q, bs, total_q,
                                max_q, q_heads, kv_heads, head_dim, page_size,
                                k_scale, v_scale, plan, tok_nseg, num_cus,
                                seg_max, part_o, part_lse, out, flags);
  if (st != SKV_OK) return st;
  st = skv::launch_segments(make_attn_args(q, kv_a, kv_b, layout, kv_dtype, page_table,
                                           pt_stride, seq_lens, cu_seqlens_q, bs, total_q,
                                           max_q, q_heads, kv_heads, head_dim, page_size, k_scale, v_scale,
                                           causal, plan, tok_nseg, num_cus, seg_max,
                                           part_o, part_lse, flags),
                            stream);
  if (st != SKV_OK) return st;
  return skv::launch_reduce(part_o, part_lse, tok_nseg, total_q, q_heads, head_dim,
                            seg_max, kv_dtype == SKV_KV_FP16, out, out_lse, stream);
}

int skv_split_reduce(const float* part_o, const float* part_lse,
                     const int32_t* tok_nseg, int total_q, int q_heads,
                     int head_dim, int seg_max, int out_dtype, void* out,
                     float* out_lse, void* stream) {
  int st = skv::check_reduce_args(part_o, part_lse, tok_nseg, total_q, q_heads,
                                  head_dim, seg_max, out_dtype, out);
  if (st != SKV_OK) return st;
  return skv::launch_reduce(part_o, part_lse, tok_nseg, total_q, q_heads, head_dim,
                            seg_max, out_dtype == SKV_KV_FP16, out, out_lse, stream);
}

int skv_kv_page_shuffle(const void* std_cache, void* k_plane, void* v_plane,
                        const int32_t* block_ids, int num_blocks, int kv_heads,
                        int page_size, int head_dim, int elem_bytes,
                        void* stream) {
  int st = skv::check_shuffle_args(std_cache, k_plane, v_plane, num_blocks,
                                   kv_heads, page_size, head_dim, elem_bytes);
  if (st != SKV_OK) return st;
  return skv::launch_shuffle(std_cache, k_plane, v_plane, block_ids, num_blocks,
                             kv_heads, page_size, head_dim, elem_bytes, stream);
}

int skv_kv_page_convert(void* k_plane, void* v_plane, const int32_t* block_ids,
                        int num_blocks, int kv_heads, int page_size,
                        int head_dim, int elem_bytes, int direction,
                        void* stream) {
  int st = skv::check_convert_args(k_plane, v_plane, num_blocks, kv_heads,
                                   page_size, head_dim, elem_bytes, direction);
  if (st != SKV_OK) return st;
  return skv::launch_convert(k_plane, v_plane, block_ids, num_blocks, kv_heads,
                             page_size, head_dim, elem_bytes, direction, stream);
}

int skv_kv_page_unshuffle(const void* k_plane, const void* v_plane,
                          void* std_cache, const int32_t* block_ids,
                          int num_blocks, int kv_heads, int page_size,
                          int head_dim, int elem_bytes, void* stream) {
  // the forward repack's argument rules
  int st = skv::check_shuffle_args(std_cache, k_plane, v_plane, num_blocks,
                                   kv_heads, page_size, head_dim, elem_bytes);
  if (st != SKV_OK) return st;
  return skv::launch_unshuffle(k_plane, v_plane, std_cache, block_ids,
                               num_blocks, kv_heads, page_size, head_dim, elem_bytes,
                               stream);
}

int skv_kv_cache_write(const void* key, const void* value,
                       const int64_t* slot_mapping, int num_tokens,
                       long long key_stride, long long value_stride,
                       void* k_plane, void* v_plane, int num_blocks,
                       int kv_heads, int page_size, int head_dim,
                       int elem_bytes, const float* k_scale,
                       const float* v_scale, void* stream) {
  int st = skv::check_cache_write_args(key, value, slot_mapping, num_tokens,
                                       key_stride, value_stride, k_plane, v_plane,
                                       num_blocks, kv_heads, page_size, head_dim,
                                       elem_bytes, k_scale, v_scale);
  if (st != SKV_OK) return st;
  return skv::launch_cache_write(key, value, slot_mapping, num_tokens, key_stride,
                                 value_stride, k_plane, v_plane, num_blocks,
                                 kv_heads, page_size, head_dim, elem_bytes, k_scale,
                                 v_scale, stream);
}

int skv_check_inputs(const int32_t* page_table, int pt_stride, const int32_t* seq_lens,
                     const int32_t* cu_seqlens_q, int bs, int total_q, int max_q,
                     int page_size, int num_blocks, int32_t* result, void* stream) {
  int st = skv::check_inputs_args(page_table, pt_stride, seq_lens, cu_seqlens_q, bs, total_q,
                                  max_q, page_size, num_blocks, result);
  if (st != SKV_OK) return st;
  return skv::launch_check_inputs(page_table, pt_stride, seq_lens, cu_seqlens_q, bs, total_q,
                                  max_q, page_size, num_blocks, result, stream);
}

const char* skv_strerror(int status) {
  switch (status) {
    case SKV_OK: return "ok";
    case SKV_EINVAL: return "invalid argument";
    case SKV_EUNSUPPORTED: return "unsupported geometry or type";
    case SKV_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
