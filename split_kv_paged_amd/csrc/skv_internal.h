// Internal declarations shared by the host-side C ABI (skv_api.cpp), the
// host-only argument checks (skv_validate.cpp) and the kernel launchers
// (*.hip). Not part of the public interface.
#ifndef SKV_INTERNAL_H_
#define SKV_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

namespace skv {

constexpr int kHeadDim = 128;
constexpr int kPageSize = 16;
constexpr int kMaxQ = 4;
constexpr int kMaxRows = 64;     // (q_heads / kv_heads) * max_q
constexpr int kMaxBs = 32767;    // seq << 16 stays a non-negative int32
constexpr int kMaxSegMax = 65535;
constexpr int kMaxConvertBytes = 128 * 1024;   // one block staged in LDS

// page sizes of every entry point: 16- or 32-token pages (the attention
// kernels stream 16-token sub-pages; a 32-token page holds two)
inline bool repack_page_size_ok(int page_size) { return page_size == 16 || page_size == 32; }
inline int page_shift_of(int page_size) { return page_size == 32 ? 5 : 4; }   // log2

// head dims of every entry point (attention: 128 on the specialised kernels,
// 64 and 256 on the generic-width segment kernel)
inline bool head_dim_ok(int head_dim) { return head_dim == 64 || head_dim == 128 || head_dim == 256; }

// ---- host-only argument checks (skv_validate.cpp; no HIP headers) ----------
int check_plan_args(const void* seq_lens, const void* cu_seqlens_q, int bs,
                    int total_q, int kv_heads, int page_size, int num_cus,
                    int seg_max, const void* plan, const void* tok_nseg);
int check_inputs_args(const void* page_table, int pt_stride, const void* seq_lens,
                      const void* cu_seqlens_q, int bs, int total_q, int max_q,
                      int page_size, int num_blocks, const void* result);
int check_attn_args(const void* q, const void* kv_a, const void* kv_b,
                    int layout, int kv_dtype, const void* page_table,
                    int pt_stride, const void* seq_lens,
                    const void* cu_seqlens_q, int bs, int total_q, int max_q,
                    int q_heads, int kv_heads, int head_dim, int page_size,
                    const void* k_scale, const void* v_scale,
                    const void* plan, const void* tok_nseg, int num_cus,
                    int seg_max, const void* part_o, const void* part_lse,
                    const void* out, int flags);
int check_reduce_args(const void* part_o, const void* part_lse,
                      const void* tok_nseg, int total_q, int q_heads,
                      int head_dim, int seg_max, int out_dtype, const void* out);
int check_shuffle_args(const void* std_cache, const void* k_plane,
                       const void* v_plane, int num_blocks, int kv_heads,
                       int page_size, int head_dim, int elem_bytes);

int check_convert_args(const void* k_plane, const void* v_plane, int num_blocks,
                       int kv_heads, int page_size, int head_dim,
                       int elem_bytes, int direction);

int check_cache_write_args(const void* key, const void* value, const void* slots,
                           int num_tokens, long long key_stride,
                           long long value_stride, const void* k_plane,
                           const void* v_plane, int num_blocks, int kv_heads,
                           int page_size, int head_dim, int elem_bytes,
                           const void* k_scale, const void* v_scale);

// Segments per sequence of the fixed split: max(1, min(seg_max,
// pow2floor(num_cus / (bs * kv_heads)))).
inline int fixed_split_count(int bs, int kv_heads, int num_cus, int seg_max) {
  const long long q = static_cast<long long>(num_cus) / (static_cast<long long>(bs) * kv_heads);
  long long p = 1;
  while (p * 2 <= q) p *= 2;
  if (q < 1) p = 1;
  return static_cast<int>(p < seg_max ? p : seg_max);
}

inline int plan_width(int bs, int kv_heads, int num_cus) {
  int cap = num_cus / kv_heads;
  return cap > bs ? cap : bs;
}

// ---- kernel launchers (*.hip); return an skv_status ------------------------
struct AttnArgs {
  const void* q;
  const void* kv_a;
  const void* kv_b;
  int layout, kv_dtype;
  const int32_t* page_table;
  int pt_stride;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int bs, total_q, max_q, q_heads, kv_heads;
  int head_dim;              // 64, 128 or 256
  int page_size;             // 16 or 32 tokens
  const float* k_scale;
  const float* v_scale;
  int causal;
  const int32_t* plan;       // NULL: fixed split
  int32_t* tok_nseg;         // read by the reduce; written by the fixed split
  int num_cus, seg_max;
  float* part_o;
  float* part_lse;
  void* out;
  float* out_lse;
  int flags;                 // 0, SKV_ATTN_DETERMINISTIC or SKV_ATTN_CLAIM_UNITS
};

int launch_plan(const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                int total_q, int kv_heads, int page_size, int num_cus, int seg_max,
                int causal, int32_t* plan, int32_t* tok_nseg, void* stream);
int launch_segments(const AttnArgs& a, void* stream);
int launch_check_inputs(const int32_t* page_table, int pt_stride, const int32_t* seq_lens,
                        const int32_t* cu_seqlens_q, int bs, int total_q, int max_q,
                        int page_size, int num_blocks, int32_t* result, void* stream);
int launch_reduce(const float* part_o, const float* part_lse,
                  const int32_t* tok_nseg, int total_q, int q_heads, int head_dim,
                  int seg_max, bool out_f16, void* out, float* out_lse, void* stream);
int launch_shuffle(const void* std_cache, void* k_plane, void* v_plane,
                   const int32_t* block_ids, int num_blocks, int kv_heads,
                   int page_size, int head_dim, int elem_bytes, void* stream);
int launch_convert(void* k_plane, void* v_plane, const int32_t* block_ids,
                   int num_blocks, int kv_heads, int page_size, int head_dim,
                   int elem_bytes, int direction, void* stream);
int launch_unshuffle(const void* k_plane, const void* v_plane, void* std_cache,
                     const int32_t* block_ids, int num_blocks, int kv_heads,
                     int page_size, int head_dim, int elem_bytes, void* stream);
int launch_cache_write(const void* key, const void* value, const int64_t* slot_mapping,
                       int num_tokens, long long key_stride, long long value_stride,
                       void* k_plane, void* v_plane, int num_blocks, int kv_heads,
                       int page_size, int head_dim, int elem_bytes, const float* k_scale,
                       const float* v_scale, void* stream);

}  // namespace skv

#endif  // SKV_INTERNAL_H_
