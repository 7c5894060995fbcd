// Device helpers shared by the segment-attention kernels (gfx950).
#ifndef SKV_ATTN_COMMON_H_
#define SKV_ATTN_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skv_internal.h"

namespace skv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Kernel arguments of one segment-attention launch.
struct SegParams {
  const uint16_t* q;          // bf16 [total_q, Hq, 128]
  const uint8_t* kv_a;        // standard pages, or K plane
  const uint8_t* kv_b;        // V plane (shuffled layout)
  const int32_t* page_table;  // [bs, pt_stride]
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const int32_t* plan;
  const float* k_scale;       // fp8 only
  const float* v_scale;
  float* part_o;              // [total_q, Hq, seg_max, 128]
  float* part_lse;            // [total_q, Hq, seg_max]
  int32_t* tok_out;           // fixed split: per-token segment counts written here
  int pt_stride, bs, Hq, Hkv, G, seg_max, causal;
  int fixed_S;                // 0: planned split (plan); > 0: fixed split, S per sequence
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// 1/sqrt(128) * log2(e): scores enter exp2 directly
constexpr float kScoreScaleLog2 = 0.08838834764831845f * kLog2e;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// two fp32 -> packed bf16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// four OCP e4m3fn codes -> four bf16, two codes per v_cvt_scalef32_pk_bf16_fp8
// (scale 1; exact: 3 mantissa bits, 2^-9..448; word select 0 = bytes 0,1)
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 w) {
  const uint2 a = fp8x4_to_bf16x4(w.x), b = fp8x4_to_bf16x4(w.y);
  return make_uint4(a.x, a.y, b.x, b.y);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Work-item prologue shared by all variants [sglang PR #39172, Modifications:
// the segment kernel decodes (seq, seg) from its work-list word and leaves on
// -1 before touching memory; tiles per segment come from the first plan word].
// Without a plan (fixed_S > 0) the grid is (sequence, segment, kv head) and
// each sequence's pages are cut into fixed_S segments of ceil(pages / fixed_S)
// pages [same PR, Motivation: the fixed split gives every sequence the same
// segment count; Modifications: bs == 1 runs it without a plan].
struct SegItem {
  int valid;
  int seq, seg, g;
  int L, c0, qn, rows;
  int seg_start, seg_end;   // absolute token range of the segment
  int seg_pages;            // fixed split: pages per segment of this sequence
};

__device__ __forceinline__ SegItem decode_fixed(const SegParams& p) {
  SegItem it;
  it.valid = 0;
  const int widx = blockIdx.x / p.Hkv;
  it.g = blockIdx.x - widx * p.Hkv;
  it.seq = widx / p.fixed_S;
  it.seg = widx - it.seq * p.fixed_S;
  it.L = p.seq_lens[it.seq];
  it.c0 = p.cu_q[it.seq];
  it.qn = p.cu_q[it.seq + 1] - it.c0;
  it.rows = p.G * it.qn;
  const int pages = it.L <= 0 ? 0 : (it.L >> 4) + ((it.L & 15) != 0);
  it.seg_pages = pages == 0 ? 1 : 1 + (pages - 1) / p.fixed_S;
  const long long seg_tokens = static_cast<long long>(it.seg_pages) * kPageSize;
  const long long s0 = it.seg * seg_tokens;
  if (s0 >= it.L || it.qn <= 0) return it;
  const long long s1 = s0 + seg_tokens;
  it.seg_start = static_cast<int>(s0);
  it.seg_end = static_cast<int>(s1 < it.L ? s1 : it.L);
  it.valid = 1;
  return it;
}

// Fixed split: the (sequence, segment 0, kv head 0) work-group writes its
// tokens' segment counts, ceil(visible / segment tokens), for the reduce.
__device__ __forceinline__ void write_fixed_counts(const SegParams& p, const SegItem& it) {
  if (p.fixed_S == 0 || it.seg != 0 || it.g != 0) return;
  const int j = threadIdx.x;
  if (j >= it.qn) return;
  int vis = it.L;
  if (p.causal) {
    vis = it.L - it.qn + j + 1;
    vis = vis < 0 ? 0 : (vis > it.L ? it.L : vis);
  }
  const long long seg_tokens = static_cast<long long>(it.seg_pages) * kPageSize;
  p.tok_out[it.c0 + j] = vis <= 0 ? 0 : static_cast<int>(1 + (vis - 1) / seg_tokens);
}

__device__ __forceinline__ SegItem decode_item(const SegParams& p) {
  if (p.fixed_S > 0) return decode_fixed(p);
  SegItem it;
  it.valid = 0;
  const int widx = blockIdx.x / p.Hkv;
  it.g = blockIdx.x - widx * p.Hkv;
  const int word = p.plan[1 + widx];
  if (word < 0) return it;
  it.seq = word >> 16;
  it.seg = word & 0xffff;
  if (it.seq >= p.bs || it.seg >= p.seg_max) return it;
  const long long T = p.plan[0];
  it.L = p.seq_lens[it.seq];
  it.c0 = p.cu_q[it.seq];
  it.qn = p.cu_q[it.seq + 1] - it.c0;
  it.rows = p.G * it.qn;
  const long long s0 = static_cast<long long>(it.seg) * T * kPageSize;
  if (s0 >= it.L || it.qn <= 0) return it;
  const long long s1 = s0 + T * kPageSize;
  it.seg_start = static_cast<int>(s0);
  it.seg_end = static_cast<int>(s1 < it.L ? s1 : it.L);
  it.valid = 1;
  return it;
}

// Last key (exclusive) row n may see inside the segment: the bottom-right
// causal limit L - qn + j + 1 (clamped) or L, capped at the segment end.
__device__ __forceinline__ int row_limit(const SegItem& it, int n, int G, int causal) {
  if (n >= it.rows) return it.seg_start;       // padding row: nothing visible
  int vis = it.L;
  if (causal) {
    const int j = n / G;
    vis = it.L - it.qn + j + 1;
    vis = vis < 0 ? 0 : (vis > it.L ? it.L : vis);
  }
  return vis < it.seg_end ? vis : it.seg_end;
}

}  // namespace skv

#endif  // SKV_ATTN_COMMON_H_
