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
  int page_shift;             // log2(tokens per page): 4 or 5
  int claim;                  // 1: waves claim their units at run time; 0: fixed order
  int row_split;              // 1, or 2: two work-groups per item, each with half the rows
  int items;                  // work-groups before the row split ((item, kv head) pairs)
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

// ---- the 16-bit element type of Q, K, V and P: bf16, or IEEE fp16 (F16) with
// an fp16 cache. Operands travel as raw 16-bit patterns; these helpers pick
// the instruction. ----
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// D(16x16) += A(16x32) B(32x16), fp32 accumulate
template <bool F16>
__device__ __forceinline__ f32x4_t mfma_k32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x16) B(16x16), fp32 accumulate
template <bool F16>
__device__ __forceinline__ f32x4_t mfma_k16(i16x4_t a, i16x4_t b, f32x4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// two fp32 -> a packed pair, round to nearest even
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (F16) {
    const f16x2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    return pack_bf16x2(lo, hi);
  }
}

// a.x * b.x + a.y * b.y + c over packed pairs, fp32 accumulate
template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
  else
    return dot2_bf16(a, b, c);
}

// the low / high element of a packed pair, widened exactly to fp32
template <bool F16>
__device__ __forceinline__ float elem_lo(uint32_t w) {
  if constexpr (F16) return static_cast<float>(__builtin_bit_cast(f16x2_t, w).x);
  else return bf16_lo(w);
}
template <bool F16>
__device__ __forceinline__ float elem_hi(uint32_t w) {
  if constexpr (F16) return static_cast<float>(__builtin_bit_cast(f16x2_t, w).y);
  else return bf16_hi(w);
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
  int row0;                 // first query row of this work-group (row split: 0 or 32)
};

// The (item, kv head) index of this work-group and its share of the rows.
// With a row split, each group of 16 consecutive work-groups holds both
// halves of 8 items, the halves 8 apart, so that they run on the same XCD
// (work-group b on XCD b mod 8) and the second reader of a page can find it
// in that XCD's L2. Indices at or past p.items carry no work.
__device__ __forceinline__ int item_of_block(const SegParams& p, int& row0) {
  if (p.row_split < 2) {
    row0 = 0;
    return blockIdx.x;
  }
  const int r = blockIdx.x & 15;
  row0 = r >= 8 ? 32 : 0;
  return (blockIdx.x >> 4) * 8 + (r & 7);
}

__device__ __forceinline__ SegItem decode_fixed(const SegParams& p) {
  SegItem it;
  it.valid = 0;
  it.seg = -1;                                  // no counts written for a missing item
  const int bid = item_of_block(p, it.row0);
  if (bid >= p.items) return it;
  const int widx = bid / p.Hkv;
  it.g = bid - widx * p.Hkv;
  it.seq = widx / p.fixed_S;
  it.seg = widx - it.seq * p.fixed_S;
  it.L = p.seq_lens[it.seq];
  it.c0 = p.cu_q[it.seq];
  it.qn = p.cu_q[it.seq + 1] - it.c0;
  it.rows = p.G * it.qn;
  const int sh = p.page_shift;
  const int pages = it.L <= 0 ? 0 : (it.L >> sh) + ((it.L & ((1 << sh) - 1)) != 0);
  it.seg_pages = pages == 0 ? 1 : 1 + (pages - 1) / p.fixed_S;
  const long long seg_tokens = static_cast<long long>(it.seg_pages) << sh;
  const long long s0 = it.seg * seg_tokens;
  if (s0 >= it.L || it.qn <= 0) return it;
  const long long s1 = s0 + seg_tokens;
  it.seg_start = static_cast<int>(s0);
  it.seg_end = static_cast<int>(s1 < it.L ? s1 : it.L);
  if (it.row0 >= it.rows) return it;            // a row half with no rows of this sequence
  it.valid = 1;
  return it;
}

// Fixed split: the (sequence, segment 0, kv head 0) work-group writes its
// tokens' segment counts, ceil(visible / segment tokens), for the reduce.
__device__ __forceinline__ void write_fixed_counts(const SegParams& p, const SegItem& it) {
  if (p.fixed_S == 0 || it.seg != 0 || it.g != 0 || it.row0 != 0) return;
  const int j = threadIdx.x;
  if (j >= it.qn) return;
  int vis = it.L;
  if (p.causal) {
    vis = it.L - it.qn + j + 1;
    vis = vis < 0 ? 0 : (vis > it.L ? it.L : vis);
  }
  const long long seg_tokens = static_cast<long long>(it.seg_pages) << p.page_shift;
  p.tok_out[it.c0 + j] = vis <= 0 ? 0 : static_cast<int>(1 + (vis - 1) / seg_tokens);
}

__device__ __forceinline__ SegItem decode_item(const SegParams& p) {
  if (p.fixed_S > 0) return decode_fixed(p);
  SegItem it;
  it.valid = 0;
  it.seg = -1;                                  // no counts written for a missing item
  const int bid = item_of_block(p, it.row0);
  if (bid >= p.items) return it;
  const int widx = bid / p.Hkv;
  it.g = bid - widx * p.Hkv;
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
  const long long s0 = (static_cast<long long>(it.seg) * T) << p.page_shift;
  if (s0 >= it.L || it.qn <= 0) return it;
  const long long s1 = s0 + (T << p.page_shift);
  it.seg_start = static_cast<int>(s0);
  it.seg_end = static_cast<int>(s1 < it.L ? s1 : it.L);
  if (it.row0 >= it.rows) return it;            // a row half with no rows of this sequence
  it.valid = 1;
  return it;
}

// 16 bytes per lane, global -> LDS at lds_base + lane * 16 (lds_base
// wave-uniform): global_load_lds_dwordx4, issued from inline asm so that the
// only waits on it are the kernels' explicit vmcnt waits (the compiler would
// otherwise drain every DMA in flight before each LDS read).
// NT: the non-temporal (streaming) cache policy. Every KV byte is read once, by
// one work-group, and streamed reads reach markedly more of the HBM peak (a
// plain read kernel: 7.1 against 6.0-6.3 TB/s). It is used where each
// instruction covers whole 128-byte lines; where an instruction gathers half
// lines (16 token rows x 64 bytes), the default policy lets L2 serve the other
// half to the next instruction, and the streaming policy was slower there.
template <bool NT>
__device__ __forceinline__ void dma16_lds(const void* g, uint8_t* lds_uniform) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)(lds_uniform)));
  // the LDS base travels in M0, which the compiler loads for the statement
  if constexpr (NT)
    asm volatile("global_load_lds_dwordx4 %0, off nt" :: "v"(g), "{m0}"(lds) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(g), "{m0}"(lds) : "memory");
}

// The same from a wave-uniform base (held in SGPRs) plus a 32-bit per-lane
// byte offset: half the VGPRs of a 64-bit per-lane address.
template <bool NT>
__device__ __forceinline__ void dma16_lds_s(const uint8_t* base_uniform, uint32_t off,
                                            uint8_t* lds_uniform) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)(lds_uniform)));
  if constexpr (NT)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(off), "s"(base_uniform), "{m0}"(lds) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base_uniform), "{m0}"(lds) : "memory");
}

// 16-bit standard pages in LDS (matrix-core kernels): a page is its 16 token
// rows of 512 bytes (K channels, then V), copied two whole rows per DMA
// instruction, with each row's thirty-two 16-byte chunks XOR-swizzled by
// token: chunk q of row tau sits at position q ^ 2 tau. The K operand reads
// (16 tokens of one chunk) and the transposing V reads (4 tokens of two
// chunks per 16-lane group) then spread over all LDS banks. (An involution:
// the DMA lane at position p fetches chunk std2_chunk_pos(tau, p).)
__device__ __forceinline__ int std2_chunk_pos(int tau, int q) { return q ^ (2 * tau); }

// The next unit (32-token block of the segment) a wave of the fp8
// private-ring kernel streams after unit cur. Fixed order: wave w takes units
// w, w + NW, w + 2 NW, ... Claimed (p.claim): the next unit not yet taken,
// from a work-group counter in LDS that starts at NW (units 0 .. NW-1 go to
// waves 0 .. NW-1). The waves of a CU do not progress at one rate (each waits
// on its own DMA), so with a fixed share the work-group waits for its slowest
// wave; with claimed units they all finish within about one unit. Returns a
// wave-uniform value; once it reaches the unit count, every later one does.
// (The 16-bit private-ring and vector-ALU kernels keep the fixed order: claims
// gained nothing there, and cost 5% where one wave per SIMD waits on them.)
template <int NW>
__device__ __forceinline__ int next_unit(const SegParams& p, int cur, int* counter, int lane) {
  if (!p.claim) return cur + NW;
  int u = 0;
  if (lane == 0) u = atomicAdd(counter, 1);
  return __builtin_amdgcn_readfirstlane(u);
}

// Pages hold 16 or 32 tokens (PSH = log2 of the page size, a template
// argument of every attention kernel); the kernels stream 16-token sub-pages
// (a 32-token page holds two: its tokens 0-15 and 16-31). Sub-page v of a
// sequence (its tokens 16v .. 16v + 15) lies in page-table entry v >> (PSH - 4),
// as sub-page v & 1 of a 32-token page.
template <int PSH>
__device__ __forceinline__ int sub_of(int v) {
  return v & ((1 << (PSH - 4)) - 1);
}

// Addresses of one sub-page of kv head g in page pid, element size E bytes.
//  * Standard pages [blocks, Hkv, P, 2D]: k (== v) is the sub-page's first
//    token row; the rows of its 16 tokens follow contiguously (each K, then V).
//  * Shuffled planes K [blocks, Hkv, D/x, P, x], V [blocks, Hkv, P/x, D, x]:
//    k is the sub-page's first token in the K plane's chunk row 0 (chunk row c
//    at k + c * kplane_row_bytes); v is the sub-page's 16 / x token groups of
//    the V plane, laid out exactly as a 16-token page's V plane.
struct SubPageAddr {
  const uint8_t* k;
  const uint8_t* v;
};

template <int E, bool SHUF, int PSH>
__device__ __forceinline__ SubPageAddr sub_page(const SegParams& p, int g, int pid, int sub) {
  const size_t head = static_cast<size_t>(pid) * p.Hkv + g;
  constexpr size_t kHalf16 = static_cast<size_t>(kPageSize) * kHeadDim * E;   // 16 tokens' K or V
  if constexpr (SHUF) {
    const size_t plane = (head * kHalf16) << (PSH - 4);
    return {p.kv_a + plane + static_cast<size_t>(sub) * kPageSize * 16,
            p.kv_b + plane + static_cast<size_t>(sub) * kHalf16};
  } else {
    const uint8_t* t = p.kv_a + (((head << (PSH - 4)) + sub) * 2 * kHalf16);
    return {t, t};
  }
}

// bytes between consecutive 16-byte chunk rows of a K-plane tile: P tokens x 16 B
template <int PSH>
constexpr int kplane_row_bytes() {
  return 16 << PSH;
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
