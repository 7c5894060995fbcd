// Split reduce: log-sum-exp merge of a query token's per-segment partials.
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Modifications: the reduce kernel reads only the
// query token's own segment count. Each segment partial is the segment's
// softmax-normalized output with its natural-log sum-exp, so the merge is
//   M = max_s lse_s,  lse = M + ln sum_s e^(lse_s - M),
//   out = sum_s e^(lse_s - lse) * o_s.
//
// MI355X design: lane l of a wave owns D/64 consecutive channels (2l and 2l+1
// at head dim 128: float2 loads, 512 contiguous bytes per segment; one or four
// channels at head dims 64 and 256); the weights are formed in fp32
// registers, the output rounded to bf16 or fp16 (RNE). Traffic is tiny next
// to the KV stream, so the kernel is latency-, not bandwidth-, shaped: what
// matters is how many partial rows are in flight at once and how many
// work-groups the launch has.
//  * Up to 256 segments per token, each lane holds the log-sum-exps of
//    segments lane, lane + 64, ... (all loaded at once), so the weights come
//    from one round trip and wave-level reductions; more segments take a
//    plain loop (max, sum, weighted rows).
//  * Narrow form (many (token, head) rows): one wave per row, four rows per
//    work-group; the first 8 partial rows are loaded before the weights are
//    known, the rest in chunks of 8 loads issued together.
//  * Wide form (at most 1024 rows, e.g. single-sequence batches whose
//    tokens each merge many segments): one work-group per row; in every
//    64-segment chunk wave w loads segments 16w .. 16w + 15 (the first
//    chunk's before the weights are known); the four partial sums are added
//    through LDS.
#include <hip/hip_runtime.h>

#include <math.h>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kReduceThreads = 256;
constexpr int kWavesPerBlock = kReduceThreads / 64;

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

// C = D / 64 consecutive channels per lane (D = 64, 128, 256)
template <int C>
struct LaneVec {
  float v[C];
};

template <int C>
__device__ __forceinline__ LaneVec<C> load_lane(const float* row, int lane) {
  LaneVec<C> r;
  if constexpr (C == 1) {
    r.v[0] = row[lane];
  } else if constexpr (C == 2) {
    const float2 t = reinterpret_cast<const float2*>(row)[lane];
    r.v[0] = t.x;
    r.v[1] = t.y;
  } else {
    const float4 t = reinterpret_cast<const float4*>(row)[lane];
    r.v[0] = t.x;
    r.v[1] = t.y;
    r.v[2] = t.z;
    r.v[3] = t.w;
  }
  return r;
}

template <bool F16>
__device__ __forceinline__ unsigned short to_out16(float f) {
  if constexpr (F16) {      // v_cvt_f16_f32: round to nearest even, overflow to inf
    return __builtin_bit_cast(unsigned short, static_cast<_Float16>(f));
  } else {
    return f32_to_bf16_rne(f);
  }
}

template <bool F16, int C>
__device__ __forceinline__ void store_row(unsigned short* orow, const LaneVec<C>& acc) {
  if constexpr (C == 1) {
    orow[0] = to_out16<F16>(acc.v[0]);
  } else if constexpr (C == 2) {
    *reinterpret_cast<unsigned int*>(orow) =
        static_cast<unsigned int>(to_out16<F16>(acc.v[0])) |
        (static_cast<unsigned int>(to_out16<F16>(acc.v[1])) << 16);
  } else {
    *reinterpret_cast<uint2*>(orow) = make_uint2(
        static_cast<unsigned int>(to_out16<F16>(acc.v[0])) |
            (static_cast<unsigned int>(to_out16<F16>(acc.v[1])) << 16),
        static_cast<unsigned int>(to_out16<F16>(acc.v[2])) |
            (static_cast<unsigned int>(to_out16<F16>(acc.v[3])) << 16));
  }
}

// General merge of one row by one wave, any segment count: max, then sum,
// then the weighted rows, 64 segments at a time. Returns the lse.
template <int D>
__device__ float merge_general(const float* lse_p, const float* o_p, int nseg, int lane,
                               LaneVec<D / 64>& acc) {
  constexpr int C = D / 64;
  float M = -INFINITY;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int s = s0 + lane;
    float v = s < nseg ? lse_p[s] : -INFINITY;
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    M = fmaxf(M, v);
  }
  if (M == -INFINITY) return -INFINITY;
  float sum = 0.f;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int s = s0 + lane;
    float v = s < nseg ? expf(lse_p[s] - M) : 0.f;
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    sum += v;
  }
  const float lse = M + logf(sum);
  for (int s0 = 0; s0 < nseg; s0 += 8) {
    LaneVec<C> o[8];
    float l[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {          // rows past nseg repeat the last one, weight 0
      const int s = s0 + k < nseg ? s0 + k : nseg - 1;
      o[k] = load_lane<C>(o_p + s * D, lane);
      l[k] = lse_p[s];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = s0 + k < nseg ? expf(l[k] - lse) : 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) acc.v[c] += w * o[k].v[c];
    }
  }
  return lse;
}

// Segments whose log-sum-exps a wave holds in registers, lane l holding
// segments l, l + 64, ... (NC of them): up to 64 * kChunks in all.
constexpr int kChunks = 4;
constexpr int kHeldSegs = 64 * kChunks;

// The log-sum-exps of up to 64 NC segments, lane l taking segments
// l, l + 64, ... (-inf past nseg); loaded ahead of the partial rows, so they
// arrive first.
template <int NC>
__device__ __forceinline__ void load_held(const float* lse_p, int nseg, int lane,
                                          float (&ls)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int s = 64 * c + lane;
    ls[c] = s < nseg ? lse_p[s] : -INFINITY;
  }
}

// Their weights: w[c] on lane l is segment 64 c + l's weight e^(lse_s - lse)
// (0 past nseg); returns the merged lse, -inf when no segment has a finite
// one (then every weight is 0).
template <int NC>
__device__ __forceinline__ float held_weights(const float (&ls)[NC], int nseg, int lane,
                                              float (&w)[NC]) {
  float M = ls[0];
#pragma unroll
  for (int c = 1; c < NC; ++c) M = fmaxf(M, ls[c]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (M == -INFINITY) {
#pragma unroll
    for (int c = 0; c < NC; ++c) w[c] = 0.f;
    return -INFINITY;
  }
  float e[NC], sum = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    e[c] = 64 * c + lane < nseg ? expf(ls[c] - M) : 0.f;
    sum += e[c];
  }
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
#pragma unroll
  for (int c = 0; c < NC; ++c) w[c] = e[c] / sum;
  return M + logf(sum);
}

// weight of segment s (wave-uniform, s < 64 NC) from the held weights
template <int NC>
__device__ __forceinline__ float held_weight(const float (&w)[NC], int s) {
  if constexpr (NC == 1) {
    return __shfl(w[0], s);
  } else {
    static_assert(NC == kChunks, "one or four chunks");
    const int c = s >> 6;
    const float v = c == 0 ? w[0] : (c == 1 ? w[1] : (c == 2 ? w[2] : w[3]));
    return __shfl(v, s & 63);
  }
}

// Narrow form, 1 <= nseg <= 64 NC: the first kPre partial rows are loaded
// before the weights are known (one memory round trip, not two), the rest in
// chunks of kPre rows with all loads of a chunk issued together. Rows past
// nseg re-read the last valid row with weight 0: entries past a token's
// segment count are unspecified and may hold NaN.
template <int NC, int D>
__device__ __forceinline__ float merge_held(const float* lse_p, const float* o_p, int nseg,
                                            int lane, LaneVec<D / 64>& acc) {
  constexpr int C = D / 64;
  constexpr int kPre = 8;
  float ls[NC];
  load_held<NC>(lse_p, nseg, lane, ls);
  LaneVec<C> pre[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int kk = k < nseg ? k : nseg - 1;
    pre[k] = load_lane<C>(o_p + kk * D, lane);
  }
  float wt[NC];
  const float lse = held_weights<NC>(ls, nseg, lane, wt);
  if (lse == -INFINITY) return lse;
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const float wk = k < nseg ? held_weight<NC>(wt, k) : 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) acc.v[c] += wk * pre[k].v[c];
  }
  for (int s0 = kPre; s0 < nseg; s0 += kPre) {
    LaneVec<C> o[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int kk = s0 + k < nseg ? s0 + k : nseg - 1;
      o[k] = load_lane<C>(o_p + kk * D, lane);
    }
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const float ws = s0 + k < nseg ? held_weight<NC>(wt, s0 + k) : 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) acc.v[c] += ws * o[k].v[c];
    }
  }
  return lse;
}

// Wide form's share of wave w, 1 <= nseg <= 64 NC: in every 64-segment chunk
// segments 16 w .. 16 w + 15, the first chunk's rows loaded before the weights
// are known. Every wave returns the merged lse.
template <int NC, int D>
__device__ __forceinline__ float merge_held_wide(const float* lse_p, const float* o_p,
                                                 int nseg, int w, int lane,
                                                 LaneVec<D / 64>& acc) {
  constexpr int C = D / 64;
  constexpr int kPer = 64 / kWavesPerBlock;       // segments per wave and chunk (16)
  const int s0 = kPer * w;
  float ls[NC];
  load_held<NC>(lse_p, nseg, lane, ls);
  LaneVec<C> pre[kPer];
  if (s0 < nseg) {                                 // wave-uniform
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int kk = s0 + k < nseg ? s0 + k : nseg - 1;
      pre[k] = load_lane<C>(o_p + kk * D, lane);
    }
  }
  float wt[NC];
  const float lse = held_weights<NC>(ls, nseg, lane, wt);
  if (lse == -INFINITY) return lse;                // uniform over the work-group
  if (s0 < nseg) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const float wk = s0 + k < nseg ? held_weight<NC>(wt, s0 + k) : 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) acc.v[c] += wk * pre[k].v[c];
    }
  }
  if constexpr (NC > 1) {
    for (int b = 64 + s0; b < nseg; b += 64) {     // later chunks, wave-uniform
      LaneVec<C> o[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int kk = b + k < nseg ? b + k : nseg - 1;
        o[k] = load_lane<C>(o_p + kk * D, lane);
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const float wk = b + k < nseg ? held_weight<NC>(wt, b + k) : 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) acc.v[c] += wk * o[k].v[c];
      }
    }
  }
  return lse;
}

// Wide form: one work-group of kWavesPerBlock waves per (token, q head) row.
template <bool F16, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_wide_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ tok_nseg, int q_heads, int seg_max,
    unsigned short* __restrict__ out, float* __restrict__ out_lse) {
  constexpr int C = D / 64;
  __shared__ float red[kWavesPerBlock - 1][64 * C];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const long long row = blockIdx.x;
  const int t = static_cast<int>(row / q_heads);
  int nseg = tok_nseg[t];
  nseg = nseg < 0 ? 0 : (nseg > seg_max ? seg_max : nseg);
  const float* lse_p = part_lse + row * seg_max;
  const float* o_p = part_o + row * seg_max * D;
  unsigned short* orow = out + row * D + C * lane;
  LaneVec<C> acc;
#pragma unroll
  for (int c = 0; c < C; ++c) acc.v[c] = 0.f;
  if (nseg > kHeldSegs || nseg == 0) {            // uniform over the work-group
    if (w == 0) {
      const float lse = nseg ? merge_general<D>(lse_p, o_p, nseg, lane, acc) : -INFINITY;
      store_row<F16, C>(orow, acc);
      if (out_lse && lane == 0) out_lse[row] = lse;
    }
    return;
  }
  const float lse = nseg <= 64 ? merge_held_wide<1, D>(lse_p, o_p, nseg, w, lane, acc)
                               : merge_held_wide<kChunks, D>(lse_p, o_p, nseg, w, lane, acc);
  if (w > 0) {
#pragma unroll
    for (int c = 0; c < C; ++c) red[w - 1][C * lane + c] = acc.v[c];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int j = 0; j < kWavesPerBlock - 1; ++j) {
#pragma unroll
      for (int c = 0; c < C; ++c) acc.v[c] += red[j][C * lane + c];
    }
    store_row<F16, C>(orow, acc);
    if (out_lse && lane == 0) out_lse[row] = lse;
  }
}

template <bool F16, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ tok_nseg, int total_q, int q_heads, int seg_max,
    unsigned short* __restrict__ out, float* __restrict__ out_lse) {
  const int lane = threadIdx.x & 63;
  const long long row = static_cast<long long>(blockIdx.x) * kWavesPerBlock +
                        (threadIdx.x >> 6);
  if (row >= static_cast<long long>(total_q) * q_heads) return;   // wave-uniform
  const int t = static_cast<int>(row / q_heads);
  int nseg = tok_nseg[t];
  nseg = nseg < 0 ? 0 : (nseg > seg_max ? seg_max : nseg);

  const float* lse_p = part_lse + row * seg_max;
  constexpr int C = D / 64;
  const float* o_p = part_o + row * seg_max * D;

  LaneVec<C> acc;
#pragma unroll
  for (int c = 0; c < C; ++c) acc.v[c] = 0.f;
  float lse = -INFINITY;
  if (nseg > 0 && nseg <= 64)
    lse = merge_held<1, D>(lse_p, o_p, nseg, lane, acc);
  else if (nseg > 64 && nseg <= kHeldSegs)
    lse = merge_held<kChunks, D>(lse_p, o_p, nseg, lane, acc);
  else if (nseg > kHeldSegs)
    lse = merge_general<D>(lse_p, o_p, nseg, lane, acc);
  store_row<F16, C>(out + row * D + C * lane, acc);
  if (out_lse && lane == 0) out_lse[row] = lse;
}

// rows up to which the wide form (one work-group per row) is used
constexpr long long kWideMaxRows = 1024;

template <int D>
void launch_reduce_d(const float* part_o, const float* part_lse, const int32_t* tok_nseg,
                     int total_q, int q_heads, int seg_max, bool out_f16, void* out,
                     float* out_lse, long long blocks, hipStream_t st) {
  const long long rows = static_cast<long long>(total_q) * q_heads;
  if (rows <= kWideMaxRows) {
    auto o = static_cast<unsigned short*>(out);
    if (out_f16)
      hipLaunchKernelGGL((reduce_wide_kernel<true, D>), dim3(static_cast<unsigned>(rows)),
                         dim3(kReduceThreads), 0, st, part_o, part_lse, tok_nseg, q_heads,
                         seg_max, o, out_lse);
    else
      hipLaunchKernelGGL((reduce_wide_kernel<false, D>), dim3(static_cast<unsigned>(rows)),
                         dim3(kReduceThreads), 0, st, part_o, part_lse, tok_nseg, q_heads,
                         seg_max, o, out_lse);
    return;
  }
  if (out_f16)
    hipLaunchKernelGGL((reduce_kernel<true, D>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kReduceThreads), 0, st, part_o, part_lse, tok_nseg, total_q,
                       q_heads, seg_max, static_cast<unsigned short*>(out), out_lse);
  else
    hipLaunchKernelGGL((reduce_kernel<false, D>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kReduceThreads), 0, st, part_o, part_lse, tok_nseg, total_q,
                       q_heads, seg_max, static_cast<unsigned short*>(out), out_lse);
}

}  // namespace

int launch_reduce(const float* part_o, const float* part_lse,
                  const int32_t* tok_nseg, int total_q, int q_heads, int head_dim,
                  int seg_max, bool out_f16, void* out, float* out_lse, void* stream) {
  const long long rows = static_cast<long long>(total_q) * q_heads;
  const long long blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffffLL) return SKV_EUNSUPPORTED;
  auto st = static_cast<hipStream_t>(stream);
  if (head_dim == 64)
    launch_reduce_d<64>(part_o, part_lse, tok_nseg, total_q, q_heads, seg_max, out_f16, out,
                        out_lse, blocks, st);
  else if (head_dim == 256)
    launch_reduce_d<256>(part_o, part_lse, tok_nseg, total_q, q_heads, seg_max, out_f16, out,
                         out_lse, blocks, st);
  else if (head_dim == kHeadDim)
    launch_reduce_d<kHeadDim>(part_o, part_lse, tok_nseg, total_q, q_heads, seg_max, out_f16,
                              out, out_lse, blocks, st);
  else
    return SKV_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace skv
