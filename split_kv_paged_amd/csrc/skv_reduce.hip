// Split reduce: log-sum-exp merge of a query token's per-segment partials.
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Modifications: the reduce kernel reads only the
// query token's own segment count. Each segment partial is the segment's
// softmax-normalized output with its natural-log sum-exp, so the merge is
//   M = max_s lse_s,  lse = M + ln sum_s e^(lse_s - M),
//   out = sum_s e^(lse_s - lse) * o_s.
//
// MI355X design: one wave64 per (token, q head); lane l owns D/64 consecutive
// channels (2l and 2l+1 at head dim 128: float2 loads, 512 contiguous bytes
// per segment; one or four channels at head dims 64 and 256); the weights
// are formed in fp32 registers, the output rounded to bf16 or fp16 (RNE). Traffic is
// tiny next to the KV stream, so this kernel is latency-, not
// bandwidth-, shaped.
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
  if (nseg > 0 && nseg <= 64) {
    // lane s holds segment s. The first kPre partial rows are loaded before
    // the weights are known, so there is one memory round trip, not two.
    constexpr int kPre = 8;
    const float ls = lane < nseg ? lse_p[lane] : -INFINITY;
    LaneVec<C> pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      // rows past nseg re-read the last valid row (weight 0): entries past a
      // token's segment count are unspecified and may hold NaN
      const int kk = k < nseg ? k : nseg - 1;
      pre[k] = load_lane<C>(o_p + kk * D, lane);
    }
    float M = ls;
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (M != -INFINITY) {
      const float e = lane < nseg ? expf(ls - M) : 0.f;
      float sum = e;
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      lse = M + logf(sum);
      const float w = e / sum;
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        const float wk = __shfl(w, k);           // 0 for k >= nseg
#pragma unroll
        for (int c = 0; c < C; ++c) acc.v[c] += wk * pre[k].v[c];
      }
      for (int s = kPre; s < nseg; ++s) {
        const float ws = __shfl(w, s);
        const LaneVec<C> o = load_lane<C>(o_p + s * D, lane);
#pragma unroll
        for (int c = 0; c < C; ++c) acc.v[c] += ws * o.v[c];
      }
    }
  } else if (nseg > 64) {
    // general path: max, then sum, then weighted rows, 64 segments at a time
    float M = -INFINITY;
    for (int s0 = 0; s0 < nseg; s0 += 64) {
      const int s = s0 + lane;
      float v = s < nseg ? lse_p[s] : -INFINITY;
      for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
      M = fmaxf(M, v);
    }
    if (M != -INFINITY) {
      float sum = 0.f;
      for (int s0 = 0; s0 < nseg; s0 += 64) {
        const int s = s0 + lane;
        float v = s < nseg ? expf(lse_p[s] - M) : 0.f;
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        sum += v;
      }
      lse = M + logf(sum);
      for (int s = 0; s < nseg; ++s) {
        const float w = expf(lse_p[s] - lse);
        const LaneVec<C> o = load_lane<C>(o_p + s * D, lane);
#pragma unroll
        for (int c = 0; c < C; ++c) acc.v[c] += w * o.v[c];
      }
    }
  }
  unsigned short* orow = out + row * D + C * lane;
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
  if (out_lse && lane == 0) out_lse[row] = lse;
}

template <int D>
void launch_reduce_d(const float* part_o, const float* part_lse, const int32_t* tok_nseg,
                     int total_q, int q_heads, int seg_max, bool out_f16, void* out,
                     float* out_lse, long long blocks, hipStream_t st) {
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
