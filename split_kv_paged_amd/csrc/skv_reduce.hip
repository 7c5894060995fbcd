// Split reduce: log-sum-exp merge of a query token's per-segment partials.
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Modifications: the reduce kernel reads only the
// query token's own segment count. Each segment partial is the segment's
// softmax-normalized output with its natural-log sum-exp, so the merge is
//   M = max_s lse_s,  lse = M + ln sum_s e^(lse_s - M),
//   out = sum_s e^(lse_s - lse) * o_s.
//
// MI355X design: one wave64 per (token, q head); lane l owns channels 2l and
// 2l+1 (float2 loads, 512 contiguous bytes per segment); the segment weights
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

template <bool F16>
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
  const float* o_p = part_o + row * seg_max * kHeadDim;

  float2 acc = make_float2(0.f, 0.f);
  float lse = -INFINITY;
  if (nseg > 0 && nseg <= 64) {
    // lane s holds segment s. The first kPre partial rows are loaded before
    // the weights are known, so there is one memory round trip, not two.
    constexpr int kPre = 8;
    const float ls = lane < nseg ? lse_p[lane] : -INFINITY;
    float2 pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      // rows past nseg re-read the last valid row (weight 0): entries past a
      // token's segment count are unspecified and may hold NaN
      const int kk = k < nseg ? k : nseg - 1;
      pre[k] = reinterpret_cast<const float2*>(o_p + kk * kHeadDim)[lane];
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
        acc.x += wk * pre[k].x;
        acc.y += wk * pre[k].y;
      }
      for (int s = kPre; s < nseg; ++s) {
        const float ws = __shfl(w, s);
        const float2 o = reinterpret_cast<const float2*>(o_p + s * kHeadDim)[lane];
        acc.x += ws * o.x;
        acc.y += ws * o.y;
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
        const float2 o = reinterpret_cast<const float2*>(o_p + s * kHeadDim)[lane];
        acc.x += w * o.x;
        acc.y += w * o.y;
      }
    }
  }
  unsigned int packed;
  if constexpr (F16) {      // v_cvt_pk_f16_f32: round to nearest even, overflow to inf
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    const f16x2_t h = {static_cast<_Float16>(acc.x), static_cast<_Float16>(acc.y)};
    packed = __builtin_bit_cast(unsigned int, h);
  } else {
    packed = static_cast<unsigned int>(f32_to_bf16_rne(acc.x)) |
             (static_cast<unsigned int>(f32_to_bf16_rne(acc.y)) << 16);
  }
  reinterpret_cast<unsigned int*>(out + row * kHeadDim)[lane] = packed;
  if (out_lse && lane == 0) out_lse[row] = lse;
}

}  // namespace

int launch_reduce(const float* part_o, const float* part_lse,
                  const int32_t* tok_nseg, int total_q, int q_heads,
                  int seg_max, bool out_f16, void* out, float* out_lse, void* stream) {
  const long long rows = static_cast<long long>(total_q) * q_heads;
  const long long blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffffLL) return SKV_EUNSUPPORTED;
  if (out_f16)
    hipLaunchKernelGGL(reduce_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kReduceThreads), 0, static_cast<hipStream_t>(stream),
                       part_o, part_lse, tok_nseg, total_q, q_heads, seg_max,
                       static_cast<unsigned short*>(out), out_lse);
  else
    hipLaunchKernelGGL(reduce_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kReduceThreads), 0, static_cast<hipStream_t>(stream),
                       part_o, part_lse, tok_nseg, total_q, q_heads, seg_max,
                       static_cast<unsigned short*>(out), out_lse);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace skv
