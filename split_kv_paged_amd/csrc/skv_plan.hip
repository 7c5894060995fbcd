// Length-aware segment planner, one work-group.
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Modifications: a single segment length T (in pages)
// is picked from the batch's sequence lengths — the smallest T that keeps the
// total segment count within num_CUs / kv_heads and every sequence within
// seg_max segments — and a compact work list of (seq << 16 | seg) words,
// padded with -1, is written with a per-query-token segment count.
//
// MI355X design: one 1024-thread work-group; integer math only. Feasibility is
// monotone in T (every per-sequence count ceil(n/T) is non-increasing), so a
// binary search over [1, max pages] returns the same T as a linear scan in
// O(log) block-wide reductions. The work list is emitted with a block-wide
// exclusive scan over per-sequence segment counts. Nothing depends on device
// data for the launch shape, so the launch is graph-capture safe.
#include <hip/hip_runtime.h>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kWaves = kPlanThreads / 64;

__device__ __forceinline__ int pages_of(int L) {
  // ceil(L / 16) without forming L + 15 (L may be close to INT_MAX)
  return L <= 0 ? 0 : (L >> 4) + ((L & 15) != 0);
}

__device__ __forceinline__ int ceil_div_pos(int a, int b) {
  return a <= 0 ? 0 : 1 + (a - 1) / b;
}

// Block-wide sum (int64) and max (int32); every thread gets both results.
__device__ void block_sum_max(long long& s, int& m, long long* red_s, int* red_m) {
  for (int off = 32; off > 0; off >>= 1) {
    s += __shfl_xor(s, off);
    m = max(m, __shfl_xor(m, off));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();                       // previous readers are done
  if (lane == 0) {
    red_s[wave] = s;
    red_m[wave] = m;
  }
  __syncthreads();
  s = 0;
  m = 0;
  for (int w = 0; w < kWaves; ++w) {
    s += red_s[w];
    m = max(m, red_m[w]);
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
    int bs, int kv_heads, int num_cus, int seg_max, int causal,
    int32_t* __restrict__ plan, int32_t* __restrict__ tok_nseg) {
  __shared__ long long red_s[kWaves];
  __shared__ int red_m[kWaves];
  __shared__ int scan[kPlanThreads];

  const int tid = threadIdx.x;
  const int cap = num_cus / kv_heads;
  const int width = cap > bs ? cap : bs;

  // longest sequence in pages
  long long dummy = 0;
  int mx = 0;
  for (int i = tid; i < bs; i += kPlanThreads) mx = max(mx, pages_of(seq_lens[i]));
  block_sum_max(dummy, mx, red_s, red_m);
  const int upper = mx > 1 ? mx : 1;

  // feasible(T): sum_i ceil(n_i/T) <= cap and max_i ceil(n_i/T) <= seg_max
  auto feasible = [&](int T) {
    long long s = 0;
    int m = 0;
    for (int i = tid; i < bs; i += kPlanThreads) {
      const int c = ceil_div_pos(pages_of(seq_lens[i]), T);
      s += c;
      m = max(m, c);
    }
    block_sum_max(s, m, red_s, red_m);
    return s <= cap && m <= seg_max;
  };

  int T;
  if (!feasible(upper)) {
    T = upper;                           // one segment per non-empty sequence
  } else {
    int lo = 1, hi = upper;              // invariant: feasible(hi)
    while (lo < hi) {
      const int mid = lo + ((hi - lo) >> 1);
      if (feasible(mid)) hi = mid; else lo = mid + 1;
    }
    T = hi;
  }

  // exclusive scan of segment counts over contiguous per-thread chunks
  const int chunk = (bs + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(bs, tid * chunk), i1 = min(bs, i0 + chunk);
  int local = 0;
  for (int i = i0; i < i1; ++i) local += ceil_div_pos(pages_of(seq_lens[i]), T);
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int total = scan[kPlanThreads - 1];
  int pos = scan[tid] - local;
  for (int i = i0; i < i1; ++i) {
    const int ns = ceil_div_pos(pages_of(seq_lens[i]), T);
    for (int s = 0; s < ns; ++s) plan[1 + pos + s] = (i << 16) | s;
    pos += ns;
  }
  for (int k = total + tid; k < width; k += kPlanThreads) plan[1 + k] = -1;
  if (tid == 0) plan[0] = T;

  // per-token segment counts: ceil(visible / (T * 16)), in 64-bit
  const long long seg_tokens = static_cast<long long>(T) * kPageSize;
  for (int i = tid; i < bs; i += kPlanThreads) {
    const int L = seq_lens[i];
    const int c0 = cu_q[i], qn = cu_q[i + 1] - c0;
    for (int j = 0; j < qn; ++j) {
      long long vis = L;
      if (causal) {
        vis = static_cast<long long>(L) - qn + j + 1;
        vis = vis < 0 ? 0 : (vis > L ? L : vis);
      }
      tok_nseg[c0 + j] = vis <= 0 ? 0 : static_cast<int>(1 + (vis - 1) / seg_tokens);
    }
  }
}

}  // namespace

int launch_plan(const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                int total_q, int kv_heads, int num_cus, int seg_max,
                int causal, int32_t* plan, int32_t* tok_nseg, void* stream) {
  (void)total_q;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0,
                     static_cast<hipStream_t>(stream), seq_lens, cu_seqlens_q,
                     bs, kv_heads, num_cus, seg_max, causal, plan, tok_nseg);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace skv
