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
// monotone in T (every per-sequence count ceil(n/T) is non-increasing), so the
// smallest feasible T is found by search between exact bounds (below):
//  * up to 4096 sequences (page counts cached in LDS): a 16-ary search, each
//    of the 16 waves testing one candidate T per pass with a wave-level
//    reduction over the batch, so a pass costs one barrier and the search
//    interval shrinks 17-fold per pass;
//  * larger batches: a binary search whose feasibility test is a block-wide
//    reduction over the sequences.
// Up to 1024 sequences every thread keeps its sequence's length, page count
// and query range in registers from the first load on, so the batch is read
// from memory once. The work list is written after a block-wide exclusive scan
// (wave scans plus one pass over the wave totals); the per-token counts use
// ceil(v / (T 2^s)) = ceil(ceil(v / 2^s) / T) in 32-bit integers. The launch
// shape never depends on device data, so the launch is graph-capture safe.
#include <hip/hip_runtime.h>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kWaves = kPlanThreads / 64;
constexpr int kLdsBs = 4096;         // page counts cached in LDS up to this batch size

__device__ __forceinline__ int pages_of(int L, int sh) {
  // ceil(L / 2^sh) (pages of 16 or 32 tokens) without forming L + 2^sh - 1
  // (L may be close to INT_MAX)
  return L <= 0 ? 0 : (L >> sh) + ((L & ((1 << sh) - 1)) != 0);
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

// Block-wide exclusive scan of one int per thread; also returns the total.
__device__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  __syncthreads();
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int t = wave_tot[w];
    before += w < wave ? t : 0;
    total += t;
  }
  return before + incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
    int bs, int kv_heads, int page_shift, int num_cus, int seg_max, int causal,
    int32_t* __restrict__ plan, int32_t* __restrict__ tok_nseg) {
  __shared__ long long red_s[kWaves];
  __shared__ int red_m[kWaves];
  __shared__ int wave_tot[kWaves];
  __shared__ int pages_lds[kLdsBs];
  __shared__ int feas[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cap = num_cus / kv_heads;
  const int width = cap > bs ? cap : bs;
  const bool one_per_thread = bs <= kPlanThreads;   // thread tid owns sequence tid

  // longest sequence, total pages and non-empty sequences (every load of the
  // batch issued here; the owned sequence's values stay in registers)
  int my_len = 0, my_pages = 0, my_c0 = 0, my_c1 = 0;
  if (one_per_thread && tid < bs) {
    my_len = seq_lens[tid];
    my_c0 = cu_q[tid];
    my_c1 = cu_q[tid + 1];
  }
  long long tot = 0;
  int mx = 0, nonempty = 0;
  if (one_per_thread) {
    my_pages = pages_of(my_len, page_shift);
    if (tid < bs) pages_lds[tid] = my_pages;
    tot = my_pages;
    mx = my_pages;
    nonempty = my_pages > 0;
  } else {
    for (int i = tid; i < bs; i += kPlanThreads) {
      const int n = pages_of(seq_lens[i], page_shift);
      if (bs <= kLdsBs) pages_lds[i] = n;
      mx = max(mx, n);
      tot += n;
      nonempty += n > 0;
    }
  }
  // the non-empty count travels in the high bits of the sum (tot < 2^47:
  // at most 2^15 sequences of fewer than 2^31 / 16 pages each)
  static_assert(kMaxBs < (1 << 15), "page total and count share one int64");
  {
    long long packed = tot + (static_cast<long long>(nonempty) << 47);
    block_sum_max(packed, mx, red_s, red_m);   // also publishes pages_lds
    tot = packed & ((1ll << 47) - 1);
    nonempty = static_cast<int>(packed >> 47);
  }
  const int upper = mx > 1 ? mx : 1;

  // Bounds on the answer. Necessary: sum ceil(n/T) >= sum n / T, so
  // T >= ceil(tot / cap); max ceil(n/T) <= seg_max iff T >= ceil(mx / seg_max).
  // Sufficient (k = non-empty sequences < cap): sum ceil(n/T) <= tot/T + k, so
  // T_ub = max(ceil(tot / (cap - k)), ceil(mx / seg_max)) is feasible. Some T
  // is feasible iff k <= cap (T = upper gives k segments of one each).
  int T;
  if (nonempty > cap) {
    T = upper;                                  // one segment per non-empty sequence
  } else {
    const long long need_sm = (static_cast<long long>(mx) + seg_max - 1) / seg_max;
    long long lo0 = cap > 0 ? (tot + cap - 1) / cap : 1;
    lo0 = lo0 > need_sm ? lo0 : need_sm;
    lo0 = lo0 < 1 ? 1 : lo0;
    long long hi0 = upper;
    if (nonempty < cap) {
      long long ub = (tot + (cap - nonempty) - 1) / (cap - nonempty);
      ub = ub > need_sm ? ub : need_sm;
      ub = ub < 1 ? 1 : ub;
      hi0 = ub < hi0 ? ub : hi0;
    }
    if (lo0 > hi0) lo0 = hi0;                   // cannot happen; keeps the search sane
    int lo = static_cast<int>(lo0), hi = static_cast<int>(hi0);   // hi feasible, lo-1 not
    if (bs <= kLdsBs) {
      // 16-ary search: wave w tests candidate lo + w * step of [lo, hi)
      while (lo < hi) {
        const int step = (hi - lo + kWaves - 1) / kWaves;
        const int cand = lo + wave * step;      // wave-uniform
        if (cand < hi) {
          long long sum = 0;
          int m = 0;
          for (int i = lane; i < bs; i += 64) {
            const int c = ceil_div_pos(pages_lds[i], cand);
            sum += c;
            m = max(m, c);
          }
          for (int off = 32; off > 0; off >>= 1) {
            sum += __shfl_xor(sum, off);
            m = max(m, __shfl_xor(m, off));
          }
          if (lane == 0) feas[wave] = sum <= cap && m <= seg_max;
        }
        __syncthreads();
        // candidates ascend with w and feasibility is monotone: the first
        // feasible one bounds the answer from above, the one before it below
        int first = kWaves, last_tested = -1;
        for (int w = 0; w < kWaves; ++w) {
          if (lo + w * step >= hi) break;
          last_tested = w;
          if (first == kWaves && feas[w]) first = w;
        }
        __syncthreads();                        // feas is rewritten next pass
        if (first < kWaves) {
          hi = lo + first * step;
          if (first > 0) lo = lo + (first - 1) * step + 1;
        } else {
          lo = lo + last_tested * step + 1;
        }
      }
      T = hi;
    } else {
      auto feasible = [&](int t) {
        long long sum = 0;
        int m = 0;
        for (int i = tid; i < bs; i += kPlanThreads) {
          const int c = ceil_div_pos(pages_of(seq_lens[i], page_shift), t);
          sum += c;
          m = max(m, c);
        }
        block_sum_max(sum, m, red_s, red_m);
        return sum <= cap && m <= seg_max;
      };
      while (lo < hi) {
        const int mid = lo + ((hi - lo) >> 1);
        if (feasible(mid)) hi = mid; else lo = mid + 1;
      }
      T = hi;
    }
  }

  // exclusive scan of segment counts over contiguous per-thread chunks
  const int chunk = (bs + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(bs, tid * chunk), i1 = min(bs, i0 + chunk);
  int local = 0;
  if (one_per_thread)
    local = ceil_div_pos(my_pages, T);
  else
    for (int i = i0; i < i1; ++i) local += ceil_div_pos(pages_of(seq_lens[i], page_shift), T);
  int total;
  int pos = block_exclusive_scan(local, wave_tot, total);
  if (one_per_thread) {
    for (int s = 0; s < local; ++s) plan[1 + pos + s] = (tid << 16) | s;
  } else {
    for (int i = i0; i < i1; ++i) {
      const int ns = ceil_div_pos(pages_of(seq_lens[i], page_shift), T);
      for (int s = 0; s < ns; ++s) plan[1 + pos + s] = (i << 16) | s;
      pos += ns;
    }
  }
  for (int k = total + tid; k < width; k += kPlanThreads) plan[1 + k] = -1;
  if (tid == 0) plan[0] = T;

  // per-token segment counts: ceil(visible / (T * page_size)), as the
  // visible page count over T
  auto token_counts = [&](int L, int c0, int qn) {
    for (int j = 0; j < qn; ++j) {
      long long vis = L;
      if (causal) {
        vis = static_cast<long long>(L) - qn + j + 1;
        vis = vis < 0 ? 0 : (vis > L ? L : vis);
      }
      tok_nseg[c0 + j] = ceil_div_pos(pages_of(static_cast<int>(vis), page_shift), T);
    }
  };
  if (one_per_thread) {
    if (tid < bs) token_counts(my_len, my_c0, my_c1 - my_c0);
  } else {
    for (int i = tid; i < bs; i += kPlanThreads) token_counts(seq_lens[i], cu_q[i], cu_q[i + 1] - cu_q[i]);
  }
}

}  // namespace

int launch_plan(const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                int total_q, int kv_heads, int page_size, int num_cus, int seg_max,
                int causal, int32_t* plan, int32_t* tok_nseg, void* stream) {
  (void)total_q;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0,
                     static_cast<hipStream_t>(stream), seq_lens, cu_seqlens_q,
                     bs, kv_heads, page_shift_of(page_size), num_cus, seg_max, causal,
                     plan, tok_nseg);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace skv
