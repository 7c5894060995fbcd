// Debug check of the attention calls' device-data contract: sequence lengths,
// the query prefix sums and the page-table entries the attention reads.
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Modifications: the plan and the segment kernel take
// seq_lens and cu_seqlens_q per sequence and read a sequence's pages through
// its page-table row; nothing there checks them, so a bad length or page id
// becomes an out-of-range access. This kernel finds such inputs before they
// are used.
//
// MI355X design: one 1024-thread work-group, integer compares only, nothing
// dereferenced through a page id. Per-sequence rules one thread per sequence;
// page-table rows of at most 64 entries one thread per row (entries loaded
// eight at a time), longer rows one wave per row with the lanes striding the
// entries. Violation bits and the smallest offending sequence are combined
// with LDS atomics (OR and MIN, independent of order) and written once.
#include <hip/hip_runtime.h>

#include <climits>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kShortRow = 64;        // rows up to this many entries: one thread each
constexpr int kLoads = 8;            // table entries loaded together per thread

__device__ __forceinline__ int pages_read(int L, int sh, int stride) {
  // entries the attention reads: ceil(L / 2^sh), at most the row's stride
  if (L <= 0) return 0;
  const int n = (L >> sh) + ((L & ((1 << sh) - 1)) != 0);
  return n < stride ? n : stride;
}

__global__ __launch_bounds__(kThreads) void check_kernel(
    const int32_t* __restrict__ table, int stride, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu, int bs, int total_q, int max_q, int sh, int num_blocks,
    int32_t* __restrict__ result) {
  __shared__ int s_mask, s_first;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    s_mask = 0;
    s_first = INT_MAX;
  }
  __syncthreads();
  int mask = 0, first = INT_MAX;
  auto flag = [&](int bits, int i) {
    mask |= bits;
    first = i < first ? i : first;
  };
  const long long cap = static_cast<long long>(stride) << sh;   // tokens a row can hold
  // what a row's entries [0, n) hold: 0 or SKV_BAD_PAGE_ID, from lane offset
  // `from` in steps of `step`
  auto scan_row = [&](int i, int n, int from, int step) {
    const int32_t* row = table + static_cast<size_t>(i) * stride;
    bool bad = false;
    for (int p0 = from; p0 < n; p0 += step * kLoads) {
      int id[kLoads];
#pragma unroll
      for (int k = 0; k < kLoads; ++k) {
        const int p = p0 + k * step;
        id[k] = row[p < n ? p : n - 1];                  // clamped: stays in the row
      }
#pragma unroll
      for (int k = 0; k < kLoads; ++k) bad |= id[k] < 0 || id[k] >= num_blocks;
    }
    return bad;
  };

  // per-sequence rules, and the short rows' entries
  for (int i = tid; i < bs; i += kThreads) {
    const int L = seq_lens[i];
    const int c0 = cu[i], c1 = cu[i + 1];
    if (L < 0)
      flag(SKV_BAD_LEN_NEGATIVE, i);
    else if (static_cast<long long>(L) > cap)
      flag(SKV_BAD_LEN_TABLE, i);
    if (c1 < c0 || (i == 0 && c0 != 0) || (i == bs - 1 && c1 != total_q))
      flag(SKV_BAD_CU, i);
    else if (c1 - c0 > max_q)
      flag(SKV_BAD_QLEN, i);
    const int n = pages_read(L, sh, stride);
    if (n > 0 && n <= kShortRow && scan_row(i, n, 0, 1)) flag(SKV_BAD_PAGE_ID, i);
  }
  // long rows: one wave per row
  for (int i = wave; i < bs; i += kWaves) {
    const int n = pages_read(seq_lens[i], sh, stride);      // wave-uniform
    if (n <= kShortRow) continue;
    const bool bad = scan_row(i, n, lane, 64);
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) flag(SKV_BAD_PAGE_ID, i);
  }
  if (mask) {
    atomicOr(&s_mask, mask);
    atomicMin(&s_first, first);
  }
  __syncthreads();
  if (tid == 0) {
    result[0] = s_mask;
    result[1] = s_mask ? s_first : -1;
  }
}

}  // namespace

int launch_check_inputs(const int32_t* page_table, int pt_stride, const int32_t* seq_lens,
                        const int32_t* cu_seqlens_q, int bs, int total_q, int max_q,
                        int page_size, int num_blocks, int32_t* result, void* stream) {
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), page_table, pt_stride, seq_lens,
                     cu_seqlens_q, bs, total_q, max_q, page_shift_of(page_size), num_blocks,
                     result);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace skv
