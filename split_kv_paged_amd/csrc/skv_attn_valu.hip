// Segment attention, vector-ALU variant: bf16 or fp16 KV (F16: fp16 Q and
// KV) with at most 4 query rows (GQA group x query tokens), too few to fill a
// 16-row matrix-core tile.
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Motivation and Modifications: one work-group per
// (segment, sequence, kv head) writes the per-segment partial of all the
// sequence's query rows of that kv head; it decodes (seq, seg) from the work
// list and leaves on -1.
//
// MI355X design:
//  * NW wave64s (8 for standard pages, 4 for shuffled planes; measured); wave
//    w takes pages w, w+NW, ... of the segment and computes all query rows of
//    each, so no wave needs another's data: each wave streams its pages
//    through a private LDS ring (128 KB / NW; 64 KB / NW for the shuffled
//    form when the launch has more work-groups than CUs, two per CU) with
//    direct-to-LDS DMA
//    (global_load_lds_dwordx4, issued from inline asm) and waits only on its
//    own vmcnt — there is no barrier in the main loop. Two waves per SIMD hide
//    each other's LDS and DPP latencies; the shuffled layout's two planes
//    prefer the deeper four-page ring of four waves. Page ids are read through
//    the constant address space (scalar loads), so waiting on them never
//    drains the DMA queue.
//  * LDS tiles are laid out for the readers: K chunk-major ([16-byte chunk]
//    [token]) so a quad of lanes per token reads its 16-byte chunks
//    conflict-free; standard V row-major (one token's channel chunks per
//    lane group); shuffled V as the plane itself (x tokens of one channel per
//    16-byte chunk).
//  * q.k: four lanes per token (a quad), each owning 32 of the 128 channels,
//    v_dot2_f32_bf16 on bf16 pairs, the quad sum by two DPP quad permutes.
//    Row max: DPP row rotations within 16 lanes, then two lane permutes.
//  * p.V, standard pages: lane (token phase, channel chunk) accumulates in
//    fp32 with p from a per-wave LDS buffer; shuffled pages: a lane owns two
//    channels and takes v_dot2 over token pairs with bf16 p.
//  * Masked scores are forced to -inf and V of tokens past the segment end is
//    zeroed, so page-tail poison (even NaN) never reaches the accumulator.
//  * fp8 KV and 5..8 rows go to the matrix-core variant: there the vector
//    ALU's widening and rows x 128 fp32 FMAs per token cannot keep up with
//    HBM, while a partly filled 16-row MFMA tile can (measured).
#include "skv_attn_common.h"
#include "skv.h"

namespace skv {
namespace {

constexpr int kD = kHeadDim;
constexpr int kRows = 4;                       // query rows per work-group (padded)
constexpr int kHalf = kPageSize * kD * 2;      // a page's K (or V) half, bf16
constexpr int kPage = 2 * kHalf;
constexpr int kInstrPerPage = kPage / 1024;    // DMA instructions per page
constexpr int kStdRow = 2 * kD * 2;            // one standard token row

template <int NW, int RING_KB>
struct VRing {
  static constexpr int kBytes = RING_KB * 1024 / NW;   // this wave's ring
  static constexpr int kNS = kBytes / kPage;       // pages in it
  static_assert(kNS >= 2, "ring needs two pages");
  static_assert((kNS - 2) * kInstrPerPage <= 63, "vmcnt range");
  static_assert(kRows * kD * 4 <= kBytes, "the wave's output slot fits its ring");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vmcnt_pages(int k) {
  if constexpr (MAXK >= 6) { if (k >= 6) { wait_vmcnt<6 * STEP>(); return; } }
  if constexpr (MAXK >= 5) { if (k == 5) { wait_vmcnt<5 * STEP>(); return; } }
  if constexpr (MAXK >= 4) { if (k == 4) { wait_vmcnt<4 * STEP>(); return; } }
  if constexpr (MAXK >= 3) { if (k == 3) { wait_vmcnt<3 * STEP>(); return; } }
  if constexpr (MAXK >= 2) { if (k == 2) { wait_vmcnt<2 * STEP>(); return; } }
  if constexpr (MAXK >= 1) { if (k == 1) { wait_vmcnt<1 * STEP>(); return; } }
  wait_vmcnt<0>();
}

// One 16-token sub-page (this wave's) into its ring slot: K half chunk-major
// [c][token][16 B]; V half row-major [token][channels] (standard) or the
// plane's sub-page as is (shuffled).
template <bool SHUF, int PSH>
__device__ __forceinline__ void issue_page(const SegParams& p, const SegItem& it, int pid,
                                           int sub, uint8_t* slot, int lane) {
  const SubPageAddr a = sub_page<2, SHUF, PSH>(p, it.g, pid, sub);
  const uint8_t* ktile = a.k;
  const uint8_t* vtile = a.v;
  const int krow = kplane_row_bytes<PSH>();
#pragma unroll
  for (int i = 0; i < kHalf / 1024; ++i) {
    const int c = 4 * i + (lane >> 4), tau = lane & 15;
    const size_t off = SHUF ? static_cast<size_t>(c) * krow + tau * 16
                            : static_cast<size_t>(tau) * kStdRow + c * 16;
    dma16_lds<SHUF>(ktile + off, slot + i * 1024);   // shuffled: whole lines
  }
#pragma unroll
  for (int i = 0; i < kHalf / 1024; ++i) {
    size_t off;
    if constexpr (SHUF) {
      off = static_cast<size_t>(i * 64 + lane) * 16;
    } else {
      constexpr int kCpr = kD * 2 / 16;                  // chunks per V row
      const int tau = i * (64 / kCpr) + lane / kCpr, c = lane % kCpr;
      off = static_cast<size_t>(tau) * kStdRow + kD * 2 + c * 16;
    }
    dma16_lds<true>(vtile + off, slot + kHalf + i * 1024);   // whole rows or the plane
  }
}

// all-reduce max over the 16 token lanes (tq) that share a quarter qq
__device__ __forceinline__ float max_over_tokens(float v) {
  v = fmaxf(v, dpp<kDppRowRor4>(v));
  v = fmaxf(v, dpp<kDppRowRor8>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

template <bool SHUF, int NW, bool F16, int PSH, int RING_KB>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW * (128 / RING_KB) / 4, NW * (128 / RING_KB) / 4)))
void seg_valu_kernel(SegParams p) {
  using R = VRing<NW, RING_KB>;
  constexpr int kNS = R::kNS;
  constexpr int kThreads = 64 * NW;
  constexpr int RM = kRows;
  constexpr int kPBytes = SHUF ? RM * 16 * 2 : 16 * RM * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NW][R::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[NW][kPBytes];
  __shared__ float sm_m[NW][RM];
  __shared__ float sm_l[NW][RM];

  const SegItem it = decode_item(p);
  write_fixed_counts(p, it);
  if (!it.valid) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tq = lane >> 2, qq = lane & 3;
  const int seg_page0 = it.seg_start >> 4;
  const int seg_pages = (it.seg_end - it.seg_start + 15) >> 4;
  const int np = seg_pages > wave ? (seg_pages - wave + NW - 1) / NW : 0;
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(
          p.page_table + static_cast<size_t>(it.seq) * p.pt_stride);
  constexpr int psh = PSH - 4;
  const float sm_scale = kScoreScaleLog2;

  int lim[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) lim[r] = row_limit(it, r, p.G, p.causal);

  uint8_t* wring = ring[wave];
  // page ids: this wave's k-th sub-page is the segment's sub-page wave + NW k
  auto vpage = [&](int k) { return seg_page0 + wave + NW * k; };
  auto pid_of = [&](int k) { return ptab[vpage(k) >> psh]; };
  // Q rows (RM x 256 bytes) come by one DMA into the ring's last slot (not
  // used before the first iteration issues into it), ahead of the prologue's
  // pages, so the latencies overlap; the wait for Q counts only on the DMAs
  // issued after it (vector-memory loads complete in order). Lane i loads
  // bytes 16 (i % 16) .. +15 of row i / 16.
  static_assert(RM * kD * 2 == 64 * 16, "the Q rows are one DMA instruction");
  static_assert((kNS - 1) * kInstrPerPage <= 63, "vmcnt range");
  uint8_t* qslot = wring + (kNS - 1) * kPage;
  {
    const int r = lane >> 4;
    const bool okr = r < it.rows;
    const int t = it.c0 + (okr ? r / p.G : 0);
    const int h = it.g * p.G + (okr ? r % p.G : 0);
    dma16_lds<false>(p.q + (static_cast<size_t>(t) * p.Hq + h) * kD + (lane & 15) * 8,
                     qslot);                     // padding rows read row 0
  }
#pragma unroll
  for (int k = 0; k < kNS - 1; ++k)
    if (k < np) issue_page<SHUF, PSH>(p, it, pid_of(k), sub_of<PSH>(vpage(k)), wring + k * kPage, lane);
  int pid_next = kNS - 1 < np ? pid_of(kNS - 1) : 0;
  wait_vmcnt_pages<kInstrPerPage, kNS - 1>(min(kNS - 1, np));   // Q landed
  // Q rows (bf16 pairs) for this lane's 32 channels: chunk 4u+qq of row r
  uint4 qr[RM][4];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      qr[r][u] = *reinterpret_cast<const uint4*>(qslot + r * kD * 2 + (4 * u + qq) * 16);
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r >= it.rows) qr[r][u] = make_uint4(0, 0, 0, 0);
      asm volatile("" : "+v"(qr[r][u].x), "+v"(qr[r][u].y), "+v"(qr[r][u].z), "+v"(qr[r][u].w));
    }

  constexpr int kAcc = SHUF ? 2 : 8;
  float acc[RM][kAcc];
  float m[RM], l[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int a = 0; a < kAcc; ++a) acc[r][a] = 0.f;
  }
  uint8_t* pw = pbuf[wave];

  for (int k = 0; k < np; ++k) {
    wait_vmcnt_pages<kInstrPerPage, kNS - 2>(min(kNS - 2, np - 1 - k));
    if (k + kNS - 1 < np) {
      issue_page<SHUF, PSH>(p, it, pid_next, sub_of<PSH>(vpage(k + kNS - 1)),
                       wring + ((k + kNS - 1) % kNS) * kPage, lane);
      if (k + kNS < np) pid_next = pid_of(k + kNS);
    }
    const uint8_t* sK = wring + (k % kNS) * kPage;
    const uint8_t* sV = sK + kHalf;
    const int tok0 = it.seg_start + 16 * (wave + NW * k);
    const int vend = it.seg_end - tok0;        // tokens of this page before the end
    const bool tail = vend < 16;

    // ---- scores: token tq, this lane's quarter of the channels ----
    uint4 kw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      kw[u] = *reinterpret_cast<const uint4*>(sK + u * 1024 + (16 * qq + tq) * 16);
    float s[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      float a = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a = dot2<F16>(kw[u].x, qr[r][u].x, a);
        a = dot2<F16>(kw[u].y, qr[r][u].y, a);
        a = dot2<F16>(kw[u].z, qr[r][u].z, a);
        a = dot2<F16>(kw[u].w, qr[r][u].w, a);
      }
      a += dpp<kDppQuadXor1>(a);
      a += dpp<kDppQuadXor2>(a);
      s[r] = tok0 + tq < lim[r] ? a * sm_scale : -INFINITY;
    }

    // ---- online softmax per row; p to the wave's LDS buffer ----
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const float bm = max_over_tokens(s[r]);
      const float mn = fmaxf(m[r], bm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      if (mn != m[r]) {                        // row max moved (wave-uniform)
        const float alpha = fast_exp2(m[r] - mu);
        l[r] *= alpha;
#pragma unroll
        for (int a = 0; a < kAcc; ++a) acc[r][a] *= alpha;
        m[r] = mn;
      }
      s[r] = fast_exp2(s[r] - mu);
      l[r] += s[r];
    }
    if constexpr (!SHUF) {
      if (qq == 0) {                           // p[tau][r] fp32
        float* dst = reinterpret_cast<float*>(pw) + tq * RM;
        *reinterpret_cast<float4*>(dst) = make_float4(s[0], s[1], s[2], s[3]);
      }
    } else {                                   // p[r][tau] 16-bit; quarter qq: row qq
#pragma unroll
      for (int r = 0; r < RM; ++r)
        if ((r & 3) == qq) {
          if constexpr (F16)
            *reinterpret_cast<_Float16*>(pw + (r * 16 + tq) * 2) = static_cast<_Float16>(s[r]);
          else
            *reinterpret_cast<__bf16*>(pw + (r * 16 + tq) * 2) = static_cast<__bf16>(s[r]);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- o += p.V ----
    if constexpr (!SHUF) {
      constexpr int kCh = kD * 2 / 16;        // chunks per V row
      constexpr int kPh = 64 / kCh;           // token phases
      const int tp = lane / kCh, c = lane % kCh;
#pragma unroll
      for (int u = 0; u < 16 / kPh; ++u) {
        const int tau = tp + kPh * u;
        uint4 v = *reinterpret_cast<const uint4*>(sV + tau * (kD * 2) + c * 16);
        if (tail && tau >= vend) v = make_uint4(0, 0, 0, 0);
        const float x[kAcc] = {elem_lo<F16>(v.x), elem_hi<F16>(v.x), elem_lo<F16>(v.y),
                               elem_hi<F16>(v.y), elem_lo<F16>(v.z), elem_hi<F16>(v.z),
                               elem_lo<F16>(v.w), elem_hi<F16>(v.w)};
        const float4 pv = *reinterpret_cast<const float4*>(
            reinterpret_cast<const float*>(pw) + tau * RM);
        const float pp[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int a = 0; a < kAcc; ++a) acc[rr][a] += pp[rr] * x[a];
      }
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint4 vv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          vv[h] = *reinterpret_cast<const uint4*>(sV + (g * kD + lane + 64 * h) * 16);
          if (tail) {
            uint32_t w[4] = {vv[h].x, vv[h].y, vv[h].z, vv[h].w};
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
              const int rel = vend - (8 * g + 2 * q2);
              w[q2] = rel <= 0 ? 0u : (rel == 1 ? (w[q2] & 0xffffu) : w[q2]);
            }
            vv[h] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r) {
          const uint4 pp = *reinterpret_cast<const uint4*>(pw + (r * 16 + 8 * g) * 2);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float a = acc[r][h];
            a = dot2<F16>(vv[h].x, pp.x, a);
            a = dot2<F16>(vv[h].y, pp.y, a);
            a = dot2<F16>(vv[h].z, pp.z, a);
            a = dot2<F16>(vv[h].w, pp.w, a);
            acc[r][h] = a;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- per-wave totals into the wave's own ring, now idle ----
  wait_vmcnt<0>();
  float(*oslot)[kD] = reinterpret_cast<float(*)[kD]>(wring);   // [RM][kD]
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    float v = l[r];                            // identical within a quad: sum over tq only
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    l[r] = v;
  }
  if constexpr (!SHUF) {
    constexpr int kCh = kD * 2 / 16;
    const int tp = lane / kCh, c = lane % kCh;
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
      for (int a = 0; a < kAcc; ++a) {
        float v = acc[r][a];
        for (int off = kCh; off < 64; off <<= 1) v += __shfl_xor(v, off);
        acc[r][a] = v;
      }
    if (tp == 0) {
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int a = 0; a < kAcc; ++a) oslot[r][c * kAcc + a] = acc[r][a];
    }
  } else {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      oslot[r][lane] = acc[r][0];
      oslot[r][lane + 64] = acc[r][1];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      sm_m[wave][r] = m[r];
      sm_l[wave][r] = l[r];
    }
  }
  __syncthreads();

  // ---- merge waves: thread -> (row, channel) elements ----
  for (int e = threadIdx.x; e < RM * kD; e += kThreads) {
    const int r = e / kD, d = e % kD;
    if (r >= it.rows) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][r]);
    const float mu = M == -INFINITY ? 0.f : M;
    float Ls = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm_m[w][r] - mu);
      Ls += sm_l[w][r] * f;
      o += reinterpret_cast<const float(*)[kD]>(ring[w])[r][d] * f;
    }
    const int t = it.c0 + r / p.G;
    const int h = it.g * p.G + r % p.G;
    const size_t prow = (static_cast<size_t>(t) * p.Hq + h) * p.seg_max + it.seg;
    const bool any = Ls > 0.f;
    p.part_o[prow * kD + d] = any ? o / Ls : 0.f;
    if (d == 0) p.part_lse[prow] = any ? (mu + fast_log2(Ls)) * kLn2 : -INFINITY;
  }
}

}  // namespace

template <bool F16, int PSH>
int launch_valu(const SegParams& sp, bool shuf, bool dual, int grid, hipStream_t st) {
  if (shuf) {
    if (dual)
      hipLaunchKernelGGL((seg_valu_kernel<true, 4, F16, PSH, 64>), dim3(grid), dim3(64 * 4), 0, st, sp);
    else
      hipLaunchKernelGGL((seg_valu_kernel<true, 4, F16, PSH, 128>), dim3(grid), dim3(64 * 4), 0, st, sp);
  } else {
    // standard pages: the 8-wave form streams consecutive work-groups without
    // a gap measurable against a two-per-CU form (705 against 706 us on a
    // 128 x 8k decode batch)
    hipLaunchKernelGGL((seg_valu_kernel<false, 8, F16, PSH, 128>), dim3(grid), dim3(64 * 8), 0, st, sp);
  }
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

int launch_segments_valu(const SegParams& sp, bool shuf, bool f16, bool dual, int grid,
                         hipStream_t st) {
  if (sp.page_shift == 5)
    return f16 ? launch_valu<true, 5>(sp, shuf, dual, grid, st)
               : launch_valu<false, 5>(sp, shuf, dual, grid, st);
  return f16 ? launch_valu<true, 4>(sp, shuf, dual, grid, st)
             : launch_valu<false, 4>(sp, shuf, dual, grid, st);
}

}  // namespace skv
