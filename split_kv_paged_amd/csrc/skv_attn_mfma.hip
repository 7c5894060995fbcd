// Segment attention, matrix-core variant on a ring shared by all waves, used
// for bf16 or fp16 KV with 33-64 query rows (GQA group x query tokens, four
// 16-row tiles).
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Motivation and Modifications: one work-group per
// (segment, sequence, kv head) computes softmax(q.K^T/sqrt(d)).V of all the
// sequence's query rows for that kv head over the segment's pages and writes a
// per-segment partial; the work-group decodes (seq, seg) from the work list.
//
// MI355X design (the plan keeps about one work-group per CU, so one
// work-group must keep a CU's share of HBM bandwidth in flight by itself):
//  * KV pages stream into an LDS ring of NS stages with direct-to-LDS DMA
//    (global_load_lds_dwordx4: 16 bytes per lane, no VGPRs held). All four
//    waves issue the DMA of each stage, one (page, K or V half) unit at a time,
//    so every DMA instruction reads from a single page. Up to NS-1 stages
//    (>= 96 KB) are in flight per CU; one barrier per stage.
//  * Wave w owns query-row tile w % NRT (16 rows) and block w / NRT of each
//    stage, so a stage holds 4/NRT 32-token blocks and every wave has work.
//    Q (16 rows) lives in registers; the O^T accumulator is 32 registers.
//  * Scores are computed transposed per page, S^T = K.Q^T, with
//    v_mfma_f32_16x16x32_bf16: the C layout leaves each lane 4 tokens of one
//    row per page, and the two pages of a block form exactly the B operand
//    (P^T, 8 tokens) of O^T += V^T.P^T, with no lane shuffles.
//  * DMA lane->chunk maps are chosen for the readers: K operands are read back
//    as contiguous 16-byte lanes; standard-layout V is stored chunk-major
//    ([channel chunk][token]) and read with gfx950's transposing LDS reads
//    (ds_read_b64_tr_b16 / _tr_b8: four or eight tokens of one channel per
//    lane from one instruction, 512 contiguous bytes per wave, a constant
//    offset per channel tile); shuffled-layout V already holds x tokens of
//    one channel per 16-byte chunk (the reason that layout exists).
//  * Online softmax in the exp2 domain with the row max/sum in registers; the
//    block max is reduced across the four 16-lane groups with lane permutes;
//    the accumulator is rescaled only when a row max moved. Masked lanes are
//    forced to -inf and V of tokens past the segment end is zeroed, so stale
//    LDS or page-tail poison (even NaN) never reaches the accumulator.
#include <type_traits>

#include "skv_attn_common.h"
#include "skv.h"

namespace skv {
namespace {

constexpr int kD = kHeadDim;
constexpr int kRingBudget = 128 * 1024;   // measured faster than the full 160 KB
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));

// waves per work-group: 8 (two per SIMD, hiding each other's latencies) when
// the ring still holds four stages of the larger stage that implies, else 4
template <int E, int NRT>
constexpr int waves_for() {
  return 2 * (2 * (8 / NRT)) * kPageSize * kD * E * 4 <= kRingBudget ? 8 : 4;
}

template <int E, int NRT>
struct Ring {
  static constexpr int kWaves = waves_for<E, NRT>();
  static constexpr int kUnitBytes = kPageSize * kD * E;          // one page's K (or V) half
  static constexpr int kUnitInstr = kUnitBytes / 1024;            // DMA instructions per unit
  static constexpr int kBlocks = kWaves / NRT;                    // 32-token blocks per stage
  static constexpr int kPages = 2 * kBlocks;
  static constexpr int kStageTok = 16 * kPages;
  static constexpr int kStageBytes = 2 * kPages * kUnitBytes;
  static constexpr int kUnitsPerWave = 2 * kPages / kWaves;
  static_assert(kUnitsPerWave >= 1, "every wave issues DMA");
  static constexpr int kInstrPerWave = kUnitsPerWave * kUnitInstr;
  static constexpr int kNS0 = kRingBudget / kStageBytes;
  static constexpr int kNS = kNS0 > 8 ? 8 : kNS0;
  static_assert(kNS >= 2, "ring needs two stages");
  static_assert((kNS - 2) * kInstrPerWave <= 63, "vmcnt range");
  static constexpr int kStdTile = kPageSize * 2 * kD * E;        // standard (block, head)
  static constexpr int kStdRow = 2 * kD * E;
};

// s_waitcnt vmcnt(N): the DMA loads this wave issued before the last N are done
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// work-group barrier that is also a compiler memory barrier, with no implied
// wait on outstanding vector-memory loads (the DMA ring stays in flight)
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("s_barrier" ::: "memory");
}

template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vmcnt_stages(int k) {
  // wait until at most k stages' worth (k * STEP instructions) remain in flight
  if constexpr (MAXK >= 6) { if (k >= 6) { wait_vmcnt<6 * STEP>(); return; } }
  if constexpr (MAXK >= 5) { if (k == 5) { wait_vmcnt<5 * STEP>(); return; } }
  if constexpr (MAXK >= 4) { if (k == 4) { wait_vmcnt<4 * STEP>(); return; } }
  if constexpr (MAXK >= 3) { if (k == 3) { wait_vmcnt<3 * STEP>(); return; } }
  if constexpr (MAXK >= 2) { if (k == 2) { wait_vmcnt<2 * STEP>(); return; } }
  if constexpr (MAXK >= 1) { if (k == 1) { wait_vmcnt<1 * STEP>(); return; } }
  wait_vmcnt<0>();
}


// Issue this wave's DMA units of one stage. Unit u of the stage is (16-token
// sub-page u/2, K half if u even, V half if odd); wave w issues units
// [w*UPW, (w+1)*UPW). v0 is the stage's first sub-page in the sequence.
// Sub-pages past the segment end are read from the segment's first sub-page
// (same instruction count keeps vmcnt exact; their tokens are masked and
// zeroed).
template <int E, bool SHUF, int NRT, int PSH>
__device__ __forceinline__ void issue_stage(const SegParams& p, const SegItem& it,
                                            const int* pids, const int* subs, uint8_t* slot,
                                            int wave, int lane) {
  using R = Ring<E, NRT>;
  const int r16 = lane & 15, j4 = lane >> 4;
  const int krow = kplane_row_bytes<PSH>();
#pragma unroll
  for (int uw = 0; uw < R::kUnitsPerWave; ++uw) {
    const int u = wave * R::kUnitsPerWave + uw;
    const int pg = u >> 1;
    const bool vhalf = u & 1;
    const SubPageAddr a = sub_page<E, SHUF, PSH>(p, it.g, pids[uw], subs[uw]);
    uint8_t* dst = slot + (2 * pg + (vhalf ? 1 : 0)) * R::kUnitBytes;
    if constexpr (!SHUF) {
      // bf16 standard pages: unit (page, row half h) = token rows 8h .. 8h+7
      // (K then V, 512 bytes each), two whole rows (1 KB of contiguous HBM) per
      // instruction, streamed; chunk q of row tau lands at position
      // std2_chunk_pos(tau, q) of the row
      const int h = u & 1;
#pragma unroll
      for (int i = 0; i < R::kUnitInstr; ++i) {
        const int row = 8 * h + 2 * i + (lane >> 5);
        const int q = std2_chunk_pos(row, lane & 31);          // the chunk stored there
        dma16_lds<true>(a.k + static_cast<size_t>(row) * R::kStdRow + q * 16, dst + i * 1024);
      }
      continue;
    }
    // shuffled planes: the K plane's chunk rows (lane reads the 16 bytes
    // compute-lane `lane` needs for k-step i) and the V plane as it is, whole
    // lines, streamed
    if (!vhalf) {
#pragma unroll
      for (int i = 0; i < R::kUnitInstr; ++i)
        dma16_lds<true>(a.k + static_cast<size_t>(4 * i + j4) * krow + r16 * 16,
                        dst + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < R::kUnitInstr; ++i)
        dma16_lds<true>(a.v + static_cast<size_t>(i * 64 + lane) * 16, dst + i * 1024);
    }
  }
}

template <int E, bool SHUF, int NRT, bool F16, int PSH>
__global__ __launch_bounds__((64 * Ring<E, NRT>::kWaves))
__attribute__((amdgpu_waves_per_eu((Ring<E, NRT>::kWaves / 4), (Ring<E, NRT>::kWaves / 4))))
void seg_mfma_kernel(SegParams p) {
  using R = Ring<E, NRT>;
  constexpr int kNS = R::kNS;
  constexpr int kWaves = R::kWaves;
  // the ring is the kernel's only LDS; after the loop it is reused for the
  // cross-wave merge (per-wave O^T tiles, then row max and sum)
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kNS * R::kStageBytes];
  static_assert(kWaves * 8 * 64 * 16 + 2 * kWaves * 16 * 4 <= kNS * R::kStageBytes,
                "merge scratch fits in the ring");
  float(*sm_m)[16] = reinterpret_cast<float(*)[16]>(ring + kWaves * 8 * 64 * 16);
  float(*sm_l)[16] = reinterpret_cast<float(*)[16]>(ring + kWaves * 8 * 64 * 16 + kWaves * 16 * 4);

  const SegItem it = decode_item(p);
  write_fixed_counts(p, it);
  if (!it.valid) return;                                          // work-group uniform
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, j4 = lane >> 4;
  const int rt = wave % NRT, bis = wave / NRT;
  const int nrt = (it.rows + 15) >> 4;
  const bool active = rt < nrt;                                   // wave-uniform
  const int ntok = it.seg_end - it.seg_start;
  const int nst = (ntok + R::kStageTok - 1) / R::kStageTok;
  const int seg_page0 = it.seg_start >> 4;
  const int seg_pages = (ntok + 15) >> 4;
  // page ids are read through the constant address space: scalar loads, so
  // waiting on them never waits on the vector-memory (DMA) queue
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(
          p.page_table + static_cast<size_t>(it.seq) * p.pt_stride);
  // scores enter exp2 as fma(raw, c, -m); c > 0 (16-bit KV has no scale)
  static_assert(E == 2, "the shared-ring kernel runs 16-bit KV");
  constexpr float c = kScoreScaleLog2;
  constexpr float out_scale = 1.f;

  // page ids and sub-pages of this wave's units for a stage (sub-pages past
  // the end -> the segment's first)
  constexpr int psh = PSH - 4;
  auto load_pids = [&](int st, int* out) {
#pragma unroll
    for (int uw = 0; uw < R::kUnitsPerWave; ++uw) {
      const int pg = st * R::kPages + ((wave * R::kUnitsPerWave + uw) >> 1);
      out[uw] = ptab[(seg_page0 + (pg < seg_pages ? pg : 0)) >> psh];
    }
  };
  auto stage_subs = [&](int st, int* out) {
#pragma unroll
    for (int uw = 0; uw < R::kUnitsPerWave; ++uw) {
      const int pg = st * R::kPages + ((wave * R::kUnitsPerWave + uw) >> 1);
      out[uw] = sub_of<PSH>(seg_page0 + (pg < seg_pages ? pg : 0));
    }
  };

  // ---- Q rows of this wave's tile (B operand of S^T = K.Q^T) ----
  // Q comes through the same LDS DMA, into the ring's last stage (not used
  // before the first iteration issues into it), ahead of the prologue's
  // stages: its latency overlaps theirs, and the wait for it below counts
  // only on the DMAs issued after it (vector-memory loads complete in order).
  // Wave w's 4 KB: piece kk at + kk * 1 KB, lane l's 16 bytes at + l * 16.
  static_assert(kWaves * 4096 <= R::kStageBytes && kNS >= 2, "Q fits the last stage");
  uint8_t* qstage = ring + (kNS - 1) * R::kStageBytes + wave * 4096;
  const int n = 16 * rt + r16;
  const int lim = row_limit(it, n, p.G, p.causal);
  // every row of the wave's tile sees at least the keys below lim_min (its
  // first row is the most restricted; padding rows are never written)
  const int lim_min = row_limit(it, 16 * rt, p.G, p.causal);
  const bool qok = active && n < it.rows;
  {
    const int t = it.c0 + (qok ? n / p.G : 0);
    const int h = it.g * p.G + (qok ? n % p.G : 0);
    const uint16_t* qr = p.q + (static_cast<size_t>(t) * p.Hq + h) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 32 * kk + 8 * j4;
      dma16_lds<false>(qr + ch, qstage + kk * 1024);   // padding rows read row 0
    }
  }

  // ---- prologue: stages 0 .. NS-2 in flight ----
  int pid_next[R::kUnitsPerWave];
#pragma unroll
  for (int s = 0; s < kNS - 1; ++s) {
    if (s < nst) {
      int pids[R::kUnitsPerWave], subs[R::kUnitsPerWave];
      load_pids(s, pids);
      stage_subs(s, subs);
      issue_stage<E, SHUF, NRT, PSH>(p, it, pids, subs, ring + s * R::kStageBytes, wave, lane);
    }
  }
  if (kNS - 1 < nst) load_pids(kNS - 1, pid_next);
  // Q landed once at most the prologue's stages remain in flight; each wave
  // reads back its own pieces (written by its own DMA) before the first
  // barrier, after which the last stage is refilled
  wait_vmcnt_stages<R::kInstrPerWave, kNS - 1>(min(kNS - 1, nst));
  bf16x8_t qb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qb[kk] = *reinterpret_cast<const bf16x8_t*>(qstage + kk * 1024 + lane * 16);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (!qok) qb[kk] = as_bf16x8(make_uint4(0, 0, 0, 0));
    asm volatile("" : "+v"(qb[kk]));           // the reads complete here
  }

  f32x4_t oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  for (int i = 0; i < nst; ++i) {
    // stage i landed (own DMA), then everyone's; stage i-1 is free again
    {
      const int later = min(kNS - 2, nst - 1 - i);
      wait_vmcnt_stages<R::kInstrPerWave, kNS - 2>(later);
    }
    barrier_keep_loads();
    if (i + kNS - 1 < nst) {
      int subs[R::kUnitsPerWave];
      stage_subs(i + kNS - 1, subs);
      issue_stage<E, SHUF, NRT, PSH>(p, it, pid_next, subs,
                                ring + ((i + kNS - 1) % kNS) * R::kStageBytes, wave, lane);
      if (i + kNS < nst) load_pids(i + kNS, pid_next);
    }
    if (!active) continue;

    const uint8_t* slot = ring + (i % kNS) * R::kStageBytes;
    const int tok0 = it.seg_start + i * R::kStageTok + bis * 32;   // this wave's block
    if (tok0 >= it.seg_end) continue;
    const uint8_t* kU[2] = {slot + (2 * (2 * bis)) * R::kUnitBytes,
                            slot + (2 * (2 * bis + 1)) * R::kUnitBytes};
    const uint8_t* vU[2] = {kU[0] + R::kUnitBytes, kU[1] + R::kUnitBytes};

    // ---- S^T per page ----
    f32x4_t sacc[2];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      bf16x8_t kop[4];
      if constexpr (!SHUF) {
        // page tile at kU[pg]: chunk 4 kk + j4 of token row r16
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          kop[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(
              kU[pg] + r16 * R::kStdRow + std2_chunk_pos(r16, 4 * kk + j4) * 16));
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          kop[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kU[pg] + kk * 1024 + lane * 16));
      }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma_k32<F16>(kop[kk], qb[kk], acc);
      sacc[pg] = acc;
    }

    // ---- online softmax (row n = 16*rt + r16; 8 tokens per lane) ----
    // raw scores; the scale folds into the fma before exp2. The masks and
    // the rescale are wave-uniform branches (kept as branches, not selects:
    // most blocks take neither)
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = sacc[e >> 2][e & 3];
    if (tok0 + 32 > lim_min) {                     // some row does not see the whole block
      asm volatile("");
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = tok0 + 16 * (e >> 2) + 4 * j4 + (e & 3);
        s[e] = pos < lim ? s[e] : -INFINITY;
      }
    }
    float bm = s[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, s[e]);
    bm = bm == -INFINITY ? -INFINITY : bm * c;
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    const float mu = mn == -INFINITY ? 0.f : mn;
    if (__builtin_amdgcn_ballot_w64(mn != m) != 0) {     // some row max moved
      asm volatile("");
      const float alpha = fast_exp2(m - mu);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
      m = mn;
    }
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float a = fast_exp2(fmaf(s[e], c, -mu)), b = fast_exp2(fmaf(s[e + 1], c, -mu));
      l += a + b;
      pk[e >> 1] = pack2<F16>(a, b);
    }
    const bf16x8_t pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));

    // ---- O^T += V^T.P^T ; element e: page e/4, token 4*j4 + e%4 ----
    const int vend = it.seg_end - tok0;       // tokens of the block before the end
    // the V-tail zeroing is compiled into a second copy of the loop, taken
    // only by the block that crosses the segment end
    auto pv = [&](auto tail_tag) __attribute__((always_inline)) {
      constexpr bool tail = decltype(tail_tag)::value;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + r16;
      uint32_t w[4];
      if constexpr (SHUF) {
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          const uint2 v = *reinterpret_cast<const uint2*>(
              vU[pg] + ((j4 >> 1) * kD + d) * 16 + (j4 & 1) * 8);
          w[2 * pg] = v.x;
          w[2 * pg + 1] = v.y;
        }
      } else {
        // transposing LDS read: in each 16-lane group, lane i receives element
        // i%4 of the 8 bytes read by lane 4k + i/4 (k = 0..3). Lane j reads
        // token tau = 4*j4 + j/4, channels 16dt + 4(j%4) .. +3, i.e. half j%2
        // of V chunk 2dt + (j/2)%2 (row chunk 16 + that, swizzled), so lane i
        // ends up with tokens 4*j4 .. 4*j4+3 of channel 16dt + i.
        const int vtau = 4 * j4 + (r16 >> 2);
        const int vq = 16 + 2 * dt + ((r16 >> 1) & 1);
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(
                  (__attribute__((address_space(3))) uint8_t*)(kU[pg]) + vtau * R::kStdRow +
                  std2_chunk_pos(vtau, vq) * 16 + (r16 & 1) * 8));
          const uint2 u = __builtin_bit_cast(uint2, v);
          w[2 * pg] = u.x;
          w[2 * pg + 1] = u.y;
        }
      }
      if (tail) {                    // zero V of tokens past the segment end
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int rel = vend - (16 * (q2 >> 1) + 4 * j4 + 2 * (q2 & 1));
          w[q2] = rel <= 0 ? 0u : (rel == 1 ? (w[q2] & 0xffffu) : w[q2]);
        }
      }
      oacc[dt] = mfma_k32<F16>(as_bf16x8(make_uint4(w[0], w[1], w[2], w[3])), pb, oacc[dt]);
    }
    };
    if (tok0 + 32 > it.seg_end) {                   // wave-uniform
      asm volatile("");
      pv(std::true_type{});
    } else {
      pv(std::false_type{});
    }
  }

  // ---- row sums across the four lane groups ----
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  constexpr int kShare = kWaves / NRT;          // waves sharing a row tile
  float M = m, Ls = l;
  if constexpr (kShare > 1) {
    wait_vmcnt<0>();
    __syncthreads();                            // ring is dead; reuse it
    f32x4_t* oslot = reinterpret_cast<f32x4_t*>(ring);
    if (j4 == 0) {
      sm_m[wave][r16] = m;
      sm_l[wave][r16] = l;
    }
    if (bis > 0) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oslot[(wave * 8 + dt) * 64 + lane] = oacc[dt];
    }
    __syncthreads();
    if (bis > 0 || !active) return;
    M = -INFINITY;
#pragma unroll
    for (int b = 0; b < kShare; ++b) M = fmaxf(M, sm_m[rt + NRT * b][r16]);
    const float mu = M == -INFINITY ? 0.f : M;
    const float f0 = fast_exp2(m - mu);
    Ls = l * f0;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] *= f0;
#pragma unroll
    for (int b = 1; b < kShare; ++b) {
      const int w2 = rt + NRT * b;
      const float f = fast_exp2(sm_m[w2][r16] - mu);
      Ls += sm_l[w2][r16] * f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] += oslot[(w2 * 8 + dt) * 64 + lane] * f;
    }
    M = mu;
  } else {
    if (!active) return;
    M = m == -INFINITY ? 0.f : m;
  }

  // ---- write this row tile's partial ----
  if (n >= it.rows) return;
  const int t = it.c0 + n / p.G;
  const int h = it.g * p.G + n % p.G;
  const size_t prow = (static_cast<size_t>(t) * p.Hq + h) * p.seg_max + it.seg;
  const bool any = Ls > 0.f;
  const float inv = any ? out_scale / Ls : 0.f;
  float* po = p.part_o + prow * kD;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<f32x4_t*>(po + 16 * dt + 4 * j4) = oacc[dt] * inv;
  if (j4 == 0) p.part_lse[prow] = any ? (M + fast_log2(Ls)) * kLn2 : -INFINITY;
}

}  // namespace

template <bool F16, int PSH>
int launch_shared(const SegParams& sp, bool shuf, int grid, hipStream_t st) {
  if (shuf)
    hipLaunchKernelGGL((seg_mfma_kernel<2, true, 4, F16, PSH>), dim3(grid),
                       dim3(64 * Ring<2, 4>::kWaves), 0, st, sp);
  else
    hipLaunchKernelGGL((seg_mfma_kernel<2, false, 4, F16, PSH>), dim3(grid),
                       dim3(64 * Ring<2, 4>::kWaves), 0, st, sp);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

// bf16 or fp16 KV with 33-64 rows (four row tiles); the other cases run on the
// private-ring variants
int launch_segments_mfma(const SegParams& sp, bool shuf, bool f16, int grid, hipStream_t st) {
  if (sp.page_shift == 5)
    return f16 ? launch_shared<true, 5>(sp, shuf, grid, st) : launch_shared<false, 5>(sp, shuf, grid, st);
  return f16 ? launch_shared<true, 4>(sp, shuf, grid, st) : launch_shared<false, 4>(sp, shuf, grid, st);
}

}  // namespace skv
