// Segment attention for head dims 64 and 256 (the head-dim-128 kernels are
// specialised for that width). One work-group per (work item, kv head),
// computing the same partials as the other kernels:
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Modifications: each (sequence, segment) of the work
// list yields one partial (normalised o, log-sum-exp) per query row, merged
// later by the split reduce.
//
// Design:
//  * Two groups of four waves; in each group wave r owns query-row tile r (16
//    rows of G x max_q <= 64; waves past the row count only move data). The
//    groups take alternate 32-token blocks of a ring stage, or, where a stage
//    is one block (256-wide 16-bit rows), one 16-token sub-page of it each
//    (scores and P.V on 16 tokens, the latter on the 16x16x16 instruction).
//    Two waves share each SIMD and hide each other's latencies (three at head
//    dim 64, whose per-byte softmax work is twice that at 128: three groups,
//    six-block stages, a 144 KB ring for 16-bit rows); the groups' states are
//    merged through LDS at the end. A wave with two or more
//    blocks per stage takes two per step (64 tokens between row-max updates).
//  * KV streams through one 128 KB LDS ring shared by the waves, in four
//    32 KB stages of 32-token blocks, by direct-to-LDS DMA (16 bytes per
//    lane, 1 KB per instruction, whole cache lines, streaming policy). Each
//    wave waits on its own DMA count, then one barrier per stage makes every
//    wave's part visible and frees the slot computed one stage earlier.
//  * Standard pages are copied as their contiguous 16-row tiles; the 16-byte
//    chunks of each token row are XOR-swizzled by the row's index, so the 16
//    rows of one K operand read, and the transposing V reads, fall on
//    different LDS banks. Shuffled planes are copied as laid out: their K
//    chunk rows and V token groups already put one operand read's 16 lanes on
//    consecutive chunks.
//  * Scores S^T = K.Q^T and O^T += V^T.P^T on the 16x16x32 matrix
//    instructions (bf16 or fp16; fp8 e4m3fn KV widened exactly to bf16), the
//    online softmax in the exp2 domain as in the other kernels: masked scores
//    are -inf, V of tokens past the segment end is zeroed, so page-tail or
//    stale-LDS poison never reaches the accumulator.
//  * The softmax keeps the per-token work down (at head dim 64 it, not HBM,
//    bounds the kernel): the score scale folds into the fma before each
//    exp2 (a negative fp8 K scale is moved into Q's sign), blocks that every
//    row of the wave sees in full skip the masks, and the running row max
//    moves only when a step's scores rise 2^8 above it, so most steps need
//    no cross-lane max and no rescale.
#include <type_traits>

#include "skv_attn_common.h"
#include "skv.h"

namespace skv {
namespace {

typedef short v4i16_gd __attribute__((ext_vector_type(4)));
typedef int v2i32_gd __attribute__((ext_vector_type(2)));

constexpr int kGdRingBudget = 128 * 1024;
// the running row max lags the true one by less than this (log2 units):
// weights stay <= 2^8, which bf16 / fp16 P and the fp32 sums carry exactly
// enough (no loss of relative precision)
constexpr float kGdSlackLog2 = 8.f;

// 16-bit 1.0 in both halves of a word (bf16 or fp16): the V^T operand of the
// extra P.V tile that sums each row's rounded weights
template <bool F16>
constexpr uint32_t kOnes2 = F16 ? 0x3c003c00u : 0x3f803f80u;
constexpr int kGdStageTarget = 32 * 1024;

template <int D, int E>
struct GdRing {
  static constexpr int kX = 16 / E;                        // elements per 16 bytes
  static constexpr int kSubBytes = kPageSize * 2 * D * E;  // one 16-token sub-page, K and V
  static constexpr int kKBytes = kPageSize * D * E;        // its K part (shuffled planes)
  static constexpr int kBlkBytes = 2 * kSubBytes;          // one 32-token block
  // head dim 64: three wave groups, two blocks each per stage
  static constexpr bool kThree = D == 64;
  static constexpr int kBlocks = kThree ? 6
                               : (kGdStageTarget / kBlkBytes > 1 ? kGdStageTarget / kBlkBytes : 1);
  static constexpr int kStageBytes = kBlocks * kBlkBytes;
  static constexpr int kStageTok = 32 * kBlocks;
  static constexpr int kInstr = kStageBytes / 1024;        // DMA instructions per stage
  // two wave groups (two waves per SIMD): alternate blocks of a stage when
  // it holds two or more, else (one block: 256-wide 16-bit rows) one
  // 16-token sub-page of the block each
  static constexpr bool kSubSplit = kBlocks == 1;
  static_assert(!kSubSplit || E == 2, "one-block stages only for 16-bit elements");
  static constexpr int kGroups = kThree ? 3 : 2;
  static constexpr int kWaves = 4 * kGroups;
  static_assert(kSubBytes % 1024 == 0, "a DMA instruction stays in one sub-page");
  static_assert(kKBytes % 1024 == 0, "a DMA instruction stays in K or in V");
  static_assert(kInstr % kWaves == 0, "every wave issues the same count");
  static constexpr int kInstrPerWave = kInstr / kWaves;
  static constexpr int kNS0 = (kThree && E == 2 ? 144 * 1024 : kGdRingBudget) / kStageBytes;
  static constexpr int kNS = kNS0 > 8 ? 8 : kNS0;
  static_assert(kNS >= 3, "ring needs three stages");
  static_assert((kNS - 2) * kInstrPerWave <= 63, "vmcnt range");
  static constexpr int kRowBytes = 2 * D * E;              // one standard token row
  static constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per row
  static constexpr int kSwz = (kChunks < 16 ? kChunks : 16) - 1;
};

// position of chunk q of standard row tau in LDS (an involution per row)
template <int D, int E>
__device__ __forceinline__ int gd_chunk_pos(int tau, int q) {
  return q ^ (tau & GdRing<D, E>::kSwz);
}

template <int N>
__device__ __forceinline__ void gd_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most k stages' worth (k * STEP instructions) remain in flight
template <int STEP, int MAXK>
__device__ __forceinline__ void gd_wait_stages(int k) {
  if constexpr (MAXK >= 6) { if (k >= 6) { gd_wait_vmcnt<6 * STEP>(); return; } }
  if constexpr (MAXK >= 5) { if (k == 5) { gd_wait_vmcnt<5 * STEP>(); return; } }
  if constexpr (MAXK >= 4) { if (k == 4) { gd_wait_vmcnt<4 * STEP>(); return; } }
  if constexpr (MAXK >= 3) { if (k == 3) { gd_wait_vmcnt<3 * STEP>(); return; } }
  if constexpr (MAXK >= 2) { if (k == 2) { gd_wait_vmcnt<2 * STEP>(); return; } }
  if constexpr (MAXK >= 1) { if (k == 1) { gd_wait_vmcnt<1 * STEP>(); return; } }
  gd_wait_vmcnt<0>();
}

// HBM addresses of sub-page `sub` (16 tokens) of page `pid`, kv head g:
// standard: the tile of its 16 token rows (K then V channels per row);
// shuffled: its first token in K chunk row 0 (chunk rows `krow` bytes apart)
// and its V token groups (contiguous, as a 16-token page's V plane).
template <int D, int E, bool SHUF, int PSH>
__device__ __forceinline__ void gd_sub_page(const SegParams& p, int g, int pid, int sub,
                                            const uint8_t*& k, const uint8_t*& v) {
  using R = GdRing<D, E>;
  const size_t head = static_cast<size_t>(pid) * p.Hkv + g;
  if constexpr (SHUF) {
    const size_t plane = (head * R::kKBytes) << (PSH - 4);
    k = p.kv_a + plane + static_cast<size_t>(sub) * kPageSize * 16;
    v = p.kv_b + plane + static_cast<size_t>(sub) * R::kKBytes;
  } else {
    k = p.kv_a + ((head << (PSH - 4)) + sub) * R::kSubBytes;
    v = k;
  }
}

// Issue this wave's DMA instructions of stage `st` into `slot`. The stage's
// sub-page j (tokens 16j .. 16j + 15 of the stage) occupies
// [j * kSubBytes, (j + 1) * kSubBytes) of the slot. Sub-pages past the
// segment end re-read the segment's first sub-page (the instruction count
// stays fixed, so the vmcnt waits stay exact; their tokens are masked and
// their V zeroed).
template <int D, int E, bool SHUF, int PSH>
__device__ __forceinline__ void gd_issue_stage(const SegParams& p, const SegItem& it,
                                               const __attribute__((address_space(4))) int32_t* ptab,
                                               int st, uint8_t* slot, int wave, int lane) {
  using R = GdRing<D, E>;
  constexpr int psh = PSH - 4;
  const int seg_sub0 = it.seg_start >> 4;
  const int seg_subs = (it.seg_end - it.seg_start + 15) >> 4;
#pragma unroll
  for (int k = 0; k < R::kInstrPerWave; ++k) {
    const int i = wave * R::kInstrPerWave + k;            // instruction of the stage
    const int j = (i * 1024) / R::kSubBytes;              // its sub-page (uniform)
    const int w = (i * 1024) % R::kSubBytes + lane * 16;  // lane's byte in the sub-page
    const int vs = st * 2 * R::kBlocks + j;               // sub-page index in the segment
    const int sv = seg_sub0 + (vs < seg_subs ? vs : 0);
    const int pid = ptab[sv >> psh];
    const uint8_t *kb, *vb;
    gd_sub_page<D, E, SHUF, PSH>(p, it.g, pid, sv & ((1 << psh) - 1), kb, vb);
    const uint8_t* src;
    if constexpr (SHUF) {
      if ((i * 1024) % R::kSubBytes < R::kKBytes)         // uniform per instruction
        src = kb + static_cast<size_t>(w >> 8) * (16 << PSH) + (w & 255);
      else
        src = vb + (w - R::kKBytes);
    } else {
      const int tau = w / R::kRowBytes;
      const int pos = (w % R::kRowBytes) >> 4;
      src = kb + tau * R::kRowBytes + gd_chunk_pos<D, E>(tau, pos) * 16;
    }
    dma16_lds<true>(src, slot + i * 1024);
  }
}

template <int D, int E, bool SHUF, bool F16, int PSH>
__global__ __launch_bounds__((64 * GdRing<D, E>::kWaves))
__attribute__((amdgpu_waves_per_eu((GdRing<D, E>::kGroups), (GdRing<D, E>::kGroups))))
void seg_gd_kernel(SegParams p) {
  using R = GdRing<D, E>;
  constexpr int kNS = R::kNS;
  constexpr int kKS = D / 32;                      // k-steps of the score product
  constexpr int kDT = D / 16;                      // output channel tiles
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kNS * R::kStageBytes];

  const SegItem it = decode_item(p);
  write_fixed_counts(p, it);
  if (!it.valid) return;                                          // work-group uniform
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, j4 = lane >> 4;
  const int rt = wave & 3, grp = wave >> 2;                       // row tile, wave group
  const int nrt = (it.rows + 15) >> 4;
  const bool active = rt < nrt;                                   // wave-uniform
  const int ntok = it.seg_end - it.seg_start;
  const int nst = (ntok + R::kStageTok - 1) / R::kStageTok;
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(
          p.page_table + static_cast<size_t>(it.seq) * p.pt_stride);
  float sm_scale = kLog2e * (D == 64 ? 0.125f : 0.0625f);        // log2(e) / sqrt(D)
  float out_scale = 1.f;
  uint32_t qflip = 0u;
  if constexpr (E == 1) {
    // scores enter exp2 as fma(raw, c, -m) with c > 0: a negative K scale
    // is moved into Q's sign (exact), a zero one becomes the least normal
    const float ks = p.k_scale[0];
    sm_scale *= fabsf(ks);
    qflip = ks < 0.f ? 0x80008000u : 0u;
    out_scale = p.v_scale[0];
  }
  const float c = fmaxf(sm_scale, 1.17549435e-38f);
  const float inv_c = 1.f / c;

  // ---- Q of this wave's row tile (B operand: row r16, channels 32kk+8j4..+7)
  const int n = 16 * rt + r16;
  const int lim = row_limit(it, n, p.G, p.causal);
  // every row of the wave sees at least the keys below lim_min (its first
  // row is the most restricted; padding rows are never written)
  const int lim_min = row_limit(it, 16 * rt, p.G, p.causal);
  const bool qok = active && n < it.rows;
  bf16x8_t qb[kKS];
  {
    const int t = it.c0 + (qok ? n / p.G : 0);
    const int h = it.g * p.G + (qok ? n % p.G : 0);
    const uint16_t* qr = p.q + (static_cast<size_t>(t) * p.Hq + h) * D + 8 * j4;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk)
      qb[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 32 * kk));
    // the loads complete here, before any DMA is issued (padding rows: zero)
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      const uint4 v = __builtin_bit_cast(uint4, qb[kk]);
      qb[kk] = as_bf16x8(qok ? make_uint4(v.x ^ qflip, v.y ^ qflip, v.z ^ qflip, v.w ^ qflip)
                             : make_uint4(0, 0, 0, 0));
      asm volatile("" : "+v"(qb[kk]));
    }
  }

  // ---- prologue: stages 0 .. NS-2 in flight ----
#pragma unroll
  for (int s = 0; s < kNS - 1; ++s)
    if (s < nst)
      gd_issue_stage<D, E, SHUF, PSH>(p, it, ptab, s, ring + s * R::kStageBytes, wave, lane);

  f32x4_t oacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // m: running row max (log2 units, -inf before any visible key), the offset
  // of every exponential; thr: raw scores at or below it keep m. l sums the
  // fp32 weights (for the lse); lacc, an extra P.V tile whose V is all ones,
  // sums the 16-bit weights P.V actually applies (every element of the lane's
  // four holds row r16's sum), and O is normalised by it: the output is then a
  // convex combination of V rows with the applied weights, so a dominant
  // key's rounding cancels (under the lazy row max its weight is up to 2^8,
  // not exactly 1)
  float m = -INFINITY, l = 0.f, thr = -INFINITY;
  f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};
  auto update_max = [&](float lm) {
    if (__builtin_amdgcn_ballot_w64(lm > thr) != 0) {     // some row max must move
      asm volatile("");                   // a branch, not a select: most steps skip it
      float bm = lm == -INFINITY ? -INFINITY : lm * c;
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
      l *= alpha;
      lacc *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[dt] *= alpha;
      m = mn;
      thr = mn == -INFINITY ? -INFINITY : (mn + kGdSlackLog2) * inv_c;
    }
  };

  for (int i = 0; i < nst; ++i) {
    // stage i landed (own DMA), then everyone's; stage i-1's slot is free
    gd_wait_stages<R::kInstrPerWave, kNS - 2>(min(kNS - 2, nst - 1 - i));
    asm volatile("s_barrier" ::: "memory");
    if (i + kNS - 1 < nst)
      gd_issue_stage<D, E, SHUF, PSH>(p, it, ptab, i + kNS - 1,
                                      ring + ((i + kNS - 1) % kNS) * R::kStageBytes, wave, lane);
    if (!active) continue;
    const uint8_t* slot = ring + (i % kNS) * R::kStageBytes;

    if constexpr (R::kSubSplit) {
      // ---- this group's sub-page of the stage's block: 16 tokens ----
      const int tok0 = it.seg_start + i * R::kStageTok + 16 * grp;
      if (tok0 >= it.seg_end) continue;
      const uint8_t* sp = slot + grp * R::kSubBytes;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
        bf16x8_t kop;
        if constexpr (SHUF)
          kop = as_bf16x8(*reinterpret_cast<const uint4*>(sp + (4 * kk + j4) * 256 + r16 * 16));
        else
          kop = as_bf16x8(*reinterpret_cast<const uint4*>(
              sp + r16 * R::kRowBytes + gd_chunk_pos<D, E>(r16, 4 * kk + j4) * 16));
        acc = mfma_k32<F16>(kop, qb[kk], acc);
      }
      float s4[4];
      float lm = -INFINITY;
      const bool masked = tok0 + 16 > lim_min;                    // wave-uniform
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s4[e] = acc[e];
        if (masked) s4[e] = tok0 + 4 * j4 + e < lim ? s4[e] : -INFINITY;
        lm = fmaxf(lm, s4[e]);
      }
      update_max(lm);
      const float mu = m == -INFINITY ? 0.f : m;
      const float p0 = fast_exp2(fmaf(s4[0], c, -mu)), p1 = fast_exp2(fmaf(s4[1], c, -mu));
      const float p2 = fast_exp2(fmaf(s4[2], c, -mu)), p3 = fast_exp2(fmaf(s4[3], c, -mu));
      l += (p0 + p1) + (p2 + p3);
      const i16x4_t pb4 = __builtin_bit_cast(i16x4_t, make_uint2(pack2<F16>(p0, p1), pack2<F16>(p2, p3)));
      lacc = mfma_k16<F16>(__builtin_bit_cast(i16x4_t, make_uint2(kOnes2<F16>, kOnes2<F16>)), pb4,
                           lacc);
      // tokens 4j4 .. 4j4+3 of the sub-page; those past the segment end zeroed
      const int vend = it.seg_end - tok0 - 4 * j4;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        uint2 u;
        if constexpr (SHUF) {
          u = *reinterpret_cast<const uint2*>(
              sp + R::kKBytes + ((j4 >> 1) * D + 16 * dt + r16) * 16 + (j4 & 1) * 8);
        } else {
          // the transposing read of the two-sub-page form, for one sub-page
          const int tau = 4 * j4 + (r16 >> 2);
          const int q = D / 8 + 2 * dt + ((r16 >> 1) & 1);
          const v4i16_gd v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_gd*)(
                  (__attribute__((address_space(3))) uint8_t*)(sp) + tau * R::kRowBytes +
                  gd_chunk_pos<D, E>(tau, q) * 16 + (r16 & 1) * 8));
          u = __builtin_bit_cast(uint2, v);
        }
        if (vend < 4) {
          u.x = vend <= 0 ? 0u : (vend == 1 ? (u.x & 0xffffu) : u.x);
          u.y = vend <= 2 ? 0u : (vend == 3 ? (u.y & 0xffffu) : u.y);
        }
        oacc[dt] = mfma_k16<F16>(__builtin_bit_cast(i16x4_t, u), pb4, oacc[dt]);
      }
      continue;
    }

    // NJ of this group's blocks at once (a 64-token step when the stage
    // holds four or more blocks): twice the independent work between the
    // dependent steps (scores, row max across lanes, exponentials, P.V), and
    // one row-max update per 64 tokens
    constexpr int NJ = R::kBlocks >= 2 * R::kGroups ? 2 : 1;
    for (int b0 = grp; b0 < R::kBlocks; b0 += NJ * R::kGroups) {
      int tokb[NJ];
      const uint8_t* sub[NJ][2];
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        const int b = b0 + jb * R::kGroups;
        tokb[jb] = it.seg_start + i * R::kStageTok + 32 * b;
        sub[jb][0] = slot + (2 * b) * R::kSubBytes;
        sub[jb][1] = slot + (2 * b + 1) * R::kSubBytes;
      }
      if (tokb[0] >= it.seg_end) break;

      // ---- S^T per sub-page: lane holds tokens 4j4..4j4+3 of row r16 ----
      f32x4_t sacc[NJ][2];
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          const uint8_t* sp = sub[jb][pg];
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < kKS; ++kk) {
            bf16x8_t kop;
            if constexpr (SHUF && E == 2) {
              kop = as_bf16x8(*reinterpret_cast<const uint4*>(sp + (4 * kk + j4) * 256 + r16 * 16));
            } else if constexpr (SHUF) {
              const uint2 c = *reinterpret_cast<const uint2*>(
                  sp + (2 * kk + (j4 >> 1)) * 256 + r16 * 16 + (j4 & 1) * 8);
              kop = as_bf16x8(fp8x8_to_bf16x8(c));
            } else if constexpr (E == 2) {
              kop = as_bf16x8(*reinterpret_cast<const uint4*>(
                  sp + r16 * R::kRowBytes + gd_chunk_pos<D, E>(r16, 4 * kk + j4) * 16));
            } else {
              const uint2 c = *reinterpret_cast<const uint2*>(
                  sp + r16 * R::kRowBytes +
                  gd_chunk_pos<D, E>(r16, 2 * kk + (j4 >> 1)) * 16 + (j4 & 1) * 8);
              kop = as_bf16x8(fp8x8_to_bf16x8(c));
            }
            acc = mfma_k32<F16>(kop, qb[kk], acc);
          }
          sacc[jb][pg] = acc;
        }
      }

      // ---- online softmax (row n; 8 NJ tokens per lane) ----
      float s[NJ][8];
      float lm = -INFINITY;
      // blocks past the end of this group's last valid block hold tokens
      // beyond the segment end, which lim (<= the segment end) masks
      const bool masked = tokb[NJ - 1] + 32 > lim_min;            // wave-uniform
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s[jb][e] = sacc[jb][e >> 2][e & 3];
        }
      }
      if (masked) {
        asm volatile("");                 // a branch, not a select: most steps skip it
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int pos = tokb[jb] + 16 * (e >> 2) + 4 * j4 + (e & 3);
            s[jb][e] = pos < lim ? s[jb][e] : -INFINITY;
          }
        }
      }
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) lm = fmaxf(lm, s[jb][e]);
      }
      update_max(lm);
      const float mu = m == -INFINITY ? 0.f : m;
      bf16x8_t pb[NJ];
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float a = fast_exp2(fmaf(s[jb][e], c, -mu));
          const float b = fast_exp2(fmaf(s[jb][e + 1], c, -mu));
          pk[e >> 1] = pack2<F16>(a, b);
          l += a + b;
        }
        pb[jb] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
        lacc = mfma_k32<F16>(as_bf16x8(make_uint4(kOnes2<F16>, kOnes2<F16>, kOnes2<F16>,
                                                  kOnes2<F16>)),
                             pb[jb], lacc);
      }

      // ---- O^T += V^T.P^T; element e: sub-page e/4, token 4j4 + e%4. The
      // V-tail zeroing is compiled into a second copy of the loop, taken only
      // by the step that holds tokens past the segment end ----
      auto pv = [&](auto tail_tag) __attribute__((always_inline)) {
        constexpr bool kTail = decltype(tail_tag)::value;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const int d = 16 * dt + r16;
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
          uint32_t w[4];
          if constexpr (SHUF && E == 2) {
#pragma unroll
            for (int pg = 0; pg < 2; ++pg) {
              const uint2 v = *reinterpret_cast<const uint2*>(
                  sub[jb][pg] + R::kKBytes + ((j4 >> 1) * D + d) * 16 + (j4 & 1) * 8);
              w[2 * pg] = v.x;
              w[2 * pg + 1] = v.y;
            }
          } else if constexpr (SHUF) {
            const uint32_t a =
                *reinterpret_cast<const uint32_t*>(sub[jb][0] + R::kKBytes + d * 16 + 4 * j4);
            const uint32_t c =
                *reinterpret_cast<const uint32_t*>(sub[jb][1] + R::kKBytes + d * 16 + 4 * j4);
            const uint4 x = fp8x8_to_bf16x8(make_uint2(a, c));
            w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
          } else if constexpr (E == 2) {
            // transposing read: in each 16-lane group, lane i receives element
            // i%4 of the 8 bytes read by lane 4k + i/4 (k = 0..3). Lane j reads
            // token 4j4 + j/4, V channels 16dt + 4(j%4) .. +3, so lane i ends
            // up with tokens 4j4 .. 4j4+3 of channel 16dt + i.
            const int tau = 4 * j4 + (r16 >> 2);
            const int q = D / 8 + 2 * dt + ((r16 >> 1) & 1);
#pragma unroll
            for (int pg = 0; pg < 2; ++pg) {
              const v4i16_gd v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) v4i16_gd*)(
                      (__attribute__((address_space(3))) uint8_t*)(sub[jb][pg]) +
                      tau * R::kRowBytes + gd_chunk_pos<D, E>(tau, q) * 16 + (r16 & 1) * 8));
              const uint2 u = __builtin_bit_cast(uint2, v);
              w[2 * pg] = u.x;
              w[2 * pg + 1] = u.y;
            }
          } else {
            // transposing byte read: in each 16-lane group, lane i receives
            // byte i%8 of the 8 bytes read by lane 2k + i/8 (k = 0..7). Lane j
            // reads sub-page j/8, token 4j4 + (j/2)%4, V channels 16dt + 8(j%2)
            // .. +7, so lane i ends up with the block's 8 tokens of channel
            // 16dt + i.
            const int tau = 4 * j4 + ((r16 >> 1) & 3);
            const int q = D / 16 + dt;
            const v2i32_gd v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i32_gd*)(
                    (__attribute__((address_space(3))) uint8_t*)(sub[jb][r16 >> 3]) +
                    tau * R::kRowBytes + gd_chunk_pos<D, E>(tau, q) * 16 + (r16 & 1) * 8));
            const uint4 x = fp8x8_to_bf16x8(__builtin_bit_cast(uint2, v));
            w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
          }
          const int vend = it.seg_end - tokb[jb];
          if (kTail && vend < 32) {      // zero V of tokens past the segment end
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
              const int rel = vend - (16 * (q2 >> 1) + 4 * j4 + 2 * (q2 & 1));
              w[q2] = rel <= 0 ? 0u : (rel == 1 ? (w[q2] & 0xffffu) : w[q2]);
            }
          }
          oacc[dt] = mfma_k32<F16>(as_bf16x8(make_uint4(w[0], w[1], w[2], w[3])), pb[jb], oacc[dt]);
        }
      }
      };
      if (tokb[NJ - 1] + 32 > it.seg_end) {                       // wave-uniform
        asm volatile("");
        pv(std::true_type{});
      } else {
        pv(std::false_type{});
      }
    }
  }
  gd_wait_vmcnt<0>();                 // no DMA outlives the work-group

  // ---- row sums across the four lane groups ----
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  float M = m, Ls = l, Lr = lacc[0];
  {
    // groups 1 .. G-1 hand their (m, l, O^T) to group 0 through the (now
    // idle) ring; slot k - 1 for group k
    constexpr int kG = R::kGroups;
    constexpr int kOBytes = (kG - 1) * 4 * (kDT + 1) * 1024;   // O^T tiles and lacc
    static_assert(kOBytes + 2 * (kG - 1) * 4 * 16 * 4 <= kNS * R::kStageBytes, "merge fits");
    f32x4_t* oslot = reinterpret_cast<f32x4_t*>(ring);
    float(*sm_m)[16] = reinterpret_cast<float(*)[16]>(ring + kOBytes);
    float(*sm_l)[16] = reinterpret_cast<float(*)[16]>(ring + kOBytes + (kG - 1) * 4 * 16 * 4);
    __syncthreads();
    if (grp > 0 && active) {
      const int slot_k = (grp - 1) * 4 + rt;
      if (j4 == 0) {
        sm_m[slot_k][r16] = m;
        sm_l[slot_k][r16] = l;
      }
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oslot[(slot_k * (kDT + 1) + dt) * 64 + lane] = oacc[dt];
      oslot[(slot_k * (kDT + 1) + kDT) * 64 + lane] = lacc;
    }
    __syncthreads();
    if (grp > 0 || !active) return;
    float mx = m;
#pragma unroll
    for (int k = 1; k < kG; ++k) mx = fmaxf(mx, sm_m[(k - 1) * 4 + rt][r16]);
    const float mu = mx == -INFINITY ? 0.f : mx;
    const float f0 = fast_exp2(m - mu);
    Ls = l * f0;
    Lr = lacc[0] * f0;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) oacc[dt] *= f0;
#pragma unroll
    for (int k = 1; k < kG; ++k) {
      const int slot_k = (k - 1) * 4 + rt;
      const float f = fast_exp2(sm_m[slot_k][r16] - mu);
      Ls += sm_l[slot_k][r16] * f;
      Lr += oslot[(slot_k * (kDT + 1) + kDT) * 64 + lane][0] * f;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
        oacc[dt] += oslot[(slot_k * (kDT + 1) + dt) * 64 + lane] * f;
    }
    M = mu;
  }

  // ---- write the partial ----
  if (n >= it.rows) return;
  const int t = it.c0 + n / p.G;
  const int h = it.g * p.G + n % p.G;
  const size_t prow = (static_cast<size_t>(t) * p.Hq + h) * p.seg_max + it.seg;
  const bool any = Ls > 0.f;
  const float inv = any ? out_scale / Lr : 0.f;
  float* po = p.part_o + prow * D;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
    *reinterpret_cast<f32x4_t*>(po + 16 * dt + 4 * j4) = oacc[dt] * inv;
  if (j4 == 0) p.part_lse[prow] = any ? (M + fast_log2(Ls)) * kLn2 : -INFINITY;
}

template <int D, int E, bool F16, int PSH>
int launch_gd_t(const SegParams& sp, bool shuf, int grid, hipStream_t st) {
  if (shuf)
    hipLaunchKernelGGL((seg_gd_kernel<D, E, true, F16, PSH>), dim3(grid),
                       dim3(64 * GdRing<D, E>::kWaves), 0, st, sp);
  else
    hipLaunchKernelGGL((seg_gd_kernel<D, E, false, F16, PSH>), dim3(grid),
                       dim3(64 * GdRing<D, E>::kWaves), 0, st, sp);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

template <int D, int PSH>
int launch_gd_d(const SegParams& sp, int e, bool f16, bool shuf, int grid, hipStream_t st) {
  if (e == 1) return launch_gd_t<D, 1, false, PSH>(sp, shuf, grid, st);
  return f16 ? launch_gd_t<D, 2, true, PSH>(sp, shuf, grid, st)
             : launch_gd_t<D, 2, false, PSH>(sp, shuf, grid, st);
}

template <int PSH>
int launch_gd_p(const SegParams& sp, int d, int e, bool f16, bool shuf, int grid, hipStream_t st) {
  if (d == 64) return launch_gd_d<64, PSH>(sp, e, f16, shuf, grid, st);
  if (d == 256) return launch_gd_d<256, PSH>(sp, e, f16, shuf, grid, st);
  return SKV_EUNSUPPORTED;
}

}  // namespace

// head dims 64 and 256, every element type, layout and page size
int launch_segments_gd(const SegParams& sp, int head_dim, int e, bool f16, bool shuf, int grid,
                       hipStream_t st) {
  if (sp.page_shift == 5) return launch_gd_p<5>(sp, head_dim, e, f16, shuf, grid, st);
  return launch_gd_p<4>(sp, head_dim, e, f16, shuf, grid, st);
}

}  // namespace skv
