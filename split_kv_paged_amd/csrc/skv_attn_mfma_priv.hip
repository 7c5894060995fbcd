// Segment attention, matrix-core variants with private per-wave rings: fp8 KV
// (32-token block slots) and bf16 or fp16 KV with up to 32 rows (16-token page
// slots);
// query rows = GQA group x query tokens, padded to 16-row tiles.
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Motivation and Modifications: one work-group per
// (segment, sequence, kv head) computes softmax(q.K^T/sqrt(d)).V of all the
// sequence's query rows for that kv head over the segment's pages and writes a
// per-segment partial; the work-group decodes (seq, seg) from the work list.
//
// MI355X design. With a skewed batch the plan leaves only some CUs streaming
// the longest segments, so what one work-group can pull through a CU sets the
// layer time. A shared ring with a barrier per stage runs every wave through
// the same serial chain (wait, LDS, widen, MFMA, softmax, MFMA) in lockstep;
// a bare DMA ring of the same depth streams about twice as fast. Here:
//  * Each of NW waves streams 32-token blocks of the segment (fp8: wave w
//    starts with block w and then claims the next unclaimed block from an LDS
//    counter, or takes w + NW, w + 2 NW, ... in the deterministic order; 16-bit
//    KV: pages w, w + NW, ...) through a private LDS ring of NP slots (direct-
//    to-LDS DMA issued from inline asm, waits on its own vmcnt only): no
//    barrier in the main loop, so the waves drift apart and one wave's MFMA or
//    VALU work overlaps another's waits.
//  * A wave computes every 16-row query tile (NRT of them) of its block, so
//    each K and V element is widened from fp8 once (v_cvt_scalef32_pk_bf16_fp8,
//    exact) and read from LDS once.
//  * Block layout in LDS as in the shared-ring variant: K chunk-major per page
//    (operand lanes read contiguous 16-byte chunks), V chunk-major for the
//    transposing byte read (ds_read_b64_tr_b8), or the shuffled V plane as is.
//  * Scores transposed per page, S^T = K.Q^T, with v_mfma_f32_16x16x32_bf16;
//    online softmax in the exp2 domain per tile (the scale folded into one fma
//    before exp2). The running row max moves only when a block's scores rise
//    2^8 above it, so most blocks need no cross-lane max and no rescale; blocks
//    that every row sees in full skip the masks. Masked scores are -inf and V
//    past the segment end is zeroed (page-tail poison never leaks).
//  * fp8 with four row tiles (64 rows) keeps two waves per SIMD by reading Q
//    from LDS instead of holding it in registers.
//  * The first block is issued before Q is loaded, so the two latencies
//    overlap. At the end the waves' (max, sum, O) are merged through LDS,
//    wave w merging channel tile w of every row tile.
#include <type_traits>

#include "skv_attn_common.h"
#include "skv.h"

namespace skv {
namespace {

constexpr int kD = kHeadDim;
constexpr int kE = 1;                                   // fp8 elements
constexpr int kUnitBytes = kPageSize * kD * kE;         // one page's K (or V) half
constexpr int kUnitInstr = kUnitBytes / 1024;           // DMA instructions per unit
constexpr int kBlockBytes = 4 * kUnitBytes;             // 2 pages x (K, V)
constexpr int kBlockInstr = 4 * kUnitInstr;
constexpr int kStdTile = kPageSize * 2 * kD * kE;       // standard (block, head)
constexpr int kStdRow = 2 * kD * kE;
typedef int v2i32_t __attribute__((ext_vector_type(2)));

template <int NW, int NRT>
struct PRing {
  static constexpr int kBytes = 128 * 1024 / NW;        // one wave's ring
  static constexpr int kNP = kBytes / kBlockBytes;      // block slots
  static_assert(kNP >= 2, "two block slots per wave");
  static_assert((kNP - 1) * kBlockInstr <= 63, "vmcnt range");
};

template <int N>
__device__ __forceinline__ void pwait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int STEP, int MAXK>
__device__ __forceinline__ void pwait_blocks(int k) {
  // wait until at most k blocks' worth (k * STEP instructions) remain in flight
  if constexpr (MAXK >= 6) { if (k >= 6) { pwait_vmcnt<6 * STEP>(); return; } }
  if constexpr (MAXK >= 5) { if (k == 5) { pwait_vmcnt<5 * STEP>(); return; } }
  if constexpr (MAXK >= 4) { if (k == 4) { pwait_vmcnt<4 * STEP>(); return; } }
  if constexpr (MAXK >= 3) { if (k == 3) { pwait_vmcnt<3 * STEP>(); return; } }
  if constexpr (MAXK >= 2) { if (k == 2) { pwait_vmcnt<2 * STEP>(); return; } }
  if constexpr (MAXK >= 1) { if (k == 1) { pwait_vmcnt<1 * STEP>(); return; } }
  pwait_vmcnt<0>();
}

// Standard pages in a slot: page pg's (block, head) tile is copied whole, 16
// token rows of 256 B (K 128 B, then V 128 B), each DMA instruction taking 4
// consecutive rows, i.e. 1 KB of contiguous HBM. Within a row the sixteen
// 16-byte chunks are stored XOR-swizzled by token and page, so the K operand
// reads (16 tokens of one chunk) and the transposing V reads (4 tokens of two
// pages) spread over all LDS banks.
__device__ __forceinline__ int std_chunk_pos(int tau, int q, int pg) {
  return q ^ tau ^ (pg << 3);
}

// One 32-token block (pages pid0, pid1) into a slot. Standard pages: page pg
// at slot + pg * 4 KB as above. Shuffled planes: unit u = (page u/2, K if u
// even, V if odd) at slot + u * kUnitBytes, the K plane's 16-token chunk rows
// and the V plane copied as they are.
template <bool SHUF, int PSH>
__device__ __forceinline__ void issue_block(const SegParams& p, const SegItem& it, int pid0,
                                            int sub0, int pid1, int sub1, uint8_t* slot,
                                            int lane) {
  const int r16 = lane & 15, j4 = lane >> 4;
  const SubPageAddr sp[2] = {sub_page<kE, SHUF, PSH>(p, it.g, pid0, sub0),
                             sub_page<kE, SHUF, PSH>(p, it.g, pid1, sub1)};
  if constexpr (!SHUF) {
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const uint8_t* tile = sp[pg].k;
#pragma unroll
      for (int i = 0; i < kStdTile / 1024; ++i) {
        const int row = 4 * i + j4;                               // lane -> (row, position r16)
        const int q = std_chunk_pos(row, r16, pg);                // the chunk stored there
        dma16_lds_s<true>(tile, row * kStdRow + q * 16, slot + pg * kStdTile + i * 1024);
      }
    }
    return;
  }
  const int krow = kplane_row_bytes<PSH>();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint8_t* dst = slot + u * kUnitBytes;
    if ((u & 1) == 0) {
#pragma unroll
      for (int i = 0; i < kUnitInstr; ++i)
        dma16_lds_s<true>(sp[u >> 1].k, (4 * i + j4) * krow + r16 * 16, dst + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < kUnitInstr; ++i)    // the sub-page's V plane as is
        dma16_lds_s<true>(sp[u >> 1].v, (i * 64 + lane) * 16, dst + i * 1024);
    }
  }
}

// The NW = 8 waves' partial states of each 16-row tile (row max m, row sum l
// and O^T, each relative to the wave's own max) are merged through LDS and the
// segment partial is written. The idle rings hold the O^T tiles, as many row
// tiles per round as fit (rounds are separated by barriers); in each round
// wave w merges channel tile w of every row tile, reading the eight waves'
// 16-byte pieces and the row statistics (stored wave-minor, rows padded to
// 48 bytes so that the 16 rows' 16-byte reads fall in disjoint LDS banks: two
// reads per row) with all loads in flight at once.
template <int NW, int NRT, int SCRATCH>
__device__ __forceinline__ void merge_and_write(const SegParams& p, const SegItem& it,
                                                uint8_t* scratch, float (*sm_m)[16][NW + 4],
                                                float (*sm_l)[16][NW + 4],
                                                f32x4_t (&oacc)[NRT][8], float (&m)[NRT],
                                                float (&l)[NRT], float out_scale, int wave,
                                                int lane) {
  static_assert(NW == 8, "wave w merges channel tile w");
  constexpr int kTileBytes = NW * 8 * 64 * 16;          // one row tile's O^T of every wave
  constexpr int kTpr = SCRATCH / kTileBytes;             // row tiles per round
  static_assert(kTpr >= 1, "a row tile's merge scratch fits");
  const int r16 = lane & 15, j4 = lane >> 4;
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    l[t] += __shfl_xor(l[t], 16);
    l[t] += __shfl_xor(l[t], 32);
  }
  if (j4 == 0) {
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      sm_m[t][r16][wave] = m[t];
      sm_l[t][r16][wave] = l[t];
    }
  }
  f32x4_t* oslot = reinterpret_cast<f32x4_t*>(scratch);   // [tile in round][w][dt][lane]
#pragma unroll
  for (int t0 = 0; t0 < NRT; t0 += kTpr) {
    __syncthreads();                 // rings idle / previous round's reads done
#pragma unroll
    for (int tt = 0; tt < kTpr; ++tt)
      if (t0 + tt < NRT) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          oslot[((tt * NW + wave) * 8 + dt) * 64 + lane] = oacc[t0 + tt][dt];
      }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < kTpr; ++tt) {
      const int t = t0 + tt;
      if (t >= NRT) break;
      const float4 ma = *reinterpret_cast<const float4*>(&sm_m[t][r16][0]);
      const float4 mb = *reinterpret_cast<const float4*>(&sm_m[t][r16][4]);
      const float4 la = *reinterpret_cast<const float4*>(&sm_l[t][r16][0]);
      const float4 lb = *reinterpret_cast<const float4*>(&sm_l[t][r16][4]);
      f32x4_t ow[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) ow[w] = oslot[((tt * NW + w) * 8 + wave) * 64 + lane];
      const float mw[NW] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
      const float lw[NW] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
      float M = mw[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, mw[w]);
      const float mu = M == -INFINITY ? 0.f : M;
      float Ls = 0.f;
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(mw[w] - mu);
        Ls += lw[w] * f;
        o += ow[w] * f;
      }
      const int n = it.row0 + 16 * t + r16;
      if (n < it.rows) {
        const int tq = it.c0 + n / p.G;
        const int h = it.g * p.G + n % p.G;
        const size_t prow = (static_cast<size_t>(tq) * p.Hq + h) * p.seg_max + it.seg;
        const bool any = Ls > 0.f;
        const float inv = any ? out_scale / Ls : 0.f;
        *reinterpret_cast<f32x4_t*>(p.part_o + prow * kD + 16 * wave + 4 * j4) = o * inv;
        if (wave == 0 && j4 == 0)
          p.part_lse[prow] = any ? (mu + fast_log2(Ls)) * kLn2 : -INFINITY;
      }
    }
  }
}

// Online softmax of a private-ring wave, per 16-row tile and lane (row
// 16t + r16): m is the running row max in the log2 domain (-inf before any
// visible key) and the offset every exponential of the row uses (0 while m is
// -inf). A block whose raw scores all stay below thr = (m + kSlackLog2) / c
// keeps m: its weights are then at most 2^kSlackLog2, which bf16 and the fp32
// sums carry without loss of relative precision, so the row max is exchanged
// across lanes (and O rescaled) only when some row's scores rise that far.
constexpr float kSlackLog2 = 8.f;

template <bool SHUF, int NRT, int NW, int PSH>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void seg_mfma_priv_kernel(SegParams p) {
  using R = PRing<NW, NRT>;
  constexpr int kNP = R::kNP;
  // four row tiles at two waves per SIMD: Q is read from LDS, not held in registers
  constexpr bool kQLds = NRT >= 4;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NW][R::kBytes];
  __shared__ __attribute__((aligned(16))) float sm_m[NRT][16][NW + 4];
  __shared__ __attribute__((aligned(16))) float sm_l[NRT][16][NW + 4];
  __shared__ uint4 qs[kQLds ? NRT * 4 * 64 : 1];
  __shared__ int next_blk;                   // next_unit's counter
  static_assert(kNP == 2, "one block in flight while another is computed");

  const SegItem it = decode_item(p);
  write_fixed_counts(p, it);
  if (!it.valid) return;                                          // work-group uniform
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, j4 = lane >> 4;
  const int ntok = it.seg_end - it.seg_start;
  const int nblk = (ntok + 31) >> 5;
  const int seg_pages = (ntok + 15) >> 4;
  const int seg_page0 = it.seg_start >> 4;          // first 16-token sub-page
  constexpr int psh = PSH - 4;
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(
          p.page_table + static_cast<size_t>(it.seq) * p.pt_stride);
  // scores enter exp2 as fma(raw, c, -m) with c > 0: a negative K scale is
  // moved into Q's sign (exact), a zero one becomes the least normal float
  const float ks = p.k_scale[0];
  const float c = fmaxf(fabsf(ks) * kScoreScaleLog2, 1.17549435e-38f);
  const float inv_c = 1.f / c;
  const uint32_t qflip = ks < 0.f ? 0x80008000u : 0u;
  const float out_scale = p.v_scale[0];
  // every row sees at least the keys below lim_min (the first row is the most
  // restricted)
  const int lim_min = row_limit(it, it.row0, p.G, p.causal);

  uint8_t* wring = ring[wave];
  // pages of block bi of the segment; pages past the end read the segment's
  // first page (masked and zeroed; keeps vmcnt exact)
  auto pids = [&](int bi, int& a, int& sa, int& b, int& sb) {
    const int pg = 2 * bi;
    const int va = seg_page0 + (pg < seg_pages ? pg : 0);
    const int vb = seg_page0 + (pg + 1 < seg_pages ? pg + 1 : 0);
    a = ptab[va >> psh];
    b = ptab[vb >> psh];
    sa = sub_of<PSH>(va);
    sb = sub_of<PSH>(vb);
  };
  // the first block is issued before Q is loaded, so the two latencies
  // overlap (the first wait for Q also waits for this DMA; nothing else
  // is in flight yet)
  int cur = wave;                              // this wave's block (next_unit order)
  if (cur < nblk) {
    int a, sa, b, sb;
    pids(cur, a, sa, b, sb);
    issue_block<SHUF, PSH>(p, it, a, sa, b, sb, wring, lane);
  }

  // ---- Q rows of every tile (B operand of S^T = K.Q^T) ----
  auto load_q = [&](int t, int kk) -> uint4 {
    const int n = it.row0 + 16 * t + r16;
    const bool ok = n < it.rows;
    const int tq = it.c0 + (ok ? n / p.G : 0);
    const int h = it.g * p.G + (ok ? n % p.G : 0);
    const uint16_t* qr = p.q + (static_cast<size_t>(tq) * p.Hq + h) * kD;
    const int ch = 64 * (kk >> 1) + 16 * j4 + 8 * (kk & 1);
    return *reinterpret_cast<const uint4*>(qr + ch);             // padding rows read row 0
  };
  auto fix_q = [&](int t, uint4 v) -> uint4 {
    if (it.row0 + 16 * t + r16 >= it.rows) return make_uint4(0, 0, 0, 0);
    return make_uint4(v.x ^ qflip, v.y ^ qflip, v.z ^ qflip, v.w ^ qflip);
  };
  bf16x8_t qb[kQLds ? 1 : NRT][4];
  if constexpr (kQLds) {
    // this wave's pieces i = wave + NW k: every load in flight before one wait
    constexpr int kQPer = (NRT * 4 + NW - 1) / NW;
    uint4 qv[kQPer];
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = wave + NW * k;
      if (i < NRT * 4) qv[k] = load_q(i >> 2, i & 3);
    }
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = wave + NW * k;
      if (i < NRT * 4) qs[i * 64 + lane] = fix_q(i >> 2, qv[k]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < NRT; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[t][kk] = as_bf16x8(load_q(t, kk));
    // consume Q here, while only the first block is in flight (a later wait
    // for it would drain the ring)
#pragma unroll
    for (int t = 0; t < NRT; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        asm volatile("" : "+v"(qb[t][kk]));
        qb[t][kk] = as_bf16x8(fix_q(t, __builtin_bit_cast(uint4, qb[t][kk])));
      }
  }
  if (threadIdx.x == 0) next_blk = NW;
  __syncthreads();                             // Q staged, the claim counter set
  int lim[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) lim[t] = row_limit(it, it.row0 + 16 * t + r16, p.G, p.causal);

  f32x4_t oacc[NRT][8];
  float m[NRT], thr[NRT], l[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    m[t] = -INFINITY;
    thr[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // token of the transposing V reads: in each 16-lane group, lane i receives
  // byte i%8 of the 8 bytes read by lane 2k + i/8, i.e. 8 tokens of one channel
  const int vtau = 4 * j4 + ((r16 >> 1) & 3);

  // the loop runs two steps per turn, one per ring slot, so each slot's LDS
  // offsets are compile-time constants (folded into the reads' offsets)
  auto step = [&](auto slot_index) __attribute__((always_inline)) {
    constexpr int SI = decltype(slot_index)::value;
    const int nxt = next_unit<NW>(p, cur, &next_blk, lane);
    if (nxt < nblk) {                           // into the slot consumed last iteration
      int a, sa, b, sb;
      pids(nxt, a, sa, b, sb);
      issue_block<SHUF, PSH>(p, it, a, sa, b, sb, wring + (SI ^ 1) * kBlockBytes, lane);
      pwait_vmcnt<kBlockInstr>();               // block cur landed
    } else {
      pwait_vmcnt<0>();
    }
    const uint8_t* slot = wring + SI * kBlockBytes;
    const uint8_t* kU[2] = {slot, slot + 2 * kUnitBytes};
    const uint8_t* vU[2] = {slot + kUnitBytes, slot + 3 * kUnitBytes};
    const int tok0 = it.seg_start + 32 * cur;
    // wave-uniform: does any key of this block lie past some row's limit?
    const bool masked = tok0 + 32 > lim_min;
    // the segment's last block: V of its tokens past the segment end is zeroed
    // in the slot before any read, so page-tail poison (even NaN) times a zero
    // weight never reaches O
    const int vend = it.seg_end - tok0;
    if (vend < 32) {
      // lane index recomputed here (not hoisted into the loop's live registers)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      if constexpr (SHUF) {
        // V plane units: channel d's 16-byte chunk holds the page's 16 tokens
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pg = r >> 1, d = 2 * ln + (r & 1);
          const int n = min(max(vend - 16 * pg, 0), 16);   // tokens kept in this page
          if (n < 16) {
            uint4* ch = reinterpret_cast<uint4*>(const_cast<uint8_t*>(vU[pg]) + d * 16);
            uint4 v = *ch;
            auto keep = [&](int b0) -> uint32_t {           // bytes b0 .. b0+3
              const int kb = n - b0;
              return kb <= 0 ? 0u : (kb >= 4 ? 0xffffffffu : (0xffffffffu >> (32 - 8 * kb)));
            };
            v.x &= keep(0); v.y &= keep(4); v.z &= keep(8); v.w &= keep(12);
            *ch = v;
          }
        }
      } else {
        // standard pages: token rows 16 pg + tau, V chunks 8 .. 15, 16 bytes each
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pair = 64 * r + ln, tok = pair >> 3, cq = 8 + (pair & 7);
          const int pg = tok >> 4, tau = tok & 15;
          if (tok >= vend)
            *reinterpret_cast<uint4*>(const_cast<uint8_t*>(slot) + pg * kStdTile + tau * kStdRow +
                                      std_chunk_pos(tau, cq, pg) * 16) = make_uint4(0, 0, 0, 0);
        }
      }
      asm volatile("" ::: "memory");
    }

    // ---- V chunks of the block: up to two row tiles, every LDS read is issued
    // before the score MFMAs, so its latency hides behind the MFMAs and the
    // softmax; four row tiles (no registers to spare) read them in the P.V loop ----
    uint2 vraw[8];
    auto read_v1 = [&](int dt) -> uint2 {
      if constexpr (SHUF) {
        const int d = 16 * dt + r16;
        return make_uint2(*reinterpret_cast<const uint32_t*>(vU[0] + d * 16 + 4 * j4),
                          *reinterpret_cast<const uint32_t*>(vU[1] + d * 16 + 4 * j4));
      } else {
        // lanes 0-7 of a group read page 0, lanes 8-15 page 1; token vtau,
        // channel chunk 8 + dt, byte half r16 & 1
        const int pgv = r16 >> 3;
        return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i32_t*)(
                (__attribute__((address_space(3))) uint8_t*)(slot) + pgv * kStdTile +
                vtau * kStdRow + std_chunk_pos(vtau, 8 + dt, pgv) * 16 + (r16 & 1) * 8)));
      }
    };
    if constexpr (!kQLds) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vraw[dt] = read_v1(dt);
    }

    // ---- S^T per page, every tile; independent MFMAs back to back ----
    f32x4_t sacc[NRT][2];
#pragma unroll
    for (int t = 0; t < NRT; ++t) sacc[t][0] = sacc[t][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8_t kop[2][2];
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        const uint4 cw = *reinterpret_cast<const uint4*>(
            SHUF ? kU[pg] + u * 1024 + lane * 16
                 : slot + pg * kStdTile + r16 * kStdRow + std_chunk_pos(r16, 4 * u + j4, pg) * 16);
        kop[pg][0] = as_bf16x8(fp8x8_to_bf16x8(make_uint2(cw.x, cw.y)));
        kop[pg][1] = as_bf16x8(fp8x8_to_bf16x8(make_uint2(cw.z, cw.w)));
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int kk = 2 * u + k2;
        bf16x8_t qo[NRT];
#pragma unroll
        for (int t = 0; t < NRT; ++t)
          qo[t] = kQLds ? as_bf16x8(qs[(t * 4 + kk) * 64 + lane]) : qb[kQLds ? 0 : t][kk];
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int t = 0; t < NRT; ++t)
            sacc[t][pg] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[pg][k2], qo[t], sacc[t][pg], 0, 0, 0);
      }
    }

    // ---- online softmax per tile (row n = 16t + r16; 8 tokens per lane). The
    // masks and the rare rescale are one wave-uniform branch each for all
    // tiles, so the exponentials of every tile and the P.V MFMAs below share
    // one basic block and the scheduler can interleave them. ----
    float sc[NRT][8];
#pragma unroll
    for (int t = 0; t < NRT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[t][e] = sacc[t][e >> 2][e & 3];
    if (masked) {
      asm volatile("");                          // a branch, not selects run every block
#pragma unroll
      for (int t = 0; t < NRT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pos = tok0 + 16 * (e >> 2) + 4 * j4 + (e & 3);
          sc[t][e] = pos < lim[t] ? sc[t][e] : -INFINITY;
        }
    }
    float lm[NRT];
    bool move = false;
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      lm[t] = sc[t][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) lm[t] = fmaxf(lm[t], sc[t][e]);
      move = move || lm[t] > thr[t];
    }
    if (__builtin_amdgcn_ballot_w64(move) != 0) {       // some tile's row max must move
      asm volatile("");
#pragma unroll
      for (int t = 0; t < NRT; ++t) {
        if (__builtin_amdgcn_ballot_w64(lm[t] > thr[t]) == 0) continue;
        float bm = lm[t] == -INFINITY ? -INFINITY : lm[t] * c;
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(m[t], bm);
        const float alpha = fast_exp2(m[t] - (mn == -INFINITY ? 0.f : mn));
        l[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[t][dt] *= alpha;
        m[t] = mn;
        thr[t] = mn == -INFINITY ? -INFINITY : (mn + kSlackLog2) * inv_c;
      }
    }
    bf16x8_t pb[NRT];
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      const float mu = m[t] == -INFINITY ? 0.f : m[t];   // the exp2 offset
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float a = fast_exp2(fmaf(sc[t][e], c, -mu));
        const float b = fast_exp2(fmaf(sc[t][e + 1], c, -mu));
        l[t] += a + b;
        pk[e >> 1] = pack_bf16x2(a, b);
      }
      pb[t] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }

    // ---- O^T += V^T.P^T, V widened once for every tile ----
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8_t vop = as_bf16x8(fp8x8_to_bf16x8(kQLds ? read_v1(dt) : vraw[dt]));
#pragma unroll
      for (int t = 0; t < NRT; ++t)
        oacc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[t], oacc[t][dt], 0, 0, 0);
    }
    cur = nxt;
  };
  while (cur < nblk) {
    step(std::integral_constant<int, 0>{});
    if (cur >= nblk) break;
    step(std::integral_constant<int, 1>{});
  }

  // ---- merge the waves' partial states; write the segment partial ----
  pwait_vmcnt<0>();
  merge_and_write<NW, NRT, NW * R::kBytes>(p, it, &ring[0][0], sm_m, sm_l, oacc, m, l,
                                          out_scale, wave, lane);
}

// ---- bf16 KV: a 32-token block is 16 KB, so the private slots are pages ----
//
// One 16-token page (16 token rows of K then V, 8 KB) per slot. Scores per page
// as above; P.V with v_mfma_f32_16x16x16bf16_1k over the page's 16 tokens: the
// score MFMA's C layout already holds 4 tokens of one row per lane (the B
// operand), and the transposing 16-bit read of the swizzled rows gives each
// lane 4 tokens of one channel (the A operand).
constexpr int kHalf2 = kPageSize * kD * 2;              // a bf16 page's K (or V) half
constexpr int kPage2 = 2 * kHalf2;
constexpr int kPageInstr2 = kPage2 / 1024;
constexpr int kStdRow2 = 2 * kD * 2;
typedef i16x4_t v4i16_t;

template <int NW, int NRT>
struct PRing2 {
  static constexpr int kBytes = 128 * 1024 / NW;
  static constexpr int kNP = kBytes / kPage2;
  static_assert(kNP >= 2, "two page slots per wave");
  static_assert((kNP - 1) * kPageInstr2 <= 63, "vmcnt range");
};

// one page into a slot: standard pages as 16 whole token rows (two per
// instruction, streamed, chunks swizzled by std2_chunk_pos); the shuffled
// planes as they are (K plane rows and the V plane are whole lines too)
template <bool SHUF, int PSH>
__device__ __forceinline__ void issue_page2(const SegParams& p, const SegItem& it, int pid,
                                            int sub, uint8_t* slot, int lane) {
  const int r16 = lane & 15, j4 = lane >> 4;
  const SubPageAddr sp = sub_page<2, SHUF, PSH>(p, it.g, pid, sub);
  if constexpr (!SHUF) {
#pragma unroll
    for (int i = 0; i < kPage2 / 1024; ++i) {
      const int row = 2 * i + (lane >> 5);
      const int q = std2_chunk_pos(row, lane & 31);          // the chunk stored there
      dma16_lds<true>(sp.k + static_cast<size_t>(row) * kStdRow2 + q * 16, slot + i * 1024);
    }
    return;
  }
  const int krow = kplane_row_bytes<PSH>();
#pragma unroll
  for (int i = 0; i < kHalf2 / 1024; ++i)
    dma16_lds<true>(sp.k + static_cast<size_t>(4 * i + j4) * krow + r16 * 16, slot + i * 1024);
#pragma unroll
  for (int i = 0; i < kHalf2 / 1024; ++i)
    dma16_lds<true>(sp.v + static_cast<size_t>(i * 64 + lane) * 16, slot + kHalf2 + i * 1024);
}

template <bool SHUF, int NRT, int NW, bool F16, int PSH>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void seg_mfma_priv2_kernel(SegParams p) {
  using R = PRing2<NW, NRT>;
  constexpr int kNP = R::kNP;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NW][R::kBytes];
  __shared__ __attribute__((aligned(16))) float sm_m[NRT][16][NW + 4];
  __shared__ __attribute__((aligned(16))) float sm_l[NRT][16][NW + 4];

  const SegItem it = decode_item(p);
  write_fixed_counts(p, it);
  if (!it.valid) return;                                          // work-group uniform
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, j4 = lane >> 4;
  const int seg_pages = (it.seg_end - it.seg_start + 15) >> 4;
  const int np = seg_pages > wave ? (seg_pages - wave + NW - 1) / NW : 0;   // this wave's pages
  const int seg_page0 = it.seg_start >> 4;          // first 16-token sub-page
  constexpr int psh = PSH - 4;
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(
          p.page_table + static_cast<size_t>(it.seq) * p.pt_stride);
  // scores enter exp2 as fma(raw, c, -m); c > 0 (16-bit KV has no scale)
  constexpr float c = kScoreScaleLog2;
  // every row sees at least the keys below lim_min (the first row is the most
  // restricted)
  const int lim_min = row_limit(it, it.row0, p.G, p.causal);

  uint8_t* wring = ring[wave];
  // this wave's k-th sub-page is the segment's sub-page wave + NW k
  auto vpage = [&](int k) { return seg_page0 + wave + NW * k; };
  auto pid_of = [&](int k) { return ptab[vpage(k) >> psh]; };
  // the first page is issued before Q is loaded, so the two latencies
  // overlap (the wait for Q also waits for this page; nothing else is in flight)
  static_assert(kNP == 2, "one page ahead");
  if (np > 0) issue_page2<SHUF, PSH>(p, it, pid_of(0), sub_of<PSH>(vpage(0)), wring, lane);

  bf16x8_t qb[NRT][4];
  int lim[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const int n = it.row0 + 16 * t + r16;
    lim[t] = row_limit(it, n, p.G, p.causal);
    const bool ok = n < it.rows;
    const int tq = it.c0 + (ok ? n / p.G : 0);
    const int h = it.g * p.G + (ok ? n % p.G : 0);
    const uint16_t* qr = p.q + (static_cast<size_t>(tq) * p.Hq + h) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qb[t][kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 32 * kk + 8 * j4));
  }
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      asm volatile("" : "+v"(qb[t][kk]));        // Q consumed while only page 0 is in flight
      if (it.row0 + 16 * t + r16 >= it.rows) qb[t][kk] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }


  f32x4_t oacc[NRT][8];
  float m[NRT], l[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // transposing 16-bit read: in each 16-lane group lane i receives element i%4
  // of the 8 bytes read by lane 4k + i/4; lane j reads token tau = 4*j4 + j/4,
  // channels 16dt + 4(j%4) .. +3 (half j%2 of V chunk 2dt + (j/2)%2, at its
  // swizzled position in the token's row), so lane i gets tokens 4*j4 .. +3 of
  // channel 16dt + i
  const int vtr_tau = 4 * j4 + (r16 >> 2);
  const int vtr_row = vtr_tau * kStdRow2 + (r16 & 1) * 8;

  for (int k = 0; k < np; ++k) {
    if (k + kNP - 1 < np)                       // slot of page k-1, consumed last iteration
      issue_page2<SHUF, PSH>(p, it, pid_of(k + kNP - 1), sub_of<PSH>(vpage(k + kNP - 1)),
                        wring + ((k + kNP - 1) % kNP) * kPage2,
                        lane);
    pwait_blocks<kPageInstr2, kNP - 1>(min(kNP - 1, np - 1 - k));   // page k landed
    const uint8_t* sK = wring + (k % kNP) * kPage2;
    const uint8_t* sV = sK + kHalf2;
    const int tok0 = it.seg_start + 16 * (wave + NW * k);

    // ---- S^T of the page, every tile ----
    bf16x8_t kop[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kop[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(
          SHUF ? sK + kk * 1024 + lane * 16
               : sK + r16 * kStdRow2 + std2_chunk_pos(r16, 4 * kk + j4) * 16));
    v4i16_t pb[NRT];
    // wave-uniform: does any key of this page lie past some row's limit?
    // (masks, rescale and V-tail zeroing stay branches, not selects: most
    // pages take none of them)
    const bool masked = tok0 + 16 > lim_min;
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma_k32<F16>(kop[kk], qb[t][kk], acc);
      // online softmax: this lane holds tokens 4*j4 .. +3 of row 16t + r16
      float s[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = acc[e];
      if (masked) {
        asm volatile("");
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = tok0 + 4 * j4 + e < lim[t] ? s[e] : -INFINITY;
      }
      float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      bm = bm == -INFINITY ? -INFINITY : bm * c;
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(m[t], bm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      if (__builtin_amdgcn_ballot_w64(mn != m[t]) != 0) {  // some row max moved
        asm volatile("");
        const float alpha = fast_exp2(m[t] - mu);
        l[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[t][dt] *= alpha;
        m[t] = mn;
      }
      const float a0 = fast_exp2(fmaf(s[0], c, -mu)), a1 = fast_exp2(fmaf(s[1], c, -mu));
      const float a2 = fast_exp2(fmaf(s[2], c, -mu)), a3 = fast_exp2(fmaf(s[3], c, -mu));
      l[t] += (a0 + a1) + (a2 + a3);
      pb[t] = __builtin_bit_cast(v4i16_t, make_uint2(pack2<F16>(a0, a1), pack2<F16>(a2, a3)));
    }

    // ---- O^T += V^T.P^T over the page's 16 tokens ----
    const int vend = it.seg_end - tok0;          // tokens of the page before the end
    auto pv = [&](auto tail_tag) __attribute__((always_inline)) {
      constexpr bool tail = decltype(tail_tag)::value;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 w;
      if constexpr (SHUF) {
        // V plane [N/x][D][x]: channel d's 16-byte chunk of token group g holds
        // tokens 8g .. 8g+7; this lane needs tokens 4*j4 .. +3
        const int d = 16 * dt + r16;
        w = *reinterpret_cast<const uint2*>(sV + ((j4 >> 1) * kD + d) * 16 + (j4 & 1) * 8);
      } else {
        const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(
                (__attribute__((address_space(3))) uint8_t*)(sK) + vtr_row +
                std2_chunk_pos(vtr_tau, 16 + 2 * dt + ((r16 >> 1) & 1)) * 16));
        w = __builtin_bit_cast(uint2, v);
      }
      if (tail) {                    // zero V of tokens past the segment end
        const int rel0 = vend - 4 * j4, rel1 = rel0 - 2;
        w.x = rel0 <= 0 ? 0u : (rel0 == 1 ? (w.x & 0xffffu) : w.x);
        w.y = rel1 <= 0 ? 0u : (rel1 == 1 ? (w.y & 0xffffu) : w.y);
      }
      const v4i16_t vop = __builtin_bit_cast(v4i16_t, w);
#pragma unroll
      for (int t = 0; t < NRT; ++t)
        oacc[t][dt] = mfma_k16<F16>(vop, pb[t], oacc[t][dt]);
    }
    };
    if (vend < 16) {                              // wave-uniform
      asm volatile("");
      pv(std::true_type{});
    } else {
      pv(std::false_type{});
    }
  }

  // ---- merge the waves' partial states; write the segment partial ----
  pwait_vmcnt<0>();
  merge_and_write<NW, NRT, NW * R::kBytes>(p, it, &ring[0][0], sm_m, sm_l, oacc, m, l,
                                          1.f, wave, lane);
}

template <bool SHUF, int PSH>
int launch_priv(const SegParams& sp, int nrt, int grid, hipStream_t st) {
  // 8 waves (two per SIMD) at every row count; four row tiles read Q from LDS
  if (nrt <= 1)
    hipLaunchKernelGGL((seg_mfma_priv_kernel<SHUF, 1, 8, PSH>), dim3(grid), dim3(64 * 8), 0, st,
                       sp);
  else if (nrt <= 2)
    hipLaunchKernelGGL((seg_mfma_priv_kernel<SHUF, 2, 8, PSH>), dim3(grid), dim3(64 * 8), 0, st,
                       sp);
  else
    hipLaunchKernelGGL((seg_mfma_priv_kernel<SHUF, 4, 8, PSH>), dim3(grid), dim3(64 * 8), 0, st,
                       sp);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

// bf16 or fp16 with up to two row tiles (four would not fit two waves per SIMD)
template <bool SHUF, bool F16, int PSH>
int launch_priv2_t(const SegParams& sp, int nrt, int grid, hipStream_t st) {
  if (nrt > 2) return SKV_EUNSUPPORTED;
  if (nrt <= 1)
    hipLaunchKernelGGL((seg_mfma_priv2_kernel<SHUF, 1, 8, F16, PSH>), dim3(grid), dim3(64 * 8), 0,
                       st, sp);
  else
    hipLaunchKernelGGL((seg_mfma_priv2_kernel<SHUF, 2, 8, F16, PSH>), dim3(grid), dim3(64 * 8), 0,
                       st, sp);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

template <int PSH>
int launch_priv_all(const SegParams& sp, int e, bool f16, bool shuf, int nrt, int grid,
                    hipStream_t st) {
  if (e == 2) {
    if (f16)
      return shuf ? launch_priv2_t<true, true, PSH>(sp, nrt, grid, st)
                  : launch_priv2_t<false, true, PSH>(sp, nrt, grid, st);
    return shuf ? launch_priv2_t<true, false, PSH>(sp, nrt, grid, st)
                : launch_priv2_t<false, false, PSH>(sp, nrt, grid, st);
  }
  return shuf ? launch_priv<true, PSH>(sp, nrt, grid, st) : launch_priv<false, PSH>(sp, nrt, grid, st);
}

}  // namespace

int launch_segments_mfma_priv(const SegParams& sp, int e, bool f16, bool shuf, int max_rows,
                              int grid, hipStream_t st) {
  const int nrt = (max_rows + 15) / 16;
  return sp.page_shift == 5 ? launch_priv_all<5>(sp, e, f16, shuf, nrt, grid, st)
                            : launch_priv_all<4>(sp, e, f16, shuf, nrt, grid, st);
}

}  // namespace skv
