// Segment attention, matrix-core variant (query rows = GQA group x query
// tokens >= 9, padded to 16-row tiles).
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Motivation and Modifications: one work-group per
// (segment, sequence, kv head) computes softmax(q.K^T/sqrt(d)).V of all the
// sequence's query rows for that kv head over the segment's pages and writes a
// per-segment partial; the work-group decodes (seq, seg) from the work list.
//
// MI355X design (one work-group per CU by construction of the plan):
//  * 256 threads = 4 wave64s, one per SIMD (waves_per_eu 1 -> 512 VGPRs each).
//    The segment is cut into 32-token blocks (two pages); wave w takes blocks
//    w, w+4, ... and keeps its own online-softmax state, so the main loop has
//    no work-group barrier. Waves merge once at the end through LDS.
//  * Scores are computed transposed, S^T = K.Q^T, with v_mfma_f32_16x16x32_bf16:
//    the A operand is 16 tokens x 32 channels of K (one 16-byte load per
//    lane), the B operand 32 channels x 16 query rows of Q, held in registers
//    for the whole segment. Two token tiles are interleaved (tile a takes
//    tokens 8j+{0..3}, tile b 8j+{4..7} of each 8-token group j) so that the
//    C layout leaves each lane with 8 consecutive tokens of one query row:
//    exactly the B operand (P^T) of the P.V product, with no lane shuffles.
//  * O^T = V^T.P^T: the A operand is 16 channels x 32 tokens of V. In the
//    shuffled layout a 16-byte V chunk already is x tokens of one channel (a
//    direct load); standard pages are staged through a per-wave LDS tile and
//    read back transposed.
//  * Online softmax in the exp2 domain with the row max/sum in registers;
//    the block max is reduced across the four 16-lane groups with lane
//    permutes. Masked lanes are forced to -inf; V rows of page-tail slots are
//    zeroed so poison (even NaN) never reaches the accumulator.
//  * fp8 e4m3fn KV is widened to bf16 exactly before the MFMA; k_scale folds
//    into the score scale and v_scale into the output.
//  * The next block's K/V loads are issued before the current block is
//    computed (register double buffering, 16 KB in flight per wave).
#include "skv_attn_common.h"
#include "skv.h"

namespace skv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBlockTok = 32;
constexpr int kD = kHeadDim;

template <int E>
struct Geo {
  static constexpr int kStdTile = kPageSize * 2 * kD * E;   // (block, head) bytes, standard
  static constexpr int kPlaneTile = kPageSize * kD * E;     // (block, head) bytes, one plane
  static constexpr int kStdRow = 2 * kD * E;                 // one token row, standard
  static constexpr int kKLoads = E == 2 ? 8 : 4;             // 16-byte K loads per lane per block
  static constexpr int kVStdLoads = E == 2 ? 8 : 4;          // 16-byte V chunks per lane (standard)
  static constexpr int kVRowLds = kD * E + 16;               // padded LDS row (standard V)
};

// channel base of the 8 channels a lane feeds into MFMA k-step kk (0..3)
template <int E>
__device__ __forceinline__ int kdim_base(int kk, int j4) {
  if constexpr (E == 2) return 32 * kk + 8 * j4;
  else return 64 * (kk >> 1) + 16 * j4 + 8 * (kk & 1);
}

template <int E, bool SHUF>
struct BlockRegs {
  uint4 k[Geo<E>::kKLoads];
  uint4 v[8];            // SHUF && E==2: V^T operands; standard: raw chunks (E==2: 8, E==1: 4)
  uint2 v8[8];           // SHUF && E==1: 8 fp8 codes per operand
};

template <int E, bool SHUF>
__device__ __forceinline__ void load_block(const SegParams& p, const SegItem& it,
                                           const int32_t* ptab, int blk, int lane,
                                           BlockRegs<E, SHUF>& r) {
  using Gm = Geo<E>;
  const int r16 = lane & 15, j4 = lane >> 4;
  const int tok0 = it.seg_start + blk * kBlockTok;        // page aligned
  const int page0 = tok0 >> 4;
  const bool has1 = tok0 + 16 < it.seg_end;
  const int pid0 = ptab[page0];
  const int pid1 = has1 ? ptab[page0 + 1] : pid0;
  const size_t hs = static_cast<size_t>(p.Hkv);
  const size_t head0 = static_cast<size_t>(pid0) * hs + it.g;
  const size_t head1 = static_cast<size_t>(pid1) * hs + it.g;
  const uint8_t* ka0 = p.kv_a + head0 * (SHUF ? Gm::kPlaneTile : Gm::kStdTile);
  const uint8_t* ka1 = p.kv_a + head1 * (SHUF ? Gm::kPlaneTile : Gm::kStdTile);

  // K: tile tb, token tau = 8*(r16/4) + r16%4 + 4*tb (page tau/16, slot tau%16)
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tau = 8 * (r16 >> 2) + (r16 & 3) + 4 * tb;
    const int pg = tau >> 4, slot = tau & 15;
    const uint8_t* base = pg ? ka1 : ka0;
    const bool ok = pg == 0 || has1;
    constexpr int per = Gm::kKLoads / 2;
#pragma unroll
    for (int u = 0; u < per; ++u) {
      // E==2: u = kk, channels 32kk + 8j4 ; E==1: u = kk pair, channels 64u + 16j4
      const int ch = E == 2 ? 32 * u + 8 * j4 : 64 * u + 16 * j4;
      size_t off;
      if constexpr (SHUF) off = (static_cast<size_t>(ch * E / 16) * kPageSize + slot) * 16;
      else off = static_cast<size_t>(slot) * Gm::kStdRow + ch * E;
      r.k[tb * per + u] = ok ? *reinterpret_cast<const uint4*>(base + off) : make_uint4(0, 0, 0, 0);
    }
  }
  if constexpr (SHUF) {
    const uint8_t* vb0 = p.kv_b + head0 * Gm::kPlaneTile;
    const uint8_t* vb1 = p.kv_b + head1 * Gm::kPlaneTile;
    const int pg = j4 >> 1;
    const uint8_t* vb = pg ? vb1 : vb0;
    const bool ok = pg == 0 || has1;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + r16;
      if constexpr (E == 2) {
        const size_t off = (static_cast<size_t>(j4 & 1) * kD + d) * 16;
        r.v[dt] = ok ? *reinterpret_cast<const uint4*>(vb + off) : make_uint4(0, 0, 0, 0);
      } else {
        const size_t off = static_cast<size_t>(d) * 16 + 8 * (j4 & 1);
        r.v8[dt] = ok ? *reinterpret_cast<const uint2*>(vb + off) : make_uint2(0, 0);
      }
    }
  } else {
    constexpr int cpr = kD * E / 16;                      // V chunks per token row
#pragma unroll
    for (int u = 0; u < Gm::kVStdLoads; ++u) {
      const int ci = u * 64 + lane;
      const int tok = ci / cpr, c = ci % cpr;
      const int pg = tok >> 4, slot = tok & 15;
      const uint8_t* base = pg ? ka1 : ka0;
      const bool ok = pg == 0 || has1;
      const size_t off = static_cast<size_t>(slot) * Gm::kStdRow + kD * E + c * 16;
      r.v[u] = ok ? *reinterpret_cast<const uint4*>(base + off) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int E, bool SHUF, int NRT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void seg_mfma_kernel(SegParams p) {
  using Gm = Geo<E>;
  constexpr int kVTile = kBlockTok * Gm::kVRowLds;               // per-wave V tile
  constexpr int kMergeSlot = 8 * NRT * 64 * 16;                  // one wave's O^T
  constexpr int kLdsBytes = (SHUF ? 0 : kWaves * kVTile) > 2 * kMergeSlot
                                ? kWaves * kVTile : 2 * kMergeSlot;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ float sm_m[kWaves][16 * NRT];
  __shared__ float sm_l[kWaves][16 * NRT];

  const SegItem it = decode_item(p);
  if (!it.valid) return;                                          // work-group uniform
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, j4 = lane >> 4;
  const int nrt = (it.rows + 15) >> 4;
  const int ntok = it.seg_end - it.seg_start;
  const int nblk = (ntok + kBlockTok - 1) / kBlockTok;
  const int32_t* ptab = p.page_table + static_cast<size_t>(it.seq) * p.pt_stride;
  float sm_scale = kScoreScaleLog2;
  float out_scale = 1.f;
  if constexpr (E == 1) {
    sm_scale *= p.k_scale[0];
    out_scale = p.v_scale[0];
  }

  int lim[NRT];
  bf16x8_t qb[NRT][4];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int n = 16 * rt + r16;
    lim[rt] = row_limit(it, n, p.G, p.causal);
    const bool ok = n < it.rows;
    const int t = it.c0 + (ok ? n / p.G : 0);
    const int h = it.g * p.G + (ok ? n % p.G : 0);
    const uint16_t* qr = p.q + (static_cast<size_t>(t) * p.Hq + h) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 v = ok ? *reinterpret_cast<const uint4*>(qr + kdim_base<E>(kk, j4))
                         : make_uint4(0, 0, 0, 0);
      qb[rt][kk] = as_bf16x8(v);
    }
  }

  f32x4_t oacc[8][NRT];
  float m[NRT], l[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  uint8_t* vt = lds + wave * kVTile;                              // standard V tile
  BlockRegs<E, SHUF> cur, nxt;
  if (wave < nblk) load_block<E, SHUF>(p, it, ptab, wave, lane, cur);

  for (int blk = wave; blk < nblk; blk += kWaves) {
    if (blk + kWaves < nblk) load_block<E, SHUF>(p, it, ptab, blk + kWaves, lane, nxt);
    const int tok0 = it.seg_start + blk * kBlockTok;
    const bool tail = tok0 + kBlockTok > it.seg_end;

    // ---- standard layout: V chunks -> LDS (tail slots zeroed) ----
    if constexpr (!SHUF) {
      constexpr int cpr = kD * E / 16;
#pragma unroll
      for (int u = 0; u < Gm::kVStdLoads; ++u) {
        const int ci = u * 64 + lane;
        const int tok = ci / cpr, c = ci % cpr;
        uint4 v = cur.v[u];
        if (tail && tok0 + tok >= it.seg_end) v = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vt + tok * Gm::kVRowLds + c * 16) = v;
      }
    }

    // ---- S^T = K.Q^T ----
    f32x4_t sacc[2][NRT];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      bf16x8_t kop[4];
      if constexpr (E == 2) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kop[kk] = as_bf16x8(cur.k[tb * 4 + kk]);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          kop[2 * u] = as_bf16x8(fp8x8_to_bf16x8(make_uint2(cur.k[tb * 2 + u].x, cur.k[tb * 2 + u].y)));
          kop[2 * u + 1] = as_bf16x8(fp8x8_to_bf16x8(make_uint2(cur.k[tb * 2 + u].z, cur.k[tb * 2 + u].w)));
        }
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        if (rt < nrt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kk], qb[rt][kk], acc, 0, 0, 0);
          sacc[tb][rt] = acc;
        }
      }
    }

    // ---- online softmax; P^T operand per row tile ----
    bf16x8_t pb[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      if (rt < nrt) {
        float s[8];
        float bm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pos = tok0 + 8 * j4 + e;
          const float v = sacc[e >> 2][rt][e & 3] * sm_scale;
          s[e] = pos < lim[rt] ? v : -INFINITY;
          bm = fmaxf(bm, s[e]);
        }
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(m[rt], bm);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float alpha = fast_exp2(m[rt] - mu);
        float ps = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float a = fast_exp2(s[e] - mu), b = fast_exp2(s[e + 1] - mu);
          ps += a + b;
          pk[e >> 1] = pack_bf16x2(a, b);
        }
        l[rt] = l[rt] * alpha + ps;
        m[rt] = mn;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt][rt] *= alpha;
        pb[rt] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
    }

    // ---- O^T += V^T.P^T ----
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint4 vw;
      if constexpr (SHUF && E == 2) {
        vw = cur.v[dt];
      } else if constexpr (SHUF) {
        vw = fp8x8_to_bf16x8(cur.v8[dt]);
      } else if constexpr (E == 2) {
        const uint8_t* col = vt + (8 * j4) * Gm::kVRowLds + (16 * dt + r16) * 2;
        uint32_t w[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(col + (2 * q2) * Gm::kVRowLds);
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(col + (2 * q2 + 1) * Gm::kVRowLds);
          w[q2] = lo | (hi << 16);
        }
        vw = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        const uint8_t* col = vt + (8 * j4) * Gm::kVRowLds + 16 * dt + r16;
        uint32_t w[2];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          uint32_t x = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            x |= static_cast<uint32_t>(col[(4 * q2 + b) * Gm::kVRowLds]) << (8 * b);
          w[q2] = x;
        }
        vw = fp8x8_to_bf16x8(make_uint2(w[0], w[1]));
      }
      if constexpr (SHUF) {
        if (tail) {                      // zero V of tokens past the segment end
          uint32_t w[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const int pos = tok0 + 8 * j4 + 2 * q2;
            if (pos >= it.seg_end) w[q2] = 0;
            else if (pos + 1 >= it.seg_end) w[q2] &= 0xffffu;
          }
          vw = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      const bf16x8_t vop = as_bf16x8(vw);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        if (rt < nrt)
          oacc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[rt], oacc[dt][rt], 0, 0, 0);
    }
    cur = nxt;
  }

  // ---- merge the four waves ----
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    l[rt] += __shfl_xor(l[rt], 16);
    l[rt] += __shfl_xor(l[rt], 32);
  }
  __syncthreads();                       // V tiles are dead; LDS is reused below
  if (j4 == 0) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      sm_m[wave][16 * rt + r16] = m[rt];
      sm_l[wave][16 * rt + r16] = l[rt];
    }
  }
  __syncthreads();
  float Lsum[NRT], Mrow[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = 16 * rt + r16;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][row]);
    const float mu = M == -INFINITY ? 0.f : M;
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Ls += sm_l[w][row] * fast_exp2(sm_m[w][row] - mu);
    Lsum[rt] = Ls;
    Mrow[rt] = mu;
    const float f = fast_exp2(m[rt] - mu);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt][rt] *= f;
  }
  f32x4_t* slot = reinterpret_cast<f32x4_t*>(lds);
  auto slot_at = [&](int s, int dt, int rt) -> f32x4_t& {
    return slot[((s * 8 + dt) * NRT + rt) * 64 + lane];
  };
  if (wave >= 2) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) slot_at(wave - 2, dt, rt) = oacc[dt][rt];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) oacc[dt][rt] += slot_at(wave, dt, rt);
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) slot_at(0, dt, rt) = oacc[dt][rt];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int n = 16 * rt + r16;
    if (n >= it.rows) continue;
    const int t = it.c0 + n / p.G;
    const int h = it.g * p.G + n % p.G;
    const size_t prow = (static_cast<size_t>(t) * p.Hq + h) * p.seg_max + it.seg;
    const bool any = Lsum[rt] > 0.f;
    const float inv = any ? out_scale / Lsum[rt] : 0.f;
    float* po = p.part_o + prow * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      f32x4_t o = (oacc[dt][rt] + slot_at(0, dt, rt)) * inv;
      *reinterpret_cast<f32x4_t*>(po + 16 * dt + 4 * j4) = o;
    }
    if (j4 == 0)
      p.part_lse[prow] = any ? (Mrow[rt] + fast_log2(Lsum[rt])) * kLn2 : -INFINITY;
  }
}

template <int E, bool SHUF>
int launch_mfma_e(const SegParams& sp, int nrt, int grid, hipStream_t st) {
  if (nrt <= 1)
    hipLaunchKernelGGL((seg_mfma_kernel<E, SHUF, 1>), dim3(grid), dim3(kThreads), 0, st, sp);
  else if (nrt <= 2)
    hipLaunchKernelGGL((seg_mfma_kernel<E, SHUF, 2>), dim3(grid), dim3(kThreads), 0, st, sp);
  else
    hipLaunchKernelGGL((seg_mfma_kernel<E, SHUF, 4>), dim3(grid), dim3(kThreads), 0, st, sp);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace

int launch_segments_mfma(const SegParams& sp, int e, bool shuf, int max_rows, int grid,
                         hipStream_t st) {
  const int nrt = (max_rows + 15) / 16;
  if (e == 2) return shuf ? launch_mfma_e<2, true>(sp, nrt, grid, st)
                          : launch_mfma_e<2, false>(sp, nrt, grid, st);
  return shuf ? launch_mfma_e<1, true>(sp, nrt, grid, st)
              : launch_mfma_e<1, false>(sp, nrt, grid, st);
}

}  // namespace skv
