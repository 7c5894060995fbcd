// Segment attention, vector-ALU variant (query rows = GQA group x query tokens
// <= 8: too few to fill a 16-row matrix-core tile).
//
// sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware split-KV
// for dynamic workload", Motivation and Modifications: one work-group per
// (segment, sequence, kv head) writes the per-segment partial of all the
// sequence's query rows of that kv head; it decodes (seq, seg) from the work
// list and leaves on -1.
//
// MI355X design:
//  * 256 threads = 4 wave64s, one per SIMD; the segment is cut into blocks of
//    four pages (two at 8 rows, to bound registers) handed to the waves
//    round-robin; each wave keeps its
//    own online-softmax state and the waves merge once through LDS.
//  * q.k: four lanes per token (a quad), each owning 32 of the 128 channels;
//    the quad's 16-byte loads cover a token's K row contiguously. Products use
//    v_dot2_f32_bf16 on bf16 pairs; the quad sum is two DPP quad permutes.
//  * Row max: DPP row rotations within 16 lanes, then two lane permutes.
//  * p.V, standard pages: lane (token phase, 8-channel chunk) loads 16-byte V
//    row chunks (coalesced) and accumulates in fp32; p comes from a per-wave LDS
//    buffer. Shuffled pages: a 16-byte V chunk is x tokens of one channel, so a
//    lane owns two channels and takes v_dot2 over token pairs with bf16 p.
//  * fp8 e4m3fn codes are widened exactly to bf16/fp32 (v_cvt_pk_f32_fp8);
//    k_scale folds into the score scale and v_scale into the output.
//  * Tail V rows are zeroed and masked scores forced to -inf, so poison in page
//    tails never reaches the result. Next-block loads are issued before the
//    current block is computed.
#include "skv_attn_common.h"
#include "skv.h"

namespace skv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kD = kHeadDim;

// NS pages (16-token steps) per block; E element bytes
template <int E, int NS>
struct VGeo {
  static constexpr int kBlockTok = 16 * NS;
  static constexpr int kStdTile = kPageSize * 2 * kD * E;
  static constexpr int kPlaneTile = kPageSize * kD * E;
  static constexpr int kStdRow = 2 * kD * E;
  static constexpr int kKLoadsPerStep = E == 2 ? 4 : 2;      // 16-byte K loads per token quarter
  static constexpr int kKLoads = NS * kKLoadsPerStep;        // per block
  static constexpr int kVLoads = (E == 2 ? 4 : 2) * NS;      // 16-byte V loads per block
};

template <int E, int NS>
struct VRegs {
  uint4 k[VGeo<E, NS>::kKLoads];
  uint4 v[VGeo<E, NS>::kVLoads];
};

template <int E, bool SHUF, int NS>
__device__ __forceinline__ void vload_block(const SegParams& p, const SegItem& it,
                                            const int32_t* ptab, int blk, int lane,
                                            VRegs<E, NS>& r) {
  using Gm = VGeo<E, NS>;
  const int tok0 = it.seg_start + blk * Gm::kBlockTok;
  const int page0 = tok0 >> 4;
  const uint8_t* ktile[NS];
  const uint8_t* vtile[NS];
  bool ok[NS];
#pragma unroll
  for (int pg = 0; pg < NS; ++pg) {
    ok[pg] = tok0 + 16 * pg < it.seg_end;
    const int pid = ok[pg] ? ptab[page0 + pg] : 0;
    const size_t head = static_cast<size_t>(pid) * p.Hkv + it.g;
    if constexpr (SHUF) {
      ktile[pg] = p.kv_a + head * Gm::kPlaneTile;
      vtile[pg] = p.kv_b + head * Gm::kPlaneTile;
    } else {
      ktile[pg] = p.kv_a + head * Gm::kStdTile;
      vtile[pg] = ktile[pg];
    }
  }
  const int tq = lane >> 2, qq = lane & 3;
  // K: step st = page st, token tq; quarter qq
#pragma unroll
  for (int st = 0; st < NS; ++st) {
#pragma unroll
    for (int k = 0; k < Gm::kKLoadsPerStep; ++k) {
      size_t off;
      if constexpr (SHUF) off = (static_cast<size_t>(4 * k + qq) * kPageSize + tq) * 16;
      else off = static_cast<size_t>(tq) * Gm::kStdRow + 64 * k + 16 * qq;
      r.k[st * Gm::kKLoadsPerStep + k] =
          ok[st] ? *reinterpret_cast<const uint4*>(ktile[st] + off) : make_uint4(0, 0, 0, 0);
    }
  }
  if constexpr (!SHUF) {
    // lane (phase tp, chunk c); tokens tp + kPh * u
    constexpr int kCh = kD * E / 16;           // chunks per V row: 16 (bf16) / 8 (fp8)
    constexpr int kPh = 64 / kCh;              // token phases: 4 / 8
    const int tp = lane / kCh, c = lane % kCh;
#pragma unroll
    for (int u = 0; u < Gm::kVLoads; ++u) {
      const int tau = tp + kPh * u;
      const int pg = tau >> 4, slot = tau & 15;
      const size_t off = static_cast<size_t>(slot) * Gm::kStdRow + kD * E + c * 16;
      r.v[u] = ok[pg] ? *reinterpret_cast<const uint4*>(vtile[pg] + off) : make_uint4(0, 0, 0, 0);
    }
  } else if constexpr (E == 2) {
    // channel d = lane + 64*h, 8-token group g (page g/2, in-page group g%2)
#pragma unroll
    for (int g = 0; g < 2 * NS; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pg = g >> 1;
        const size_t off = (static_cast<size_t>(g & 1) * kD + lane + 64 * h) * 16;
        r.v[2 * g + h] = ok[pg] ? *reinterpret_cast<const uint4*>(vtile[pg] + off)
                                : make_uint4(0, 0, 0, 0);
      }
  } else {
    // x = 16: one chunk per (page, channel) holds the page's 16 tokens
#pragma unroll
    for (int pg = 0; pg < NS; ++pg)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const size_t off = static_cast<size_t>(lane + 64 * h) * 16;
        r.v[2 * pg + h] = ok[pg] ? *reinterpret_cast<const uint4*>(vtile[pg] + off)
                                 : make_uint4(0, 0, 0, 0);
      }
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

template <int E, bool SHUF, int RM, int NS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void seg_valu_kernel(SegParams p) {
  using Gm = VGeo<E, NS>;
  constexpr int kBlockTok = Gm::kBlockTok;
  constexpr int kPBytes = SHUF ? RM * kBlockTok * 2 : kBlockTok * RM * 4;
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[kWaves][kPBytes];
  __shared__ __attribute__((aligned(16))) float oslot[kWaves][RM][kD];
  __shared__ float sm_m[kWaves][RM];
  __shared__ float sm_l[kWaves][RM];

  const SegItem it = decode_item(p);
  if (!it.valid) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tq = lane >> 2, qq = lane & 3;
  const int ntok = it.seg_end - it.seg_start;
  const int nblk = (ntok + kBlockTok - 1) / kBlockTok;
  const int32_t* ptab = p.page_table + static_cast<size_t>(it.seq) * p.pt_stride;
  float sm_scale = kScoreScaleLog2;
  float out_scale = 1.f;
  if constexpr (E == 1) {
    sm_scale *= p.k_scale[0];
    out_scale = p.v_scale[0];
  }

  // Q rows (bf16 pairs) for this lane's 32 channels
  uint4 qr[RM][4];
  int lim[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    lim[r] = row_limit(it, r, p.G, p.causal);
    const bool okr = r < it.rows;
    const int t = it.c0 + (okr ? r / p.G : 0);
    const int h = it.g * p.G + (okr ? r % p.G : 0);
    const uint16_t* q = p.q + (static_cast<size_t>(t) * p.Hq + h) * kD;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // E==2: chunk k=u -> channels 32u + 8qq; E==1: (k=u/2, half u%2) -> 64k + 16qq + 8h
      const int ch = E == 2 ? 32 * u + 8 * qq : 64 * (u >> 1) + 16 * qq + 8 * (u & 1);
      qr[r][u] = okr ? *reinterpret_cast<const uint4*>(q + ch) : make_uint4(0, 0, 0, 0);
    }
  }

  constexpr int kAcc = SHUF ? 2 : (E == 2 ? 8 : 16);
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
  VRegs<E, NS> cur, nxt;
  if (wave < nblk) vload_block<E, SHUF, NS>(p, it, ptab, wave, lane, cur);

  for (int blk = wave; blk < nblk; blk += kWaves) {
    if (blk + kWaves < nblk) vload_block<E, SHUF, NS>(p, it, ptab, blk + kWaves, lane, nxt);
    const int tok0 = it.seg_start + blk * kBlockTok;
    const bool tail = tok0 + kBlockTok > it.seg_end;

    // ---- scores: s[st][r] for token 16*st + tq ----
    float s[NS][RM];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      uint4 kw[4];
      if constexpr (E == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) kw[u] = cur.k[st * 4 + u];
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint4 c = cur.k[st * 2 + k];
          kw[2 * k] = fp8x8_to_bf16x8(make_uint2(c.x, c.y));
          kw[2 * k + 1] = fp8x8_to_bf16x8(make_uint2(c.z, c.w));
        }
      }
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a = dot2_bf16(kw[u].x, qr[r][u].x, a);
          a = dot2_bf16(kw[u].y, qr[r][u].y, a);
          a = dot2_bf16(kw[u].z, qr[r][u].z, a);
          a = dot2_bf16(kw[u].w, qr[r][u].w, a);
        }
        a += dpp<kDppQuadXor1>(a);
        a += dpp<kDppQuadXor2>(a);
        const int pos = tok0 + 16 * st + tq;
        s[st][r] = pos < lim[r] ? a * sm_scale : -INFINITY;
      }
    }

    // ---- online softmax per row; p to the wave's LDS buffer ----
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      float bm = s[0][r];
#pragma unroll
      for (int st = 1; st < NS; ++st) bm = fmaxf(bm, s[st][r]);
      bm = max_over_tokens(bm);
      const float mn = fmaxf(m[r], bm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[r] - mu);
      float ps = 0.f;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s[st][r] = fast_exp2(s[st][r] - mu);
        ps += s[st][r];
      }
      l[r] = l[r] * alpha + ps;
      m[r] = mn;
#pragma unroll
      for (int a = 0; a < kAcc; ++a) acc[r][a] *= alpha;
    }
    if constexpr (!SHUF) {
      // p[tau][r] fp32, written by quarter 0 of each token quad
      if (qq == 0) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          float* dst = reinterpret_cast<float*>(pw) + (16 * st + tq) * RM;
#pragma unroll
          for (int r4 = 0; r4 < RM; r4 += 4)
            *reinterpret_cast<float4*>(dst + r4) =
                make_float4(s[st][r4], s[st][r4 + 1], s[st][r4 + 2], s[st][r4 + 3]);
        }
      }
    } else {
      // p[r][tau] bf16; quarter qq writes rows qq, qq + 4
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        if ((r & 3) == qq) {
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const __bf16 b = static_cast<__bf16>(s[st][r]);
            *reinterpret_cast<__bf16*>(pw + (r * kBlockTok + 16 * st + tq) * 2) = b;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- o += p.V ----
    const int vend = it.seg_end - tok0;      // tokens >= vend are past the segment
    if constexpr (!SHUF) {
      constexpr int kCh = kD * E / 16;
      constexpr int kPh = 64 / kCh;
      const int tp = lane / kCh;
#pragma unroll
      for (int u = 0; u < Gm::kVLoads; ++u) {
        const int tau = tp + kPh * u;
        uint4 v = cur.v[u];
        if (tail && tau >= vend) v = make_uint4(0, 0, 0, 0);
        float x[kAcc];
        if constexpr (E == 2) {
          x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
          x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[q2]), false);
            const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[q2]), true);
            x[4 * q2] = a[0]; x[4 * q2 + 1] = a[1]; x[4 * q2 + 2] = b[0]; x[4 * q2 + 3] = b[1];
          }
        }
        const float* pr = reinterpret_cast<const float*>(pw) + tau * RM;
#pragma unroll
        for (int r4 = 0; r4 < RM; r4 += 4) {
          const float4 pv = *reinterpret_cast<const float4*>(pr + r4);
          const float pp[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int a = 0; a < kAcc; ++a) acc[r4 + rr][a] += pp[rr] * x[a];
        }
      }
    } else if constexpr (E == 2) {
#pragma unroll
      for (int g = 0; g < 2 * NS; ++g) {
        uint4 vv[2] = {cur.v[2 * g], cur.v[2 * g + 1]};
        if (tail) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint32_t w[4] = {vv[h].x, vv[h].y, vv[h].z, vv[h].w};
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
              const int tau = 8 * g + 2 * q2;
              if (tau >= vend) w[q2] = 0;
              else if (tau + 1 >= vend) w[q2] &= 0xffffu;
            }
            vv[h] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r) {
          const uint4 pp = *reinterpret_cast<const uint4*>(pw + (r * kBlockTok + 8 * g) * 2);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float a = acc[r][h];
            a = dot2_bf16(vv[h].x, pp.x, a);
            a = dot2_bf16(vv[h].y, pp.y, a);
            a = dot2_bf16(vv[h].z, pp.z, a);
            a = dot2_bf16(vv[h].w, pp.w, a);
            acc[r][h] = a;
          }
        }
      }
    } else {
#pragma unroll
      for (int pg = 0; pg < NS; ++pg) {
        uint4 vb[2][2];               // [h][half]: 16 tokens as bf16 pairs
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint4 c = cur.v[2 * pg + h];
          if (tail) {
            uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int b = 0; b < 16; ++b)
              if (16 * pg + b >= vend) w[b >> 2] &= ~(0xffu << (8 * (b & 3)));
            c = make_uint4(w[0], w[1], w[2], w[3]);
          }
          vb[h][0] = fp8x8_to_bf16x8(make_uint2(c.x, c.y));
          vb[h][1] = fp8x8_to_bf16x8(make_uint2(c.z, c.w));
        }
#pragma unroll
        for (int r = 0; r < RM; ++r) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint4 pp = *reinterpret_cast<const uint4*>(
                pw + (r * kBlockTok + 16 * pg + 8 * half) * 2);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float a = acc[r][h];
              a = dot2_bf16(vb[h][half].x, pp.x, a);
              a = dot2_bf16(vb[h][half].y, pp.y, a);
              a = dot2_bf16(vb[h][half].z, pp.z, a);
              a = dot2_bf16(vb[h][half].w, pp.w, a);
              acc[r][h] = a;
            }
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cur = nxt;
  }

  // ---- per-wave totals ----
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    float v = l[r];                           // identical within a quad: sum over tq only
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    l[r] = v;
  }
  if constexpr (!SHUF) {
    constexpr int kCh = kD * E / 16;
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
        for (int a = 0; a < kAcc; ++a) oslot[wave][r][c * kAcc + a] = acc[r][a];
    }
  } else {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      oslot[wave][r][lane] = acc[r][0];
      oslot[wave][r][lane + 64] = acc[r][1];
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
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
    const float mu = M == -INFINITY ? 0.f : M;
    float Ls = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm_m[w][r] - mu);
      Ls += sm_l[w][r] * f;
      o += oslot[w][r][d] * f;
    }
    const int t = it.c0 + r / p.G;
    const int h = it.g * p.G + r % p.G;
    const size_t prow = (static_cast<size_t>(t) * p.Hq + h) * p.seg_max + it.seg;
    const bool any = Ls > 0.f;
    p.part_o[prow * kD + d] = any ? o * (out_scale / Ls) : 0.f;
    if (d == 0) p.part_lse[prow] = any ? (mu + fast_log2(Ls)) * kLn2 : -INFINITY;
  }
}

template <int E, bool SHUF>
int launch_valu_e(const SegParams& sp, int rows, int grid, hipStream_t st) {
  if (rows <= 4)
    hipLaunchKernelGGL((seg_valu_kernel<E, SHUF, 4, 4>), dim3(grid), dim3(kThreads), 0, st, sp);
  else
    hipLaunchKernelGGL((seg_valu_kernel<E, SHUF, 8, 2>), dim3(grid), dim3(kThreads), 0, st, sp);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace

int launch_segments_valu(const SegParams& sp, int e, bool shuf, int max_rows, int grid,
                         hipStream_t st) {
  if (e == 2) return shuf ? launch_valu_e<2, true>(sp, max_rows, grid, st)
                          : launch_valu_e<2, false>(sp, max_rows, grid, st);
  return shuf ? launch_valu_e<1, true>(sp, max_rows, grid, st)
              : launch_valu_e<1, false>(sp, max_rows, grid, st);
}

}  // namespace skv
