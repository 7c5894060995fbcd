// Standard <-> shuffled repack of whole units of heads through LDS: the
// in-place conversion of received byte halves, its inverse, and the
// out-of-place unshuffle.
//
// vLLM RFC #59111, "NixlConnector: convert standard KV pages to ROCm AITER
// shuffled pages on the decode side":
//  * Background: one block's standard form is [H, N, 2D] (per head, N token
//    rows of K channels then V channels); the shuffled form keeps K as
//    [H, D/x, N, x] and V as [H, N/x, D, x] in two planes, x = 16 / element
//    bytes.
//  * Proposed Change §3 (Descriptors): a decoder with separate K and V planes
//    receives a remote standard block as two regions of half a block each,
//    so after the transfer K-plane block b holds the standard block's first
//    byte half and V-plane block b its second half.
//  * Proposed Change §4 (Convert) and Test plan: the received blocks are
//    converted into the shuffled planes; a round trip must restore them.
//
// MI355X design (16- or 32-token pages, head dim 64, 128 or 256): one
// work-group per unit. A unit is
// a whole block (all H heads) for the in-place conversion, because the two
// halves interleave heads:
// writing any shuffled byte of a block destroys standard bytes of other heads
// (with odd H one head straddles the halves), so the whole block is staged in
// LDS before anything is written. For the out-of-place unshuffle a unit is one
// (block, head). Phase 1 reads the unit's bytes with coalesced 16-byte loads
// (eight in flight per thread, from clamped indexes so no load waits on a
// branch) into an LDS image of the standard tile; after one barrier, phase 2
// writes the destination with coalesced 16-byte stores. The standard image's
// 16-byte chunk c of token row n is stored at column c ^ n, so the 16 rows one
// K-plane chunk column gathers fall in distinct LDS banks. Every HBM byte is
// read once and written once. Units must be distinct blocks: listing a block
// twice makes two work-groups rewrite it concurrently.
#include <hip/hip_runtime.h>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;             // 16-byte loads in flight per thread

template <int E, int kN, int kD>
struct Geo {
  static constexpr int kX = 16 / E;                  // elements per 16 bytes
  static constexpr int kRowChunks = 2 * kD * E / 16; // chunks per standard row
  static constexpr int kKChunks = kD * E / 16;       // chunks of a row's K part
  static constexpr int kPlaneChunks = kN * kKChunks; // one head in one plane
  static constexpr int kHeadChunks = 2 * kPlaneChunks;
  static_assert((kRowChunks & (kRowChunks - 1)) == 0, "swizzle needs 2^k");
};

// LDS chunk index of standard chunk c of token row n of head h
template <int E, int kN, int kD>
__device__ __forceinline__ int slot(int h, int n, int c) {
  using G = Geo<E, kN, kD>;
  return (h * kN + n) * G::kRowChunks + (c ^ (n & (G::kRowChunks - 1)));
}

// Global 16-byte loads and stores with the non-temporal (streaming) cache
// policy: every byte is read once and written once, and streamed accesses
// reach markedly more of the HBM bandwidth than the default policy.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gld16(const uint8_t* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void gst16(uint8_t* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_nt*>(p));
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(uint8_t* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Unit u covers `uh` heads starting at head h0 of block b. Its standard bytes
// are two regions of uh*P bytes each (P = one head's plane bytes): the first
// at sa + base*s_mul, the second at sb + base*s_mul, base = (b*H + h0)*P; its
// shuffled bytes are at kp + base and vp + base. In place: sa = kp, sb = vp,
// s_mul = 1. Out of place: sa = std, sb = std + P, s_mul = 2, uh = 1.
template <int E, int kN, int kD, int CAP, bool TO_SHUF>
__global__ __launch_bounds__(kThreads) void repack_kernel(
    uint8_t* sa, uint8_t* sb, int s_mul, uint8_t* kp, uint8_t* vp,
    const int32_t* __restrict__ block_ids, int kv_heads, int uh) {
  using G = Geo<E, kN, kD>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[CAP];
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int per_block = kv_heads / uh;           // units per block
  const int li = u / per_block;
  const int b = block_ids ? block_ids[li] : li;
  const int h0 = (u % per_block) * uh;
  const size_t P = static_cast<size_t>(G::kPlaneChunks) * 16;
  const size_t base = (static_cast<size_t>(b) * kv_heads + h0) * P;
  uint8_t* A = sa + base * s_mul;                // standard, first half
  uint8_t* B = sb + base * s_mul;                // standard, second half
  uint8_t* K = kp + base;
  uint8_t* V = vp + base;
  const int half = uh * G::kPlaneChunks;         // chunks per region
  const int total = 2 * half;

  if constexpr (TO_SHUF) {
    // 1. standard chunks (row-major over [uh, N, 2D]) -> LDS image
    for (int i0 = tid; i0 < total; i0 += kThreads * kBatch) {
      uint4 v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        int i = i0 + k * kThreads;
        i = i < total ? i : total - 1;
        v[k] = gld16(i < half ? A + 16 * i : B + 16 * (i - half));
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int i = i0 + k * kThreads;
        if (i < total) {
          const int h = i / G::kHeadChunks, r = i % G::kHeadChunks;
          st16(lds + 16 * slot<E, kN, kD>(h, r / G::kRowChunks, r % G::kRowChunks), v[k]);
        }
      }
    }
    __syncthreads();
    // 2a. K plane: chunk o = (h, c, n) is token n's K chunk c
    for (int o = tid; o < half; o += kThreads) {
      const int h = o / G::kPlaneChunks, r = o % G::kPlaneChunks;
      gst16(K + 16 * o, ld16(lds + 16 * slot<E, kN, kD>(h, r % kN, r / kN)));
    }
    // 2b. V plane: chunk o = (h, g, d) holds tokens g*x .. g*x+x-1 of channel d
    for (int o = tid; o < half; o += kThreads) {
      const int h = o / G::kPlaneChunks, r = o % G::kPlaneChunks;
      const int g = r / kD, d = r % kD;
      const int cc = G::kKChunks + (d * E) / 16, off = (d * E) % 16;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 4 / E; ++j) {
          const int n = g * G::kX + q * (4 / E) + j;
          const uint8_t* p = lds + 16 * slot<E, kN, kD>(h, n, cc) + off;
          const uint32_t e = E == 2 ? *reinterpret_cast<const uint16_t*>(p) : *p;
          acc |= e << (8 * E * j);
        }
        w[q] = acc;
      }
      gst16(V + 16 * o, make_uint4(w[0], w[1], w[2], w[3]));
    }
  } else {
    // 1a. K plane chunks -> LDS image
    for (int o0 = tid; o0 < half; o0 += kThreads * kBatch) {
      uint4 v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int o = o0 + k * kThreads;
        v[k] = gld16(K + 16 * (o < half ? o : half - 1));
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int o = o0 + k * kThreads;
        if (o < half) {
          const int h = o / G::kPlaneChunks, r = o % G::kPlaneChunks;
          st16(lds + 16 * slot<E, kN, kD>(h, r % kN, r / kN), v[k]);
        }
      }
    }
    // 1b. V plane chunks -> scattered into the rows' V parts
    for (int o0 = tid; o0 < half; o0 += kThreads * kBatch) {
      uint4 v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int o = o0 + k * kThreads;
        v[k] = gld16(V + 16 * (o < half ? o : half - 1));
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int o = o0 + k * kThreads;
        if (o < half) {
          const int h = o / G::kPlaneChunks, r = o % G::kPlaneChunks;
          const int g = r / kD, d = r % kD;
          const int cc = G::kKChunks + (d * E) / 16, off = (d * E) % 16;
          const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int j = 0; j < 4 / E; ++j) {
              const int n = g * G::kX + q * (4 / E) + j;
              uint8_t* p = lds + 16 * slot<E, kN, kD>(h, n, cc) + off;
              const uint32_t e = w[q] >> (8 * E * j);
              if constexpr (E == 2)
                *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(e);
              else
                *p = static_cast<uint8_t>(e);
            }
          }
        }
      }
    }
    __syncthreads();
    // 2. LDS image -> standard chunks
    for (int i = tid; i < total; i += kThreads) {
      const int h = i / G::kHeadChunks, r = i % G::kHeadChunks;
      const uint4 v = ld16(lds + 16 * slot<E, kN, kD>(h, r / G::kRowChunks, r % G::kRowChunks));
      gst16(i < half ? A + 16 * i : B + 16 * (i - half), v);
    }
  }
}

template <int E, int kN, int kD, bool TO_SHUF>
int launch_cap(size_t lds_bytes, unsigned units, uint8_t* sa, uint8_t* sb,
               int s_mul, uint8_t* kp, uint8_t* vp, const int32_t* ids,
               int kv_heads, int uh, hipStream_t st) {
  const dim3 grid(units), block(kThreads);
#define SKV_CAP(C)                                                                    \
  if (lds_bytes <= (C)) {                                                             \
    hipLaunchKernelGGL((repack_kernel<E, kN, kD, (C), TO_SHUF>), grid, block, 0, st, \
                       sa, sb, s_mul, kp, vp, ids, kv_heads, uh);                     \
    return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;                    \
  }
  SKV_CAP(8 * 1024)
  SKV_CAP(16 * 1024)
  SKV_CAP(32 * 1024)
  SKV_CAP(64 * 1024)
  SKV_CAP(kMaxConvertBytes)
#undef SKV_CAP
  return SKV_EUNSUPPORTED;
}

template <int kD>
int launch_repack_d(uint8_t* sa, uint8_t* sb, int s_mul, uint8_t* kp, uint8_t* vp,
                    const int32_t* ids, unsigned n, int kv_heads, int uh, int page_size,
                    int elem_bytes, bool to_shuf, hipStream_t st) {
  const size_t lds = static_cast<size_t>(uh) * page_size * 2 * kD * elem_bytes;
#define SKV_GO(E, N)                                                                   \
  return to_shuf                                                                       \
      ? launch_cap<E, N, kD, true>(lds, n, sa, sb, s_mul, kp, vp, ids, kv_heads, uh, st) \
      : launch_cap<E, N, kD, false>(lds, n, sa, sb, s_mul, kp, vp, ids, kv_heads, uh, st)
  if (page_size == 32) {
    if (elem_bytes == 2) SKV_GO(2, 32);
    SKV_GO(1, 32);
  }
  if (elem_bytes == 2) SKV_GO(2, 16);
  SKV_GO(1, 16);
#undef SKV_GO
}

int launch_repack(uint8_t* sa, uint8_t* sb, int s_mul, uint8_t* kp, uint8_t* vp,
                  const int32_t* ids, long long units, int kv_heads, int uh,
                  int page_size, int head_dim, int elem_bytes, bool to_shuf, void* stream) {
  if (units > 0x7fffffffLL) return SKV_EUNSUPPORTED;
  auto st = static_cast<hipStream_t>(stream);
  const auto n = static_cast<unsigned>(units);
  switch (head_dim) {
    case 64:
      return launch_repack_d<64>(sa, sb, s_mul, kp, vp, ids, n, kv_heads, uh, page_size,
                                 elem_bytes, to_shuf, st);
    case 128:
      return launch_repack_d<128>(sa, sb, s_mul, kp, vp, ids, n, kv_heads, uh, page_size,
                                  elem_bytes, to_shuf, st);
    case 256:
      return launch_repack_d<256>(sa, sb, s_mul, kp, vp, ids, n, kv_heads, uh, page_size,
                                  elem_bytes, to_shuf, st);
    default:
      return SKV_EUNSUPPORTED;
  }
}

}  // namespace

int launch_convert(void* k_plane, void* v_plane, const int32_t* block_ids,
                   int num_blocks, int kv_heads, int page_size, int head_dim,
                   int elem_bytes, int direction, void* stream) {
  auto kp = static_cast<uint8_t*>(k_plane);
  auto vp = static_cast<uint8_t*>(v_plane);
  return launch_repack(kp, vp, 1, kp, vp, block_ids, num_blocks, kv_heads, kv_heads,
                       page_size, head_dim, elem_bytes, direction == SKV_TO_SHUFFLED,
                       stream);
}

int launch_unshuffle(const void* k_plane, const void* v_plane, void* std_cache,
                     const int32_t* block_ids, int num_blocks, int kv_heads,
                     int page_size, int head_dim, int elem_bytes, void* stream) {
  auto s = static_cast<uint8_t*>(std_cache);
  const size_t P = static_cast<size_t>(page_size) * head_dim * elem_bytes;
  // the planes are only read in this direction
  auto kp = const_cast<uint8_t*>(static_cast<const uint8_t*>(k_plane));
  auto vp = const_cast<uint8_t*>(static_cast<const uint8_t*>(v_plane));
  return launch_repack(s, s + P, 2, kp, vp, block_ids,
                       static_cast<long long>(num_blocks) * kv_heads, kv_heads, 1,
                       page_size, head_dim, elem_bytes, false, stream);
}

}  // namespace skv
