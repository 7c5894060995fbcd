// Standard -> shuffled KV page repack.
//
// vLLM RFC #59111, "NixlConnector: convert standard KV pages to ROCm AITER
// shuffled pages on the decode side", Background and Proposed Change §4: a
// standard block holds per head N token rows of 2D channels (K, then V); the
// shuffled layout stores K as [H, D/x, N, x] and V as [H, N/x, D, x] with
// x = 16 / element bytes, and received blocks are converted block by block.
//
// MI355X design: one wave64 per (listed block, head); 16- or 32-token pages
// (the RFC's decoders use both). The wave copies the head's whole standard
// tile (16 x 2D elements per 16 tokens: 8 KB bf16 at head dim 128) into LDS
// with coalesced 16-byte
// loads (1 KB contiguous per wave instruction), then writes both planes with
// coalesced 16-byte stores: a K chunk is one 16-byte row chunk moved as a unit;
// a V chunk gathers x tokens of one channel from LDS. Every HBM byte is read
// once and written once (the 2x-bytes ideal). LDS rows are padded by 16 bytes
// so the 16 rows a K store reads land in distinct banks.
#include <hip/hip_runtime.h>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kShufThreads = 256;
constexpr int kShufWaves = kShufThreads / 64;
template <int E, int kN, int kD>
struct ShufGeom {
  static constexpr int kX = 16 / E;                   // elements per 16 bytes
  static constexpr int kRowBytes = 2 * kD * E;        // one standard token row
  static constexpr int kTileBytes = kN * kRowBytes;   // one head's block
  static constexpr int kPlaneBytes = kN * kD * E;     // one head's K (or V) plane
  static constexpr int kLdsRow = kRowBytes + 16;      // padded LDS row
  static constexpr int kChunks = kTileBytes / 16;     // 16-byte chunks per tile
};

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

template <int E, int kN, int kD>
__global__ __launch_bounds__(kShufThreads) void shuffle_kernel(
    const uint8_t* __restrict__ src, uint8_t* __restrict__ kpl,
    uint8_t* __restrict__ vpl, const int32_t* __restrict__ block_ids,
    int num_units, int kv_heads) {
  using G = ShufGeom<E, kN, kD>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kShufWaves][kN * G::kLdsRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.x * kShufWaves + wave;
  if (unit >= num_units) return;                        // wave-uniform
  const int b = block_ids ? block_ids[unit / kv_heads] : unit / kv_heads;
  const int h = unit % kv_heads;
  const size_t head = static_cast<size_t>(b) * kv_heads + h;
  const uint8_t* s = src + head * G::kTileBytes;
  uint8_t* kd = kpl + head * G::kPlaneBytes;
  uint8_t* vd = vpl + head * G::kPlaneBytes;
  uint8_t* t = lds[wave];

  // 1. tile -> LDS (chunk c: row c / chunks_per_row, column c % chunks_per_row)
  constexpr int kPerRow = G::kRowBytes / 16;
  uint4 buf[G::kChunks / 64];
#pragma unroll
  for (int k = 0; k < G::kChunks / 64; ++k)
    buf[k] = gld16(s + 16 * (k * 64 + lane));
#pragma unroll
  for (int k = 0; k < G::kChunks / 64; ++k) {
    const int c = k * 64 + lane;
    *reinterpret_cast<uint4*>(t + (c / kPerRow) * G::kLdsRow + (c % kPerRow) * 16) = buf[k];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 2. K plane: output chunk o = c * N + n is token n's K bytes [16c, 16c + 16)
  constexpr int kKChunks = G::kPlaneBytes / 16;
#pragma unroll
  for (int k = 0; k < kKChunks / 64; ++k) {
    const int o = k * 64 + lane;
    const int c = o / kN, n = o % kN;
    gst16(kd + 16 * o, *reinterpret_cast<const uint4*>(t + n * G::kLdsRow + c * 16));
  }
  // 3. V plane: output chunk o = g * D + d holds tokens g*x .. g*x + x - 1 of
  //    V channel d (byte offset D*E + d*E in each row)
#pragma unroll
  for (int k = 0; k < kKChunks / 64; ++k) {
    const int o = k * 64 + lane;
    const int g = o / kD, d = o % kD;
    const uint8_t* col = t + (g * G::kX) * G::kLdsRow + kD * E + d * E;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (E == 2) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(col + (2 * q) * G::kLdsRow);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(col + (2 * q + 1) * G::kLdsRow);
        w[q] = lo | (hi << 16);
      } else {
        uint32_t v = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v |= static_cast<uint32_t>(col[(4 * q + r) * G::kLdsRow]) << (8 * r);
        w[q] = v;
      }
    }
    gst16(vd + 16 * o, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

template <int kN, int kD>
int launch_shuffle_n(const uint8_t* s, uint8_t* k, uint8_t* v, const int32_t* block_ids,
                     long long units, int kv_heads, int elem_bytes, hipStream_t st) {
  const long long blocks = (units + kShufWaves - 1) / kShufWaves;
  if (elem_bytes == 2)
    hipLaunchKernelGGL((shuffle_kernel<2, kN, kD>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kShufThreads), 0, st, s, k, v, block_ids,
                       static_cast<int>(units), kv_heads);
  else
    hipLaunchKernelGGL((shuffle_kernel<1, kN, kD>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kShufThreads), 0, st, s, k, v, block_ids,
                       static_cast<int>(units), kv_heads);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

template <int kN>
int launch_shuffle_d(const uint8_t* s, uint8_t* k, uint8_t* v, const int32_t* block_ids,
                     long long units, int kv_heads, int head_dim, int elem_bytes,
                     hipStream_t st) {
  if (head_dim == 64)
    return launch_shuffle_n<kN, 64>(s, k, v, block_ids, units, kv_heads, elem_bytes, st);
  if (head_dim == 256)
    return launch_shuffle_n<kN, 256>(s, k, v, block_ids, units, kv_heads, elem_bytes, st);
  if (head_dim == kHeadDim)
    return launch_shuffle_n<kN, kHeadDim>(s, k, v, block_ids, units, kv_heads, elem_bytes, st);
  return SKV_EUNSUPPORTED;
}

}  // namespace

int launch_shuffle(const void* std_cache, void* k_plane, void* v_plane,
                   const int32_t* block_ids, int num_blocks, int kv_heads,
                   int page_size, int head_dim, int elem_bytes, void* stream) {
  const long long units = static_cast<long long>(num_blocks) * kv_heads;
  if (units > 0x7fffffffLL) return SKV_EUNSUPPORTED;
  auto st = static_cast<hipStream_t>(stream);
  auto s = static_cast<const uint8_t*>(std_cache);
  auto k = static_cast<uint8_t*>(k_plane);
  auto v = static_cast<uint8_t*>(v_plane);
  if (page_size == 32)
    return launch_shuffle_d<32>(s, k, v, block_ids, units, kv_heads, head_dim, elem_bytes, st);
  return launch_shuffle_d<16>(s, k, v, block_ids, units, kv_heads, head_dim, elem_bytes, st);
}

}  // namespace skv
