// Cache writer: new tokens' K and V straight into shuffled pages.
//
// vLLM RFC #59111, "NixlConnector: convert standard KV pages to ROCm AITER
// shuffled pages on the decode side", Background and Proposed Change §4: the
// shuffled backend's writer places each token at the slot its slot mapping
// names (block = slot / N, row = slot % N), K as [H, D/x, N, x] and V as
// [H, N/x, D, x] per block, x = 16 / element bytes; padding tokens carry a
// negative slot.
//
// MI355X design (16- or 32-token pages, head dim 64, 128 or 256): one wave64
// per (token, kv head). The token's K row is D*e bytes = D/x chunks of 16
// bytes (at most 32), and each chunk lands whole in the K plane (x
// consecutive channels of one row), so lanes 0 .. D/x-1 move one 16-byte
// chunk each. In the V plane consecutive tokens of one channel share a
// 16-byte chunk, so a token's V row scatters: lane l writes channels 2l and
// 2l+1 (e bytes each) at stride x*e, and channels 128 + 2l, 128 + 2l + 1 at
// head dim 256. Tokens of one block write disjoint bytes,
// so concurrent waves need no ordering. Decode steps write few tokens; the
// kernel is launch-bound, not bandwidth-bound. With per-tensor scales, bf16
// rows are quantised into an fp8 cache on the way (the RFC leaves the fp8
// writer's scale handling to its own treatment; the reading here is
// code = e4m3fn(value / scale), the inverse of the attention path's
// value = code * scale).
#include <hip/hip_runtime.h>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int E, int kN, int kD>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    const int64_t* __restrict__ slots, int num_tokens, long long key_stride,
    long long value_stride, uint8_t* __restrict__ kp, uint8_t* __restrict__ vp,
    int kv_heads, long long num_slots) {
  constexpr int kX = 16 / E;
  constexpr int kKChunks = kD * E / 16;
  constexpr size_t kPlane = static_cast<size_t>(kN) * kD * E;   // one head of one block
  const int lane = threadIdx.x & 63;
  const long long unit = static_cast<long long>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (unit >= static_cast<long long>(num_tokens) * kv_heads) return;   // wave-uniform
  const int t = static_cast<int>(unit / kv_heads);
  const int h = static_cast<int>(unit % kv_heads);
  const long long slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;                           // padding / out of range
  const long long b = slot / kN;
  const int n = static_cast<int>(slot % kN);
  const size_t head = static_cast<size_t>(b) * kv_heads + h;
  const uint8_t* krow = key + (t * key_stride + static_cast<long long>(h) * kD) * E;
  const uint8_t* vrow = value + (t * value_stride + static_cast<long long>(h) * kD) * E;
  uint8_t* kdst = kp + head * kPlane;
  uint8_t* vdst = vp + head * kPlane;
  // K: chunk c1 (channels c1*x .. c1*x + x-1) -> k_plane[b, h, c1, n, :]
  if (lane < kKChunks) {
    const uint4 v = *reinterpret_cast<const uint4*>(krow + 16 * lane);
    *reinterpret_cast<uint4*>(kdst + (static_cast<size_t>(lane) * kN + n) * 16) = v;
  }
  // V: channel d -> v_plane[b, h, n / x, d, n % x]
  const size_t vbase = static_cast<size_t>(n / kX) * kD * kX + n % kX;
#pragma unroll
  for (int d = 2 * lane; d < kD; d += 128) {
    if constexpr (E == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(vrow + 2 * d);
      reinterpret_cast<uint16_t*>(vdst)[vbase + static_cast<size_t>(d) * kX] =
          static_cast<uint16_t>(w);
      reinterpret_cast<uint16_t*>(vdst)[vbase + static_cast<size_t>(d + 1) * kX] =
          static_cast<uint16_t>(w >> 16);
    } else {
      const uint16_t w = *reinterpret_cast<const uint16_t*>(vrow + d);
      vdst[vbase + static_cast<size_t>(d) * kX] = static_cast<uint8_t>(w);
      vdst[vbase + static_cast<size_t>(d + 1) * kX] = static_cast<uint8_t>(w >> 8);
    }
  }
}

// fp32 -> OCP e4m3fn code: round to nearest, ties to even; magnitudes at or
// above 448 (infinity included) saturate to +-448; NaN stays NaN; the sign of
// zero is kept. Integer rounding of the fp32 mantissa for the normal range
// (>= 2^-6); below it the code counts 2^-9 steps, so v * 512 (exact) is
// rounded to an integer, half to even.
__device__ __forceinline__ uint32_t e4m3fn_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;            // 448.0f
  const uint32_t e = a >> 23;
  if (e >= 121u) {                                      // 2^-6: first normal e4m3fn exponent
    const uint32_t m = a & 0x7fffffu;
    uint32_t q = m >> 20;
    const uint32_t rem = m & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    return sign | (((e - 120u) << 3) + q);              // a carry moves into the exponent
  }
  return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
}

// bf16 K/V rows quantised into an fp8 cache: code = e4m3fn(value / scale),
// the division in fp32. Same placement as cache_write_kernel<1, kN, kD>.
template <int kN, int kD>
__global__ __launch_bounds__(kThreads) void cache_write_quant_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    const int64_t* __restrict__ slots, int num_tokens, long long key_stride,
    long long value_stride, uint8_t* __restrict__ kp, uint8_t* __restrict__ vp,
    int kv_heads, long long num_slots, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  constexpr int kX = 16;
  constexpr int kKChunks = kD / 16;
  constexpr size_t kPlane = static_cast<size_t>(kN) * kD;
  const int lane = threadIdx.x & 63;
  const long long unit = static_cast<long long>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (unit >= static_cast<long long>(num_tokens) * kv_heads) return;   // wave-uniform
  const int t = static_cast<int>(unit / kv_heads);
  const int h = static_cast<int>(unit % kv_heads);
  const long long slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const long long b = slot / kN;
  const int n = static_cast<int>(slot % kN);
  const size_t head = static_cast<size_t>(b) * kv_heads + h;
  const uint16_t* krow = key + t * key_stride + static_cast<long long>(h) * kD;
  const uint16_t* vrow = value + t * value_stride + static_cast<long long>(h) * kD;
  const float ks = *k_scale, vs = *v_scale;
  if (lane < kKChunks) {
    // 16 channels -> one 16-byte K chunk
    const uint4 lo = reinterpret_cast<const uint4*>(krow + 16 * lane)[0];
    const uint4 hi = reinterpret_cast<const uint4*>(krow + 16 * lane)[1];
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = w[2 * q], bb = w[2 * q + 1];
      c[q] = e4m3fn_rne_sat(__uint_as_float(a << 16) / ks) |
             (e4m3fn_rne_sat(__uint_as_float(a & 0xffff0000u) / ks) << 8) |
             (e4m3fn_rne_sat(__uint_as_float(bb << 16) / ks) << 16) |
             (e4m3fn_rne_sat(__uint_as_float(bb & 0xffff0000u) / ks) << 24);
    }
    *reinterpret_cast<uint4*>(kp + head * kPlane + (static_cast<size_t>(lane) * kN + n) * 16) =
        make_uint4(c[0], c[1], c[2], c[3]);
  }
  const size_t vbase = static_cast<size_t>(n / kX) * kD * kX + n % kX;
  uint8_t* vdst = vp + head * kPlane;
#pragma unroll
  for (int d = 2 * lane; d < kD; d += 128) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(vrow + d);
    vdst[vbase + static_cast<size_t>(d) * kX] =
        static_cast<uint8_t>(e4m3fn_rne_sat(__uint_as_float(w << 16) / vs));
    vdst[vbase + static_cast<size_t>(d + 1) * kX] =
        static_cast<uint8_t>(e4m3fn_rne_sat(__uint_as_float(w & 0xffff0000u) / vs));
  }
}

}  // namespace

namespace {

template <int kD>
int launch_cache_write_d(const void* key, const void* value, const int64_t* slot_mapping,
                         int num_tokens, long long key_stride, long long value_stride,
                         uint8_t* kp, uint8_t* vp, int kv_heads, long long num_slots,
                         int page_size, int elem_bytes, const float* k_scale,
                         const float* v_scale, dim3 grid, hipStream_t st) {
  const dim3 block(kThreads);
  auto k = static_cast<const uint8_t*>(key);
  auto v = static_cast<const uint8_t*>(value);
  if (k_scale) {
    auto kq = static_cast<const uint16_t*>(key);
    auto vq = static_cast<const uint16_t*>(value);
    if (page_size == 32)
      hipLaunchKernelGGL((cache_write_quant_kernel<32, kD>), grid, block, 0, st, kq, vq,
                         slot_mapping, num_tokens, key_stride, value_stride, kp, vp,
                         kv_heads, num_slots, k_scale, v_scale);
    else
      hipLaunchKernelGGL((cache_write_quant_kernel<16, kD>), grid, block, 0, st, kq, vq,
                         slot_mapping, num_tokens, key_stride, value_stride, kp, vp,
                         kv_heads, num_slots, k_scale, v_scale);
    return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
  }
#define SKV_W(E, N)                                                                      \
  hipLaunchKernelGGL((cache_write_kernel<E, N, kD>), grid, block, 0, st, k, v, slot_mapping, \
                     num_tokens, key_stride, value_stride, kp, vp, kv_heads, num_slots)
  if (page_size == 32) {
    if (elem_bytes == 2) SKV_W(2, 32); else SKV_W(1, 32);
  } else {
    if (elem_bytes == 2) SKV_W(2, 16); else SKV_W(1, 16);
  }
#undef SKV_W
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // namespace

int launch_cache_write(const void* key, const void* value, const int64_t* slot_mapping,
                       int num_tokens, long long key_stride, long long value_stride,
                       void* k_plane, void* v_plane, int num_blocks, int kv_heads,
                       int page_size, int head_dim, int elem_bytes, const float* k_scale,
                       const float* v_scale, void* stream) {
  const long long units = static_cast<long long>(num_tokens) * kv_heads;
  const long long blocks = (units + kWaves - 1) / kWaves;
  if (blocks > 0x7fffffffLL) return SKV_EUNSUPPORTED;
  const long long num_slots = static_cast<long long>(num_blocks) * page_size;
  auto st = static_cast<hipStream_t>(stream);
  auto kp = static_cast<uint8_t*>(k_plane);
  auto vp = static_cast<uint8_t*>(v_plane);
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (head_dim) {
    case 64:
      return launch_cache_write_d<64>(key, value, slot_mapping, num_tokens, key_stride,
                                      value_stride, kp, vp, kv_heads, num_slots, page_size,
                                      elem_bytes, k_scale, v_scale, grid, st);
    case 128:
      return launch_cache_write_d<128>(key, value, slot_mapping, num_tokens, key_stride,
                                       value_stride, kp, vp, kv_heads, num_slots, page_size,
                                       elem_bytes, k_scale, v_scale, grid, st);
    case 256:
      return launch_cache_write_d<256>(key, value, slot_mapping, num_tokens, key_stride,
                                       value_stride, kp, vp, kv_heads, num_slots, page_size,
                                       elem_bytes, k_scale, v_scale, grid, st);
    default:
      return SKV_EUNSUPPORTED;
  }
}

}  // namespace skv
