// Paged decode attention without a caller-provided workspace: the partials
// (part_o, part_lse) live in a fixed device array of the library, so the call
// allocates nothing. For callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array below is a device symbol: in host code its name stands for a
// host-side shadow, not a device address, so it is never passed to a kernel or
// a copy. Its device address is looked up once per device, with that device
// current, and kept per device; every GPU holds its own copy at its own
// address. Every call on a GPU shares that GPU's copy: calls that overlap on
// one GPU (other streams, other threads) race. Nothing in it needs clearing:
// the segment kernel writes every partial that the reduce then reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
namespace {

static __device__ __align__(256) unsigned char scratch[SKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call
// made with that device current. Returns SKV_OK or SKV_ELAUNCH.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SKV_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SKV_ELAUNCH;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SKV_OK;
}

}  // namespace
}  // namespace skv

extern "C" int skv_paged_decode_attn_static(
    const void* q, const void* kv_a, const void* kv_b, int layout, int kv_dtype,
    const int32_t* page_table, int pt_stride, const int32_t* seq_lens,
    const int32_t* cu_seqlens_q, int bs, int total_q, int max_q, int q_heads,
    int kv_heads, int head_dim, int page_size, const float* k_scale,
    const float* v_scale, int causal, const int32_t* plan, int32_t* tok_nseg,
    int num_cus, int seg_max, void* out, float* out_lse, int flags, void* stream) {
  // the workspace entry point's argument rules (non-NULL stand-ins for the
  // partials, which this call supplies itself), then the size limit
  const int st = skv::check_attn_args(q, kv_a, kv_b, layout, kv_dtype, page_table, pt_stride,
                                      seq_lens, cu_seqlens_q, bs, total_q, max_q, q_heads,
                                      kv_heads, head_dim, page_size, k_scale, v_scale, plan,
                                      tok_nseg, num_cus, seg_max, q, q, out, flags);
  if (st != SKV_OK) return st;
  const size_t need = skv_workspace_bytes(total_q, q_heads, head_dim, seg_max);
  if (need == 0 || need > SKV_STATIC_SCRATCH_BYTES) return SKV_EUNSUPPORTED;
  void* base = nullptr;
  const int sp = skv::scratch_ptr(&base);
  if (sp != SKV_OK) return sp;
  const size_t rows = static_cast<size_t>(total_q) * q_heads * seg_max;
  float* part_o = static_cast<float*>(base);
  float* part_lse = part_o + rows * head_dim;
  return skv_paged_decode_attn(q, kv_a, kv_b, layout, kv_dtype, page_table, pt_stride,
                               seq_lens, cu_seqlens_q, bs, total_q, max_q, q_heads, kv_heads,
                               head_dim, page_size, k_scale, v_scale, causal, plan, tok_nseg,
                               num_cus, seg_max, part_o, part_lse, out, out_lse, flags, stream);
}
