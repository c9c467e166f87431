// tree_attn_verify_noalloc: tree_attn_verify for callers that cannot allocate
// (graph capture, tight serving loops).  The split-KV partial results live in
// a fixed device array of this library instead of a caller workspace; the
// kernels and the plan are tree_attn_verify's own.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ta_internal.h"
#include "tree_attn.h"

namespace {

// One copy per GPU, held until the process ends.  In host code `scratch` names
// a host-side stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[TA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Supplies the current device's scratch array for a plan that needs `need`
// bytes.  The address is looked up once per device (with that device current)
// and kept.  Rejects plans larger than the array before touching the device.
int device_scratch(size_t need, void* stream, void** ws) {
  if (need > TA_NOALLOC_SCRATCH_BYTES) return TA_ERR_SCRATCH;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    ta::set_last_error(e, "tree_attn_verify_noalloc: hipGetDevice");
    return TA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return TA_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) {
      ta::set_last_error(e, "tree_attn_verify_noalloc: hipStreamGetDevice");
      return TA_ERR_HIP;
    }
    if (sdev != dev) return TA_ERR_INVALID_ARG;  // the stream must be on the current device
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      ta::set_last_error(e != hipSuccess ? e : hipErrorInvalidSymbol,
                         "tree_attn_verify_noalloc: hipGetSymbolAddress(scratch)");
      return TA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ws = g_scratch_ptr[dev];
  return TA_OK;
}

}  // namespace

extern "C" int tree_attn_verify_noalloc(const void* q, ta_kv kv, const int32_t* prefix_len,
                                        const int32_t* parent, const int32_t* n_nodes, int B,
                                        int n_max, int Hq, int Hkv, int d, int dtype, float scale,
                                        void* out, float* lse, const ta_attn_opts* opts,
                                        void* stream) {
  return ta::run_attention(q, kv, prefix_len, parent, n_nodes, B, n_max, n_max, 0, Hq, Hkv, d,
                           dtype, scale, out, lse, nullptr, 0, opts, stream, device_scratch,
                           nullptr);
}
