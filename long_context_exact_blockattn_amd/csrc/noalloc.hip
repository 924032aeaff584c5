// Allocation-free variant of the backward entry point: the delta rows live in a
// static device buffer of the library instead of a caller's workspace argument.
#include "../../include/blockattn.h"

#include <hip/hip_runtime.h>

#include <mutex>

int ba_bwd_impl(const ba_desc* d, const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, float* delta, float* dq_acc, void* dk, void* dv,
                int32_t dkv_dtype, void* dq_final, int32_t flags, hipStream_t stream);

namespace {

// One copy per GPU, allocated when the code object is loaded.  In host code the
// name is only a handle for hipGetSymbolAddress: the device address is looked
// up once per device and every use goes through that address.
static __device__ __align__(256) float scratch[BLOCKATTN_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];  // device address of `scratch`, per device (null: not looked up yet)

int scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BA_ERR_WORKSPACE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BA_ERR_WORKSPACE;
    g_addr[dev] = p;
  }
  *out = (float*)g_addr[dev];
  return BA_OK;
}

}  // namespace

extern "C" int blockattn_bwd_noalloc(const ba_desc* desc, const void* q, const void* k, const void* v,
                                     const void* o, const void* dout, const float* lse, float* dq_acc,
                                     void* dk, void* dv, int32_t dkv_dtype, void* dq_final, int32_t flags,
                                     hipStream_t stream) {
  if (!desc) return BA_ERR_NULL;
  if (desc->batch < 0 || desc->heads_q < 1 || desc->seqlen_q < 0) return BA_ERR_SHAPE;
  if ((int64_t)desc->batch * desc->heads_q > BLOCKATTN_NOALLOC_MAX_ROWS ||
      (int64_t)desc->batch * desc->heads_q * desc->seqlen_q > BLOCKATTN_NOALLOC_MAX_ROWS)
    return BA_ERR_WORKSPACE;
  if (flags & ~(BA_BWD_COMPUTE_DELTA | BA_BWD_FINALIZE_DQ)) return BA_ERR_MODE;
  float* delta = nullptr;
  const int r = scratch_address(&delta);
  if (r) return r;
  return ba_bwd_impl(desc, q, k, v, o, dout, lse, delta, dq_acc, dk, dv, dkv_dtype, dq_final,
                     flags | BA_BWD_COMPUTE_DELTA, stream);
}
