// mla_absorb_attn_noalloc: mla_absorb_attn for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The workspace
// (absorbed query, split statistics and partial rows) lives in one file-scope device array of a
// fixed size instead of a caller buffer; every other argument, the kernels and the results are
// those of mla_absorb_attn.
#include <hip/hip_runtime.h>

#include <stdio.h>

#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // MLA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == MLA_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");

// One copy per GPU, held until the process ends.  In host code this name is a host-side stand-in,
// not a device address: kernels get the address hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's copy of the scratch array (looked up once per device, with that device
// current).
int32_t scratch_for_current_device(void **ptr) {
  char msg[192];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof(msg), "no usable current HIP device (hipGetDevice: %s, device %d)", hipGetErrorName(e), dev);
    return mla::set_error(MLA_ERR_HIP, msg);
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
               hipGetErrorName(e));
      return mla::set_error(MLA_ERR_HIP, msg);
    }
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_absorb_attn_noalloc(const void *q_nope, const void *q_pe, const void *kv_cache, const void *pe_cache,
                                const void *wkv_b, int64_t end_pos, float softmax_scale, void *out,
                                const mla_attn_shape *shape, int32_t dtype, const mla_attn_options *options,
                                void *stream) {
  size_t need = 0;
  int32_t rc = mla::absorb_attn_dry_run(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos, softmax_scale, out, shape,
                                        dtype, options, &need);
  if (rc != MLA_OK) return rc;
  if (need > kScratchBytes) {
    char msg[192];
    snprintf(msg, sizeof(msg), "this call needs %zu bytes of workspace; the no-allocation entry point holds %zu",
             need, kScratchBytes);
    return mla::set_error(MLA_ERR_WORKSPACE, msg);
  }
  void *ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc != MLA_OK) return rc;
  return mla_absorb_attn(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos, softmax_scale, out, shape, dtype, options,
                         ws, kScratchBytes, stream);
}

}  // extern "C"
