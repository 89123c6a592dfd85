// noalloc.hip -- ls_gdn_frame_forward_noalloc: the frame-wise GDN scan for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  Its workspace is
// the file-scope device array `scratch`, which every GPU the library runs on
// holds (at its own address) until the process ends.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "../../include/linscan.h"

namespace linscan {
ls_status set_error(ls_status st, const char* msg);
ls_status gdn_forward_plain(const ls_shape* s, float key_scale, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, void* o, const float* state_in, float* state_out,
                            void* workspace, size_t workspace_bytes, uint32_t* fault, void* stream);
}  // namespace linscan

namespace {

// In host code `scratch` names a host-side stand-in, not device memory: only
// the address hipGetSymbolAddress returns for the current device is used.
static __device__ __align__(256) uint8_t scratch[LS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device.
ls_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  char msg[160];
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
    return linscan::set_error(LS_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof(msg), "device index %d is not below %d", dev, kMaxDevices);
    return linscan::set_error(LS_ERR_INTERNAL, msg);
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return linscan::set_error(LS_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LS_OK;
}

}  // namespace

extern "C" ls_status ls_gdn_frame_forward_noalloc(const ls_shape* shape, float key_scale, const void* q, const void* k,
                                                  const void* v, const float* alpha, const float* beta, void* o,
                                                  const float* state_in, float* state_out, unsigned int* fault_word,
                                                  void* stream) {
  // host-only checks first: an invalid shape (size 0) is reported by the
  // shared checks below without a workspace; a valid one must fit
  const size_t need = ls_gdn_frame_workspace_size(shape);
  if (need > LS_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    snprintf(msg, sizeof(msg), "this call needs %zu bytes of scratch; the static scratch holds %zu",
             need, (size_t)LS_NOALLOC_SCRATCH_BYTES);
    return linscan::set_error(LS_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  if (((uintptr_t)fault_word & 3u) != 0) return linscan::set_error(LS_ERR_MISALIGNED, "fault_word must be 4-byte aligned");
  void* ws = nullptr;
  if (need > 0) {
    const ls_status st = scratch_on_current_device(&ws);
    if (st != LS_OK) return st;
  }
  return linscan::gdn_forward_plain(shape, key_scale, q, k, v, alpha, beta, o, state_in, state_out, ws,
                                    ws ? (size_t)LS_NOALLOC_SCRATCH_BYTES : 0, (uint32_t*)fault_word, stream);
}
