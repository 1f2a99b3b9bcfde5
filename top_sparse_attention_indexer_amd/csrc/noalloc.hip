// dsa_fused_forward without a caller workspace: the scratch memory comes from
// a fixed device array of this library, so the call allocates nothing (for
// callers that cannot allocate: code under graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array is a file-scope device global; its host-side name is only a
// stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (on the first call made on that device, with the
// device current) and that address is what the kernels receive.  Every call
// on a device shares the device's array and leaves its contents behind;
// the kernels clear or epoch-tag everything they read before writing it.
// Calls that overlap on one device (two streams, two threads) race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[64] = {};   // device address of `scratch`, per device

}  // namespace

extern "C" {

dsa_status dsa_fused_forward_noalloc(const dsa_problem* p, const void* q_idx, const void* k_idx,
                                     const void* q, const void* k, const void* v,
                                     const float* gate, const float* y2, const uint8_t* route,
                                     float* out, int32_t* topk_idx_out, void* stream) {
  size_t need = 0;
  dsa_status st = dsa::fused_ws_need(p, &need);
  if (st != DSA_OK) return st;
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "the problem needs %zu bytes of scratch; the no-allocation entry point holds at "
             "most %zu (use dsa_fused_forward with a workspace)",
             need, kScratchBytes);
    return dsa::report(DSA_ERR_WORKSPACE, msg);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return dsa::report(DSA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return dsa::report(DSA_ERR_UNSUPPORTED, "device ordinal above 63");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
      // set-up on this device: the array's device address, and what a first
      // decode launch would otherwise create
      void* addr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !addr) {
        char msg[256];
        snprintf(msg, sizeof(msg), "hipGetSymbolAddress of the scratch array: %s",
                 hipGetErrorString(e));
        return dsa::report(DSA_ERR_HIP, msg);
      }
      if (dsa::decode_setup() != hipSuccess)
        return dsa::report(DSA_ERR_HIP, "creating the decode ordering event failed");
      g_ptr[dev] = addr;
    }
    ptr = g_ptr[dev];
  }
  return dsa_fused_forward(p, q_idx, k_idx, q, k, v, gate, y2, route, out, topk_idx_out, ptr,
                           kScratchBytes, stream);
}

}  // extern "C"
