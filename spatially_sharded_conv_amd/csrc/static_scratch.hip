// Band decode that allocates nothing: its workspace is a file-scope device array.
//
// vaep_decode_bands_noalloc runs exactly the kernels of vaep_decode_bands; the workspace
// those kernels use (activation buffers, Q/K/V, statistics records) is `scratch` below
// instead of a caller-supplied buffer.  Each GPU the library runs on holds its own copy of
// the array (kScratchBytes) until the process ends.  In host code the array's name is only
// a host-side stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is handed to the
// kernels.  No part of the decode needs the workspace to start at zero: every region is
// written before it is read.
#include "vaep_internal.h"

#include <cstdio>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's `scratch`, looked up on the first call per device.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[160];
    std::snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
    return vaep::set_error(VAEP_ERR_NOT_READY, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) return vaep::set_error(VAEP_ERR_UNSUPPORTED, "device ordinal beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return vaep::set_error(VAEP_ERR_HIP, msg);
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return VAEP_OK;
}

}  // namespace

extern "C" {

size_t vaep_noalloc_scratch_bytes(void) { return kScratchBytes; }

int vaep_decode_bands_noalloc(vaep_model* model, const void* latent, int batch, int frames, int latent_h,
                              int latent_w, const int32_t* row_starts, int n_bands, void* out, void* stream,
                              vaep_decode_info* info) {
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  rc = vaep_decode_bands(model, latent, batch, frames, latent_h, latent_w, row_starts, n_bands, out, ws,
                         kScratchBytes, stream, info);
  if (rc == VAEP_ERR_WORKSPACE) {
    char msg[256];
    std::snprintf(msg, sizeof(msg),
                  "vaep_decode_bands_noalloc: this decode needs more than the %zu MiB static scratch (%s); "
                  "use vaep_decode_bands with a workspace",
                  kScratchBytes >> 20, vaep_last_error());
    return vaep::set_error(VAEP_ERR_WORKSPACE, msg);
  }
  return rc;
}

}  // extern "C"
