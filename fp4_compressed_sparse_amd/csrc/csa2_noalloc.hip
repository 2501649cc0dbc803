// csa2_layer_group_noalloc: the layer group with its workspace in a fixed device array of
// the library, for callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array lives in this file's device code object, one copy per device, held until the
// process ends.  Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): at the first call on a device, with that device
// current, its address is taken once with hipGetSymbolAddress and kept per device, and
// only that pointer is handed to the kernels as their workspace.  The same one-time set-up
// makes the device's side stream for the SWA branch.  After it, a call makes no
// allocation of any kind.
//
// Every call on a device shares that device's array, which keeps the last call's contents:
// calls that overlap on one device (several host threads, or several streams) race.  No
// kernel of the layer group relies on the workspace starting at zero (the chunked Top-K's
// histograms are cleared by the scoring launch of the same call).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/csa2.h"
#include "csa2_internal.h"

namespace {

constexpr size_t kScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;          // device address of this device's `scratch`
  hipError_t err = hipSuccess;
  csa2::Side side;              // side stream and events; !side.ok: SWA on the caller's stream
};
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

extern "C" csa2_status csa2_layer_group_noalloc(const csa2_layer_desc* L, int32_t n_layers,
                                                const csa2_group_args* g, void* stream) {
  csa2_status st = csa2::layer_group_validate(L, n_layers, g);
  if (st) return st;
  if (g->T == 0) return CSA2_OK;
  const size_t need = csa2_workspace_bytes(CSA2_OP_LAYER_GROUP, g);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg), "csa2_layer_group_noalloc: this group needs %zu workspace "
             "bytes; the static scratch holds %zu (use csa2_layer_group with a workspace)",
             need, kScratchBytes);
    return csa2::set_error(CSA2_ERR_WORKSPACE, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    char msg[256];
    snprintf(msg, sizeof(msg), "csa2_layer_group_noalloc: no usable current device (%s)",
             e != hipSuccess ? hipGetErrorString(e) : "ordinal out of range");
    return csa2::set_error(CSA2_ERR_HIP, msg);
  }
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d] {
    d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess && !d.ptr) d.err = hipErrorInvalidSymbol;
    if (d.err == hipSuccess) (void)csa2::side_create(&d.side);
  });
  if (d.err != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof(msg), "csa2_layer_group_noalloc: hipGetSymbolAddress: %s",
             hipGetErrorString(d.err));
    return csa2::set_error(CSA2_ERR_HIP, msg);
  }
  return csa2::layer_group_run(L, n_layers, g, d.ptr, kScratchBytes,
                               static_cast<hipStream_t>(stream), d.side.ok ? &d.side : nullptr);
}
