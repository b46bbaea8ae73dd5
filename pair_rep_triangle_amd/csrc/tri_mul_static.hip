// The allocation-free forward call (tri_mul_forward_static in include/tri_mul.h): the same
// three kernels as tri_mul_forward, with the a | b | x workspace taken from a file-scope
// device array instead of a caller buffer.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address
// on each GPU comes from hipGetSymbolAddress, looked up once per device (at tri_mul_create
// on the handle's device, or at the first static call there) and cached. Only that address
// is ever passed to the kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "host_common.h"
#include "tri_mul.h"

static __device__ __align__(256) unsigned char scratch[TRI_MUL_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_slots[kMaxDevices];

}  // namespace

namespace trimul_host {

// The device address of this library's static workspace on device `dev` (which must be the
// current device), looked up on the first call for that device.
int static_workspace(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return TRI_MUL_ERR_UNSUPPORTED_DEVICE;
  ScratchSlot& s = g_slots[dev];
  std::call_once(s.once, [&] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess) s.ptr = p;
  });
  if (s.err != hipSuccess) return hip_fail(s.err, "hipGetSymbolAddress(static workspace)");
  *ptr = s.ptr;
  return TRI_MUL_OK;
}

}  // namespace trimul_host

extern "C" int tri_mul_forward_static(tri_mul_handle* h, const void* z, const void* pair_mask,
                                      void* out, int batch, int n, int direction,
                                      void* stream) {
  size_t need = 0;
  int rc = tri_mul_workspace_bytes(h, batch, n, &need);
  if (rc != TRI_MUL_OK) return rc;
  if (need > (size_t)TRI_MUL_STATIC_WORKSPACE_BYTES) return TRI_MUL_ERR_WORKSPACE_TOO_SMALL;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return trimul_host::hip_fail(e, "hipGetDevice");
  void* ws = nullptr;
  rc = trimul_host::static_workspace(dev, &ws);
  if (rc != TRI_MUL_OK) return rc;
  return tri_mul_forward(h, z, pair_mask, out, batch, n, direction, ws,
                         (size_t)TRI_MUL_STATIC_WORKSPACE_BYTES, stream);
}
