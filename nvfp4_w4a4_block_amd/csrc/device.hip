// Per-device set-up of the library: once per device, on the first call that launches work on
// it, from whichever host thread makes that call.  std::call_once makes concurrent first calls
// safe: one thread runs the set-up while the others wait for it.  The device is the one the
// caller's stream belongs to, not the calling thread's current device.
#include <mutex>

#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kMaxDevices = 64;

struct DeviceSlot {
  std::once_flag once;
  int status = NVFP4_ERR_HIP;
  DeviceInfo info{};
};

DeviceSlot g_devices[kMaxDevices];

// Runs with device `dev` current (restoring the caller's device afterwards): the kernel files'
// own set-up steps, then the compute-unit count.
int setup_device(int dev, DeviceInfo& info) {
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return NVFP4_ERR_HIP;
  if (prev != dev && hipSetDevice(dev) != hipSuccess) return NVFP4_ERR_HIP;
  int st = gemm_device_setup();
  if (st == NVFP4_OK) st = quantize_device_setup(&info.quant_scratch);
  if (st == NVFP4_OK &&
      (hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || info.cus <= 0))
    st = NVFP4_ERR_HIP;
  if (prev != dev && hipSetDevice(prev) != hipSuccess) st = NVFP4_ERR_HIP;
  return st;
}

}  // namespace

int device_info(hipStream_t stream, DeviceInfo& info) {
  int dev = 0;
  const hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return NVFP4_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  DeviceSlot& s = g_devices[dev];
  std::call_once(s.once, [&] { s.status = setup_device(dev, s.info); });
  if (s.status != NVFP4_OK) return s.status;
  info = s.info;
  return NVFP4_OK;
}

}  // namespace nvfp4
