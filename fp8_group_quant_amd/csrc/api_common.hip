// api_common.hip — status strings, thread-local error detail and the device check of
// the C ABI (include/fp8q.h).
#include <atomic>
#include <cstring>

#include "fp8q_internal.h"

namespace fp8q {

namespace {
thread_local std::string g_last_error;
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_device_cus[kMaxDevices];
std::atomic<int> g_device_xcds[kMaxDevices];
}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

static int query_device(int device) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count)
    return fail(FP8Q_EDEVICE, "no HIP device " + std::to_string(device));
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess)
    return fail(FP8Q_EDEVICE, "cannot query HIP device " + std::to_string(device));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(FP8Q_EDEVICE, std::string("device is ") + prop.gcnArchName + ", this library targets gfx950");
  int xcds = 1;
  if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, device) != hipSuccess || xcds < 1) xcds = 1;
  if (device < kMaxDevices) {
    g_device_cus[device].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1, std::memory_order_relaxed);
    g_device_xcds[device].store(xcds, std::memory_order_relaxed);
  }
  return FP8Q_OK;
}

int check_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(FP8Q_EDEVICE, "no current HIP device");
  if (dev < kMaxDevices) {
    const int st = g_device_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return FP8Q_OK;
    if (st == 2) return fail(FP8Q_EDEVICE, "current device is not a gfx950");
  }
  const int rc = query_device(dev);
  if (dev < kMaxDevices) g_device_state[dev].store(rc == FP8Q_OK ? 1 : 2, std::memory_order_relaxed);
  return rc;
}

DeviceShape current_device_shape() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DeviceShape{256, 8};
  const int cus = g_device_cus[dev].load(std::memory_order_relaxed);
  const int xcds = g_device_xcds[dev].load(std::memory_order_relaxed);
  return DeviceShape{cus > 0 ? cus : 256, xcds > 0 ? xcds : 8};
}

}  // namespace fp8q

extern "C" {

const char* fp8q_status_string(int status) {
  switch (status) {
    case FP8Q_OK: return "FP8Q_OK";
    case FP8Q_EINVAL: return "FP8Q_EINVAL: invalid argument (pointer, shape, stride or layout)";
    case FP8Q_EUNSUPPORTED: return "FP8Q_EUNSUPPORTED: dtype, group size, scale format or mode not supported";
    case FP8Q_EALIGN: return "FP8Q_EALIGN: pointer or row stride not aligned as required";
    case FP8Q_EDEVICE: return "FP8Q_EDEVICE: no gfx950 device";
    case FP8Q_ELAUNCH: return "FP8Q_ELAUNCH: kernel launch failed";
    default: return "unknown fp8q status";
  }
}

const char* fp8q_last_error(void) { return fp8q::g_last_error.c_str(); }

int fp8q_device_check(int device) { return fp8q::query_device(device); }

}  // extern "C"
