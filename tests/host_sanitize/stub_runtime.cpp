// The handful of HIP runtime calls the C-ABI host code makes, for a build
// that runs without a GPU: code-object registration does nothing, the
// device is 0, the address of the library's device array is a host buffer
// of the same size (only ever passed on to the stub launchers), and the
// device property query reports that there is no device.
#include <stddef.h>

namespace {
alignas(256) unsigned char g_fake_symbol[64];
int g_modules_handle;
}  // namespace

extern "C" {
void** __hipRegisterFatBinary(const void*) { return reinterpret_cast<void**>(&g_modules_handle); }
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
void __hipUnregisterFatBinary(void**) {}
int hipGetDevice(int* device) {
  *device = 0;
  return 0;
}
int hipGetSymbolAddress(void** ptr, const void*) {
  *ptr = g_fake_symbol;
  return 0;
}
const char* hipGetErrorString(int) { return "stub runtime error"; }
// no device to describe: the property query fails (hipErrorNoDevice)
int hipGetDevicePropertiesR0600(void*, int) { return 100; }
int hipGetLastError(void) { return 0; }
}
