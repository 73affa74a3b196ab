// hip_stub.cpp -- host-only stand-ins for the HIP runtime calls and kernel
// launchers that attn_api.cpp makes, so that its argument checks, device check
// and parameter folding can run under AddressSanitizer/UBSan on a machine
// without a GPU. Test infrastructure only: never linked into the library.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "attn_launch.h"
#include "attn_params.h"

namespace {
int g_device = 0;
int g_launches = 0;
fbc::AttnParams g_last;
int g_last_kind = -1, g_last_dqk = 0, g_last_mode = 0, g_last_grid = 0;
}  // namespace

extern "C" {
// the architecture the stubbed device reports: STUB_ARCH, default gfx950
hipError_t hipGetDevice(int* d) {
  *d = g_device;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int) {
  std::memset(prop, 0, sizeof *prop);
  const char* arch = std::getenv("STUB_ARCH");
  std::strncpy(prop->gcnArchName, arch ? arch : "gfx950", sizeof prop->gcnArchName - 1);
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }

void stub_set_device(int d) { g_device = d; }
int stub_launches(void) { return g_launches; }
const fbc::AttnParams* stub_last_params(void) { return &g_last; }
int stub_last_kind(void) { return g_last_kind; }
int stub_last_grid(void) { return g_last_grid; }
int stub_last_mode(void) { return g_last_mode; }
int stub_last_dqk(void) { return g_last_dqk; }
}

namespace fbc {
hipError_t launch_attn_fwd_fp8(const AttnParams& p, int dqk, int mode, int grid, hipStream_t) {
  ++g_launches;
  g_last = p;
  g_last_kind = 1;
  g_last_dqk = dqk;
  g_last_mode = mode;
  g_last_grid = grid;
  return hipSuccess;
}
hipError_t launch_attn_fwd_bf16(const AttnParams& p, int dqk, int grid, hipStream_t) {
  ++g_launches;
  g_last = p;
  g_last_kind = 0;
  g_last_dqk = dqk;
  g_last_mode = 0;
  g_last_grid = grid;
  return hipSuccess;
}
hipError_t launch_quantize_e4m3(const void*, void*, float*, int64_t, int, int, hipStream_t) {
  ++g_launches;
  g_last_kind = 2;
  return hipSuccess;
}
}  // namespace fbc
