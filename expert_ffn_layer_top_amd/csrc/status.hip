// Status codes, per-thread last-error text and the shared shape rules of the C ABI.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

#include "common.h"

namespace moe {

static thread_local char g_last_error[512] = "";

int set_error(int st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int gemm_workgroups(long long tiles_upper) {
  long long g = (tiles_upper + 7) / 8 * 8;
  long long cap = cu_count() / 8 * 8;
  if (const char* env = getenv("MOE_GG_WORKGROUPS")) {
    const long long v = atoll(env) / 8 * 8;
    if (v >= 8 && v < cap) cap = v;
  }
  if (cap < 8) cap = 8;
  return static_cast<int>(g < cap ? g : cap);
}

int check_layer_shape(int T, int E, int k) {
  MOE_REQUIRE(T >= 1, MOE_ERR_UNSUPPORTED, "T must be >= 1 (got %d)", T);
  MOE_REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "E must be in [1, 256] (got %d)", E);
  MOE_REQUIRE(k >= 1 && k <= E && k <= 16, MOE_ERR_UNSUPPORTED, "k must be in [1, min(E, 16)] (got %d)", k);
  MOE_REQUIRE(static_cast<long long>(T) * k < (1LL << 31), MOE_ERR_UNSUPPORTED, "T*k must be < 2^31");
  return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_MI355X_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* moe_last_error_string(void) { return moe::g_last_error; }

}  // extern "C"
