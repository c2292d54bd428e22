// abi.cpp -- error reporting shared by every entry point of libarepi.
#include <hip/hip_runtime.h>

#include <string>

#include "arepi_internal.h"

namespace arepi {

static thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

int ok() {
    g_last_error.clear();
    return AREPI_OK;
}

int64_t default_spin_bound() {
    // one second of the device's constant-rate clock, read once per device
    // (100 MHz assumed if the runtime cannot say)
    constexpr int kMaxDevices = 64;
    static int64_t ticks[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -int64_t(100000000);
    if (ticks[dev] == 0) {
        int khz = 0;
        const bool known = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0;
        ticks[dev] = known ? int64_t(khz) * 1000 : int64_t(100000000);
    }
    return -ticks[dev];
}

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(AREPI_ELAUNCH, std::string(what) + ": launch failed: " + hipGetErrorString(e));
    return ok();
}

}  // namespace arepi

extern "C" const char *arepi_last_error(void) { return arepi::g_last_error.c_str(); }

extern "C" const char *arepi_version(void) { return "arepi 0.1 gfx950"; }
