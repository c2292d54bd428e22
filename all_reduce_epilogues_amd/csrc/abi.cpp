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

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(AREPI_ELAUNCH, std::string(what) + ": launch failed: " + hipGetErrorString(e));
    return ok();
}

}  // namespace arepi

extern "C" const char *arepi_last_error(void) { return arepi::g_last_error.c_str(); }

extern "C" const char *arepi_version(void) { return "arepi 0.1 gfx950"; }
