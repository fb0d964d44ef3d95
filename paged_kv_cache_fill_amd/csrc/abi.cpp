// abi.cpp -- status plumbing of the C ABI (pkv_last_error, pkv_version).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv_internal.h"

namespace pkv {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

int check_launch(const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

extern "C" const char* pkv_version(void) { return "0.1.0"; }
