// C ABI plumbing: version, last-error storage and shared argument checks.
#include <stdarg.h>
#include <stdio.h>

#include "abi_util.h"

namespace moe {

static thread_local char g_last_error[512] = "";

int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

int check_launch(const char* what) {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    return MOE_OK;
}

int ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done, const char* what) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return MOE_OK;
    err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    done.fetch_or(bit, std::memory_order_release);
    return MOE_OK;
}

int device_cu_count(const char* what) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    int n = cached[dev & 63].load(std::memory_order_relaxed);
    if (n > 0) return n;
    err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    cached[dev & 63].store(n, std::memory_order_relaxed);
    return n;
}

bool valid_block_m(int32_t block_m) {
    return block_m == 16 || block_m == 32 || block_m == 64 || block_m == 128 || block_m == 256;
}

int check_shape(const char* fn, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I) {
    if (T < 0 || H < 0 || E < 0 || k < 0) return set_error(MOE_ERR_INVALID, "%s: negative size", fn);
    if (E < 1 || E > kMaxExperts)
        return set_error(MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1, %d]", fn, E, kMaxExperts);
    if (k < 1 || k > E || k > kMaxTopK)
        return set_error(MOE_ERR_UNSUPPORTED, "%s: k=%d outside [1, min(E=%d, %d)]", fn, k, E, kMaxTopK);
    if (H != 0 && (H % 64 != 0)) return set_error(MOE_ERR_UNSUPPORTED, "%s: H=%d is not a multiple of 64", fn, H);
    if (H == 0) return set_error(MOE_ERR_UNSUPPORTED, "%s: H must be positive", fn);
    if (I >= 0 && (I == 0 || I % 32 != 0))
        return set_error(MOE_ERR_UNSUPPORTED, "%s: I=%d is not a positive multiple of 32", fn, I);
    if (T * (int64_t)k >= ((int64_t)1 << 31))
        return set_error(MOE_ERR_UNSUPPORTED, "%s: T*k=%lld does not fit int32 indices", fn, (long long)(T * k));
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char* moe_last_error(void) { return moe::g_last_error; }
