// Host-side helpers for the C ABI: thread-local error message, argument
// checks, launch error capture.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "moe_mi355x.h"

namespace moe {

// Records a printf-style message for moe_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// After a launch: MOE_OK, or MOE_ERR_HIP with the HIP error string.
int check_launch(const char* what);

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 32;

// Raises `kernel`'s dynamic LDS limit to `bytes` (HIP's default is 64 KB)
// once per device; `done` is the call site's mask of devices already set
// (thread-safe: a race only repeats the idempotent attribute call).
int ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done, const char* what);

// Compute units of the current device (cached per device), or a negative
// MOE_ERR_HIP code with the message set.
int device_cu_count(const char* what);

// Shared limits on (T, H, E, k, I); I < 0 means "not used by this call".
int check_shape(const char* fn, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I);
bool valid_block_m(int32_t block_m);

}  // namespace moe
