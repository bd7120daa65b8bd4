// fsdp_internal.h -- status and dtype helpers shared by the host-side sources
// of libfsdp_shard.so (fsdp_abi.cpp, fsdp_ckpt.cpp).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsdp {

// Record a message for fsdp_last_error() and return `code` (negative).
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return FSDP_OK.
int ok();
// FSDP_E_HIP with the runtime's description of `e`.
int hip_fail(hipError_t e, const char* what);
bool valid_dtype(int dt);
int64_t dt_size(int dt);
const char* last_error();

}  // namespace fsdp
