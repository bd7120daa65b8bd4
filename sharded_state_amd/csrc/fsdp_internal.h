// fsdp_internal.h -- status, dtype and optimizer-scalar helpers shared by the
// host-side sources of libfsdp_shard.so (fsdp_abi.cpp, fsdp_ckpt.cpp,
// fsdp_offload.cpp).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fsdp_kernels.h"
#include "fsdp_shard.h"

namespace fsdp {

// Largest element count of a unit, a shard times the world, or any buffer the
// library addresses: below it, an element count times 16 bytes still fits an
// int64, so no byte offset or alias check can wrap.  Larger sizes are refused
// with FSDP_E_SIZE.
constexpr int64_t kMaxElems = INT64_MAX / 16;

// Record a message for fsdp_last_error() and return `code` (negative).
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return FSDP_OK.
int ok();
// FSDP_E_HIP with the runtime's description of `e`.
int hip_fail(hipError_t e, const char* what);
bool valid_dtype(int dt);
int64_t dt_size(int dt);
const char* last_error();
// AdamW constants of step hp->step, computed in double and rounded once to fp32
// (decay = 1 - lr*wd, step_size = lr / (1 - beta1^t), bc2_sqrt = sqrt(1 - beta2^t)).
AdamScalars adam_scalars(const fsdp_adamw_hp& hp);
// Compute units of the current device (cached per device; 256 if unknown).
int cu_count();
// The divisor of the reduce-scatter average: N, and 1/N for the specialised kernels.
ReduceScalars reduce_scalars(int world);
// FSDP_E_INVAL (message prefixed with fn) unless hp is non-NULL, step >= 1,
// both betas lie in [0, 1) and lr, weight_decay and eps are >= 0 (not NaN).
int check_hp(const char* fn, const fsdp_adamw_hp* hp);

}  // namespace fsdp
