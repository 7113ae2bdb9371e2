// host_util.h -- host helpers shared by the entry points of libssmscan.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ssm {

// Records a failed HIP call for ssm_last_hip_error() and returns SSM_ERR_HIP.
int hip_fail(hipError_t e);

// Compute units of the current device (queried once per device; 256 when the
// query fails).
int cu_count_cached();

// Workgroups of `block` threads of kernel f one compute unit holds at once
// (registers and LDS decide), or 0 when the runtime cannot say (no device);
// cached per kernel.
int blocks_per_cu(const void *f, int block);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace ssm
