// HIP runtime and fixed-width integer types for the kernel headers, which are compiled both by
// hipcc (into the library) and by hipRTC at run time (runtime-compiled score and mask
// modifications).  hipRTC provides the device API itself and keeps the integer types in its
// own namespace.
#pragma once

#ifdef __HIPCC_RTC__
using __hip_internal::int8_t;
using __hip_internal::int16_t;
using __hip_internal::int32_t;
using __hip_internal::int64_t;
using __hip_internal::uint8_t;
using __hip_internal::uint16_t;
using __hip_internal::uint32_t;
using __hip_internal::uint64_t;
#ifndef INFINITY
#define INFINITY __builtin_inff()
#endif
// Only named by the host launch declarations of launch.h, never used at run time.
typedef int hipError_t;
typedef struct ihipStream_t *hipStream_t;
#else
#include <hip/hip_runtime.h>
#include <stdint.h>
#endif
