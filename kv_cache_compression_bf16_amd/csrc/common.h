// Shared definitions for the libkvc HIP sources (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc.h"

namespace kvc {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // one MFMA operand (8 x bf16)
typedef __attribute__((ext_vector_type(16))) float f32x16;   // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // 16 raw bytes

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---- host-side launch bookkeeping (kvc_common.hip) -------------------------
// Every launch goes through launch_begin / launch_end so that kernel timing
// (kvc_timing_enable) and launch-error mapping live in one place.
int launch_begin(const char* name, hipStream_t s);
kvc_status launch_end(int slot, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device (queried once per device), or 0 if the
// query fails.
int device_cu_count();
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace kvc

// Launch `kernel<<<grid, block, shm, stream>>>(args...)` with timing and error
// mapping; returns from the calling function on failure.
#define KVC_LAUNCH_SHM(name, kernel, grid, block, shm, stream, ...)             \
  do {                                                                         \
    int kvc_slot_ = ::kvc::launch_begin(name, stream);                         \
    hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);         \
    kvc_status kvc_st_ = ::kvc::launch_end(kvc_slot_, stream);                 \
    if (kvc_st_ != KVC_OK) return kvc_st_;                                     \
  } while (0)
#define KVC_LAUNCH(name, kernel, grid, block, stream, ...) \
  KVC_LAUNCH_SHM(name, kernel, grid, block, 0, stream, __VA_ARGS__)
