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

// Row constants of the scoring path's softmax (score.hip), for callers that
// need softmax(scale q k^T) over the first n rows of each KV head of k: q is
// [Hkv*G heads][w][128] bf16 with head stride q_hs, k [Hkv][>= n][128] bf16
// with head stride k_hs; *rowc receives a pointer into ws, [Hkv][G*w] floats
// max + log2(sum) in log2 units.  n >= 1.
size_t score_rowc_workspace_size(int Hkv, int G, int w, int n, int64_t q_hs);
kvc_status score_rowc(const uint16_t* q, int64_t q_hs, const uint16_t* k, int64_t k_hs, int Hkv, int G, int w,
                      int n, float scale, void* ws, size_t ws_bytes, const float** rowc, hipStream_t s);

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
