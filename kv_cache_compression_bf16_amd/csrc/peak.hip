// libkvc_peak: on-chip peak probes for the benchmark's roofline figures.
//
// Measurement support only -- not part of the compression path.  Each probe is
// one kernel launch on the caller's stream; the caller times it (HIP events on
// the same stream) and divides the work below by the duration:
//   kvc_peak_read  -- every byte of a buffer read once with 16-byte loads,
//                     consecutive lanes on consecutive 16-byte chunks (a plain
//                     read stream; a buffer well above the 256 MB Infinity
//                     Cache measures HBM, one below it the cache);
//   kvc_peak_mfma  -- back-to-back v_mfma_f32_32x32x16_bf16 with four
//                     independent accumulators per wave, 8 waves per SIMD
//                     worth of workgroups: dense bf16 matrix throughput;
//   kvc_peak_valu  -- 16 independent chains per lane of one vector
//                     instruction class (fp32 FMA, fp32 add, exp2, log2, the
//                     32x32->64 integer product of a Philox round together
//                     with one three-input xor, or the three-input xor
//                     alone), 8 waves per SIMD: the issue rate of that class.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc_peak.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

// Each thread reads kReadUnroll chunks of 16 bytes per step, all in flight,
// grid-striding over the buffer; the xor of everything read goes to sink so
// no load is dead.
__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4* src, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

constexpr int kMfmaThreads = 512;

__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  const u32x4 va = {0x3c003c00u ^ (uint32_t)(lane & 0x7f), 0x3c003c00u, 0x3c003c00u ^ (uint32_t)((lane * 3) & 0x7f),
                    0x3c003c00u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, va), b = a;
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  sink[(int64_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

constexpr int kValuThreads = 1024;
constexpr int kChains = 16;

template <int kOp>
__global__ __launch_bounds__(kValuThreads) void valu_kernel(float* sink, int iters, float a) {
  float x[kChains];
  uint32_t u[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) {
    x[i] = 0.25f + 0.01f * (float)i + (float)threadIdx.x * 1e-6f;
    u[i] = threadIdx.x * 2654435761u + (uint32_t)i;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
      if constexpr (kOp == KVC_PEAK_FMA) x[i] = fmaf(x[i], a, 0.125f);
      if constexpr (kOp == KVC_PEAK_ADD) x[i] = x[i] + a;
      if constexpr (kOp == KVC_PEAK_EXP2) x[i] = __builtin_amdgcn_exp2f(-x[i]);             // stays in [0.5, 1]
      if constexpr (kOp == KVC_PEAK_LOG2) x[i] = __builtin_amdgcn_logf(fabsf(x[i]));        // |x|: a free source modifier
      if constexpr (kOp == KVC_PEAK_MAD_U64) {
        const uint64_t p = (uint64_t)0xD2511F53u * u[i];   // the 32x32->64 product of a Philox round
        u[i] = __builtin_amdgcn_bitop3_b32((uint32_t)(p >> 32), (uint32_t)p, (uint32_t)i, 0x96);
      }
    }
    if constexpr (kOp == KVC_PEAK_BITOP3) {
      uint32_t v[kChains];
#pragma unroll
      for (int i = 0; i < kChains; ++i) v[i] = __builtin_amdgcn_bitop3_b32(u[i], u[(i + 1) % kChains], 0x9E3779B9u, 0x96);
#pragma unroll
      for (int i = 0; i < kChains; ++i) u[i] = v[i];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += x[i] + (float)u[i];
  sink[(int64_t)blockIdx.x * kValuThreads + threadIdx.x] = s;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

}  // namespace

extern "C" {

int kvc_peak_cus(void) { return device_cus(); }

size_t kvc_peak_read_sink_words(void) {
  const int cus = device_cus();
  return cus > 0 ? (size_t)cus * 8 * kReadThreads : 0;
}

int kvc_peak_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  const int cus = device_cus();
  if (!buf || !sink || cus <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15)) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(cus * 8), dim3(kReadThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

size_t kvc_peak_mfma_sink_words(void) {
  const int cus = device_cus();
  return cus > 0 ? (size_t)cus * 2 * kMfmaThreads : 0;
}

double kvc_peak_mfma_flops(int iters) {
  const int cus = device_cus();
  // waves x iterations x 4 MFMAs x 32*32*16*2 flops
  return (double)cus * 2 * (kMfmaThreads / 64) * (double)iters * 4 * 32768.0;
}

int kvc_peak_mfma(float* sink, int iters, void* stream) {
  const int cus = device_cus();
  if (!sink || cus <= 0 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3(cus * 2), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream), sink,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

size_t kvc_peak_valu_sink_words(void) {
  const int cus = device_cus();
  return cus > 0 ? (size_t)cus * 2 * kValuThreads : 0;
}

double kvc_peak_valu_wave_instructions(int iters) {
  const int cus = device_cus();
  return (double)cus * 2 * (kValuThreads / 64) * (double)iters * kChains;
}

int kvc_peak_valu(int op, float* sink, int iters, void* stream) {
  const int cus = device_cus();
  if (!sink || cus <= 0 || iters < 1) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(cus * 2), block(kValuThreads);
  switch (op) {
    case KVC_PEAK_FMA: hipLaunchKernelGGL(valu_kernel<KVC_PEAK_FMA>, grid, block, 0, s, sink, iters, 0.999f); break;
    case KVC_PEAK_ADD: hipLaunchKernelGGL(valu_kernel<KVC_PEAK_ADD>, grid, block, 0, s, sink, iters, 0.999f); break;
    case KVC_PEAK_EXP2: hipLaunchKernelGGL(valu_kernel<KVC_PEAK_EXP2>, grid, block, 0, s, sink, iters, 0.999f); break;
    case KVC_PEAK_LOG2: hipLaunchKernelGGL(valu_kernel<KVC_PEAK_LOG2>, grid, block, 0, s, sink, iters, 0.999f); break;
    case KVC_PEAK_MAD_U64:
      hipLaunchKernelGGL(valu_kernel<KVC_PEAK_MAD_U64>, grid, block, 0, s, sink, iters, 0.999f);
      break;
    case KVC_PEAK_BITOP3:
      hipLaunchKernelGGL(valu_kernel<KVC_PEAK_BITOP3>, grid, block, 0, s, sink, iters, 0.999f);
      break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
