// kvc_pool_importance: SnapKV's 1D pooling of each head's importance.
//
// ZigZagKV blog page, SnapKV section: the window-averaged scores are pooled
// along the keys before the top-k, so the neighbours of a strong token are
// kept with it.  Here (the page gives no parameters): odd kernel k, stride 1,
// window [j - k/2, j + k/2]; average pooling counts positions outside [0, n)
// as zeros and divides by k, max pooling takes the maximum over the in-range
// part of the window.
//
// Design: one 256-thread workgroup per 1024 outputs of a row stages the tile
// plus its halo in LDS (padding value outside the row), then each thread
// produces 4 outputs, each summed (or maxed) over its window in a fixed
// order, so the result is bit-reproducible.  HBM-bound: one read and one
// write of the importance.
#include <math.h>

#include "common.h"

namespace kvc {
namespace {

constexpr int kPoolOut = 1024;     // outputs per workgroup
constexpr int kPoolMaxK = 255;     // largest kernel size

template <int kMode>
__global__ __launch_bounds__(256) void pool_kernel(const float* in, int64_t ins, float* out, int64_t outs, int n,
                                                    int k) {
  __shared__ float tile[kPoolOut + kPoolMaxK];
  const int row = blockIdx.y, j0 = blockIdx.x * kPoolOut, h = k >> 1;
  const float* x = in + (int64_t)row * ins;
  const float pad = kMode == KVC_POOL_AVG ? 0.f : -INFINITY;
  for (int i = threadIdx.x; i < kPoolOut + 2 * h; i += 256) {
    const int j = j0 - h + i;
    tile[i] = (j >= 0 && j < n) ? x[j] : pad;
  }
  __syncthreads();
  float* y = out + (int64_t)row * outs;
#pragma unroll
  for (int q = 0; q < kPoolOut / 256; ++q) {
    const int o = q * 256 + threadIdx.x, j = j0 + o;
    if (j >= n) break;
    float acc = tile[o];
    for (int i = 1; i < k; ++i) acc = kMode == KVC_POOL_AVG ? acc + tile[o + i] : fmaxf(acc, tile[o + i]);
    y[j] = kMode == KVC_POOL_AVG ? acc / (float)k : acc;
  }
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_pool_importance(const float* in, int64_t in_stride, float* out, int64_t out_stride,
                                          int32_t rows, int32_t n, int32_t kernel, int32_t mode, void* stream) {
  using namespace kvc;
  if (rows < 1 || n < 1 || kernel < 1 || !(kernel & 1) || kernel > kPoolMaxK) return KVC_E_ARG;
  if (mode != KVC_POOL_AVG && mode != KVC_POOL_MAX) return KVC_E_ARG;
  if (!in || !out || in == out) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(in) & 3) || (reinterpret_cast<uintptr_t>(out) & 3)) return KVC_E_ARG;
  if (rows > 1 && (in_stride < n || out_stride < n)) return KVC_E_SHAPE;
  if (rows > 65535) return KVC_E_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((n + kPoolOut - 1) / kPoolOut, rows), block(256);
  if (mode == KVC_POOL_AVG)
    KVC_LAUNCH("pool_importance", pool_kernel<KVC_POOL_AVG>, grid, block, s, in, in_stride, out, out_stride, n, kernel);
  else
    KVC_LAUNCH("pool_importance", pool_kernel<KVC_POOL_MAX>, grid, block, s, in, in_stride, out, out_stride, n, kernel);
  return KVC_OK;
}
