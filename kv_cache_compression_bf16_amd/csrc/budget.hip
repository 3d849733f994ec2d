// kvc_lmba_budget: ZigZag per-layer budgets.
//
// ZigZagKV blog page, section on its new observations: MBA is the fewest KV
// entries that keep 90% of a head's total attention score, LMBA the mean MBA of
// a layer's heads; section on the space allocation: every layer gets a minimum,
// and the rest of the total budget is shared in proportion to LMBA.
//
// Design:
//  * mba_kernel, one workgroup per (layer, head): the row's total mass is an
//    fp64 sum in a fixed order; the threshold key T (the largest score whose
//    "at least T" mass reaches mass*total) is found by an 8-level, 16-way
//    search over the order-preserving 32-bit keys of the scores.  At each level
//    every thread accumulates the mass and count of each of the 16 digit
//    buckets in registers, and buckets are combined across the workgroup in a
//    fixed tree order, so the result is bit-reproducible (no floating-point
//    atomics).  MBA = (#scores > T) + the fewest T-valued scores that close the
//    remaining gap.
//  * allocate_kernel, one workgroup: exact int64 largest-remainder shares with
//    the floor, capacity clamping and re-sharing (water-filling).
#include <math.h>

#include "common.h"

namespace kvc {
namespace {

constexpr int kMbaThreads = 1024;
constexpr int kMbaWaves = kMbaThreads / kWave;
constexpr int kAllocThreads = 1024;
constexpr int kMaxLayers = 1024;

__device__ __forceinline__ double shfl_xor_f64(double x, int o) {
  return __shfl_xor(x, o);
}

// Fixed-order workgroup sum of one double per thread (all threads get it).
__device__ double block_sum_f64(double x, double* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += shfl_xor_f64(x, o);
  if (lane == 0) scratch[wid] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kMbaWaves; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kMbaThreads) void mba_kernel(const float* imp, int n, double mass,
                                                         int32_t* mba_out) {
  __shared__ double sm[kMbaWaves][16];
  __shared__ uint32_t sc[kMbaWaves][16];
  __shared__ double sred[kMbaWaves];

  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(imp + (int64_t)row * n);

  double part = 0.0;
#pragma unroll 4
  for (int j = tid; j < n; j += kMbaThreads) part += (double)__uint_as_float(v[j]);
  const double total = block_sum_f64(part, sred);
  const double target = mass * total;
  if (!(target > 0.0)) {
    if (tid == 0) mba_out[row] = 0;
    return;
  }

  uint32_t prefix = 0;       // digits of T fixed so far
  double above_m = 0.0;      // mass of scores whose key exceeds every key still in play
  int64_t above_c = 0;
  uint32_t eq_count = 0;
  for (int sh = 28; sh >= 0; sh -= 4) {
    double bm[16];
    uint32_t bc[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      bm[d] = 0.0;
      bc[d] = 0u;
    }
#pragma unroll 4
    for (int j = tid; j < n; j += kMbaThreads) {
      const uint32_t key = v[j];   // scores are >= 0: raw bits already order-preserving
      const bool live = (sh == 28) || ((key >> (sh + 4)) == (prefix >> (sh + 4)));
      if (live) {
        const uint32_t d = (key >> sh) & 15u;
        const double x = (double)__uint_as_float(key);
#pragma unroll
        for (int dd = 0; dd < 16; ++dd) {
          bm[dd] += (d == (uint32_t)dd) ? x : 0.0;
          bc[dd] += (d == (uint32_t)dd) ? 1u : 0u;
        }
      }
    }
    // fixed-order reduction of the 16 buckets: wave butterfly, then waves 0..3
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      double m = bm[d];
      uint32_t cnt = bc[d];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        m += shfl_xor_f64(m, o);
        cnt += __shfl_xor(cnt, o);
      }
      if (lane == 0) {
        sm[wid][d] = m;
        sc[wid][d] = cnt;
      }
    }
    __syncthreads();
    // every thread walks the 16 digits from the top (identical, uniform result):
    // T's digit is the highest one whose bucket brings the mass to the target
    bool found = false;
    int dstar = -1, dlow = -1;
    double cum = above_m, mlow = 0.0;
    int64_t cumc = above_c;
    uint32_t clow = 0;
#pragma unroll
    for (int d = 15; d >= 0; --d) {
      double m = 0.0;
      uint32_t cnt = 0;
#pragma unroll
      for (int w = 0; w < kMbaWaves; ++w) {
        m += sm[w][d];
        cnt += sc[w][d];
      }
      if (!found && cnt > 0) {
        if (cum + m >= target) {
          found = true;
          dstar = d;
          eq_count = cnt;
        } else {
          cum += m;
          cumc += cnt;
          dlow = d;
          mlow = m;
          clow = cnt;
        }
      }
    }
    if (!found) {   // rounding kept the target out of reach: T lies in the lowest live bucket
      dstar = dlow;
      cum -= mlow;
      cumc -= clow;
      eq_count = clow;
    }
    above_m = cum;
    above_c = cumc;
    prefix |= (uint32_t)dstar << sh;
    __syncthreads();
  }
  if (tid == 0) {
    const double t = (double)__uint_as_float(prefix);
    const double need = target - above_m;
    int64_t e;
    if (!(t > 0.0)) {
      e = eq_count;
    } else {
      e = (int64_t)ceil(need / t);
      if (e < 1) e = 1;
      if (e > (int64_t)eq_count) e = eq_count;
      while (e > 1 && above_m + (double)(e - 1) * t >= target) --e;
      while (e < (int64_t)eq_count && above_m + (double)e * t < target) ++e;
    }
    mba_out[row] = (int32_t)(above_c + e);
  }
}

// Fixed-order workgroup sum of int64 (all threads get it).
__device__ int64_t block_sum_i64(int64_t x, int64_t* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  if (lane == 0) scratch[wid] = x;
  __syncthreads();
  int64_t t = 0;
  for (int i = 0; i < kAllocThreads / kWave; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kAllocThreads) void allocate_kernel(const int32_t* mba, int L, int Hkv,
                                                                int64_t total, int floor_l, int cap,
                                                                int32_t* budgets) {
  __shared__ int64_t s_rem[kMaxLayers];
  __shared__ int s_free[kMaxLayers];
  __shared__ int64_t scratch[kAllocThreads / kWave];

  const int l = threadIdx.x;
  const bool has = l < L;
  int64_t M = 0;
  if (has)
    for (int g = 0; g < Hkv; ++g) M += mba[(int64_t)l * Hkv + g];
  bool clamped = false;
  for (int iter = 0; iter <= L; ++iter) {
    const int64_t nclamped = block_sum_i64(has && clamped ? 1 : 0, scratch);
    const int64_t R = total - (int64_t)L * floor_l - nclamped * (int64_t)(cap - floor_l);
    const bool fr = has && !clamped;
    const int64_t Wsum = block_sum_i64(fr ? M : 0, scratch);
    const int64_t nfree = block_sum_i64(fr ? 1 : 0, scratch);
    const int64_t w = fr ? (Wsum > 0 ? M : 1) : 0;
    const int64_t W = Wsum > 0 ? Wsum : nfree;
    int64_t q = 0, rem = 0;
    if (fr && W > 0) {
      q = (R * w) / W;
      rem = (R * w) % W;
    }
    const int64_t left = R - block_sum_i64(q, scratch);
    if (has) {
      s_rem[l] = rem;
      s_free[l] = fr ? 1 : 0;
    }
    __syncthreads();
    if (fr) {
      int64_t rank = 0;
      for (int m = 0; m < L; ++m) {
        if (!s_free[m]) continue;
        const int64_t rm = s_rem[m];
        rank += (rm > rem || (rm == rem && m < l)) ? 1 : 0;
      }
      if (rank < left) q += 1;
    }
    __syncthreads();
    const bool over = fr && (int64_t)floor_l + q > (int64_t)cap;
    const int64_t nover = block_sum_i64(over ? 1 : 0, scratch);
    if (nover == 0) {
      if (has) budgets[l] = clamped ? cap : (int32_t)(floor_l + q);
      return;
    }
    if (over) clamped = true;
  }
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_lmba_budget_workspace_size(int32_t L, int32_t Hkv, int32_t n) {
  (void)n;
  if (L < 1 || Hkv < 1) return 0;
  return kvc::align_up((size_t)L * Hkv * sizeof(int32_t), 256);
}

extern "C" kvc_status kvc_lmba_budget(const float* importance, int32_t L, int32_t Hkv, int32_t n,
                                      double mass, int64_t total_budget, int32_t floor_per_layer,
                                      int32_t capacity, int32_t* mba, int32_t* budgets, void* ws,
                                      size_t ws_bytes, void* stream) {
  using namespace kvc;
  if (L < 1 || L > kMaxLayers || Hkv < 1 || n < 1) return KVC_E_ARG;
  if (!(mass > 0.0 && mass <= 1.0)) return KVC_E_ARG;
  if (floor_per_layer < 0 || capacity < floor_per_layer) return KVC_E_ARG;
  if (total_budget < (int64_t)L * floor_per_layer || total_budget > (int64_t)L * capacity) return KVC_E_ARG;
  if (total_budget >= ((int64_t)1 << 31) || (int64_t)Hkv * n >= ((int64_t)1 << 31)) return KVC_E_SHAPE;
  if ((int64_t)L * Hkv > 65535) return KVC_E_SHAPE;
  if (!importance || !budgets) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(importance) & 3) || (reinterpret_cast<uintptr_t>(budgets) & 3) ||
      (reinterpret_cast<uintptr_t>(mba) & 3))
    return KVC_E_ARG;
  int32_t* mba_buf = mba;
  if (!mba_buf) {
    if (!ws || ws_bytes < kvc_lmba_budget_workspace_size(L, Hkv, n)) return KVC_E_WORKSPACE;
    mba_buf = static_cast<int32_t*>(ws);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  KVC_LAUNCH("lmba_mba", mba_kernel, dim3(L * Hkv), dim3(kMbaThreads), s, importance, n, mass, mba_buf);
  KVC_LAUNCH("lmba_allocate", allocate_kernel, dim3(1), dim3(kAllocThreads), s, mba_buf, L, Hkv,
             total_budget, floor_per_layer, capacity, budgets);
  return KVC_OK;
}
