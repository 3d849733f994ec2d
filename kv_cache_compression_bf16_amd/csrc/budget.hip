// kvc_lmba_budget: ZigZag per-layer budgets.
//
// ZigZagKV blog page, section on its new observations: MBA is the fewest KV
// entries that keep 90% of a head's total attention score, LMBA the mean MBA of
// a layer's heads; section on the space allocation: every layer gets a minimum,
// and the rest of the total budget is shared in proportion to LMBA.
//
// Design:
//  * mba_kernel, one workgroup per (layer, head).  Masses are exact 64-bit
//    fixed-point integers x_fix = floor(x * 2^shift), with shift chosen so that
//    n copies of the row's largest score still fit in 62 bits; integer sums
//    are exact and order-independent, so LDS atomics keep the result
//    bit-reproducible.  (Truncation loses less than n * 2^-shift of the total,
//    about 1e-10 of the largest score for n = 16K.)  The threshold key T (the
//    largest score whose "at least T" mass reaches mass*total) is found by a
//    radix search on key - min over the order-preserving 32-bit keys, each
//    level taking the next (up to) 11 bits below the top set bit of max - min
//    and histogramming count and mass per bin.  MBA = (#scores > T) + the
//    fewest T-valued scores that close the remaining gap.
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

// Workgroup-wide exclusive prefix sum of uint64 values; *total gets the sum.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t x, uint64_t* wsum, uint64_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint64_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  uint64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kMbaWaves; ++i) {
    const uint64_t s = wsum[i];
    before += (i < wid) ? s : 0ull;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + v - x;
}

// The mass a head's kept scores must reach: ceil of the fp64 product
// total * mass (the rounding the threshold test of the MBA definition uses in
// fp64), never more than total, and exactly total for mass = 1.  Without the
// clamp, the rounding of total to fp64 can put the target above the total,
// and then no bin of the radix search below reaches it.
__device__ __forceinline__ uint64_t mass_target(uint64_t total, double mass) {
  if (mass >= 1.0) return total;
  const double t = ceil((double)total * mass);
  if (!(t < 18446744073709551616.0)) return total;   // 2^64: out of range (cannot happen for mass < 1)
  const uint64_t u = (uint64_t)t;
  return u < total ? u : total;
}

constexpr int kMbaBins = 2048;
constexpr int kMbaBPT = kMbaBins / kMbaThreads;   // bins per thread in the suffix scans

// kKPT > 0: the row is read once, kKPT keys per thread held in registers
// together with their fixed-point masses (n <= kKPT * kMbaThreads), and
// every later pass works on those; kKPT = 0: every pass reads the row again.
// Both walk the same keys and add the same integers, so they agree exactly.
template <int kKPT>
__global__ __launch_bounds__(kMbaThreads) void mba_kernel(const float* imp, int n, double mass,
                                                         int32_t* mba_out) {
  __shared__ uint32_t hc[kMbaBins];   // count per bin
  __shared__ uint64_t hm[kMbaBins];   // fixed-point mass per bin
  __shared__ uint64_t wsum[kMbaWaves];
  __shared__ uint32_t wlo[kMbaWaves], whi[kMbaWaves];
  __shared__ uint32_t s_bin;
  __shared__ uint64_t s_above_m;
  __shared__ uint32_t s_above_c;

  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(imp + (int64_t)row * n);

  constexpr int kR = kKPT > 0 ? kKPT : 1;
  uint32_t kr[kR];
  uint64_t fr[kR];
  if constexpr (kKPT > 0) {
#pragma unroll
    for (int i = 0; i < kKPT; ++i) {
      const int j = tid + i * kMbaThreads;
      kr[i] = v[j < n ? j : n - 1];   // clamped address; entries past n are never used
    }
  }
  // -0.0 (bits 0x80000000) is a valid zero score: fold it onto +0.0 so that
  // the raw bits of every score >= 0 are order-preserving keys
  auto key_of = [](uint32_t b) -> uint32_t { return b == 0x80000000u ? 0u : b; };
  // f(key) over this thread's keys: j = tid + i * kMbaThreads, in order
  auto for_keys = [&](auto&& f) {
    if constexpr (kKPT > 0) {
#pragma unroll
      for (int i = 0; i < kKPT; ++i)
        if (tid + i * kMbaThreads < n) f(key_of(kr[i]), i);
    } else {
#pragma unroll 4
      for (int j = tid; j < n; j += kMbaThreads) f(key_of(v[j]), 0);
    }
  };

  // key range (scores are >= 0, so the raw bits are order-preserving keys)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for_keys([&](uint32_t k, int) {
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor(kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, o));
  }
  if (lane == 0) {
    wlo[wid] = kmin;
    whi[wid] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMbaWaves; ++i) {
    kmin = min(kmin, wlo[i]);
    kmax = max(kmax, whi[i]);
  }
  if (kmax == 0u) {   // every score is zero: nothing to keep
    if (tid == 0) mba_out[row] = 0;
    return;
  }

  // fixed point: max < 2^e_max, n < 2^l_n, shift = 62 - l_n - e_max
  int e_max;
  (void)frexp((double)__uint_as_float(kmax), &e_max);
  const int l_n = 32 - __clz((uint32_t)n);
  const int shift = 62 - l_n - e_max;
  auto fix = [&](uint32_t key) -> uint64_t { return (uint64_t)ldexp((double)__uint_as_float(key), shift); };

  uint64_t part = 0;
  for_keys([&](uint32_t k, int i) {
    const uint64_t f = fix(k);
    if constexpr (kKPT > 0) fr[i] = f;
    part += f;
  });
  // fixed-point mass of a key: cached in the register path
  auto fixed = [&](uint32_t k, int i) -> uint64_t {
    if constexpr (kKPT > 0) return fr[i];
    return fix(k);
  };
  uint64_t total;
  (void)block_excl_scan_u64(part, wsum, &total);
  const uint64_t target = mass_target(total, mass);   // keep at least this much (<= total)
  if (target == 0) {
    if (tid == 0) mba_out[row] = 0;
    return;
  }

  // radix search on d = key - kmin, MSB first: bits [top, 32) of T - kmin are
  // known (= hi); the keys above T hold above_m / above_c
  int top = 32 - __clz(kmax - kmin);
  uint32_t hi = 0, above_c = 0, eq = (uint32_t)n;   // eq: keys equal to T (all, if they are all equal)
  uint64_t above_m = 0;
  while (top > 0) {
    const int width = top < 11 ? top : 11;
    const int sh = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    const uint32_t hmask = top >= 32 ? 0u : (0xFFFFFFFFu << top);
    const uint32_t hval = top >= 32 ? 0u : (hi << top);
    for (int b = tid; b < kMbaBins; b += kMbaThreads) {
      hc[b] = 0u;
      hm[b] = 0ull;
    }
    if (tid == 0) {
      s_bin = 0u;
      s_above_m = 0ull;
      s_above_c = 0u;
    }
    __syncthreads();
    for_keys([&](uint32_t k, int i) {
      const uint32_t d = k - kmin;
      if ((d & hmask) == hval) {
        const uint32_t b = (d >> sh) & dmask;
        atomicAdd(&hc[b], 1u);
        atomicAdd(reinterpret_cast<unsigned long long*>(&hm[b]), (unsigned long long)fixed(k, i));
      }
    });
    __syncthreads();
    // suffix sums of mass and count: the thread owns kMbaBPT bins from base
    const int base = kMbaBPT * (kMbaThreads - 1 - tid);
    uint64_t m_own = 0;
    uint32_t c_own = 0;
#pragma unroll
    for (int i = 0; i < kMbaBPT; ++i) {
      m_own += hm[base + i];
      c_own += hc[base + i];
    }
    uint64_t mtot;
    const uint64_t m_higher = block_excl_scan_u64(m_own, wsum, &mtot);   // mass in bins >= base + kMbaBPT
    const uint64_t c_higher = block_excl_scan_u64(c_own, wsum, &mtot);
    // the crossing bin: the highest b with above_m + mass(bins >= b) >= target
    uint64_t sm = m_higher;
    uint64_t sc = c_higher;
#pragma unroll
    for (int i = kMbaBPT - 1; i >= 0; --i) {
      const uint64_t up_m = sm, up_c = sc;   // bins > base + i
      sm += hm[base + i];
      sc += hc[base + i];
      if (above_m + sm >= target && above_m + up_m < target) {
        s_bin = (uint32_t)(base + i);
        s_above_m = up_m;
        s_above_c = (uint32_t)up_c;
      }
    }
    __syncthreads();
    hi = (hi << width) | s_bin;
    above_m += s_above_m;
    above_c += s_above_c;
    eq = hc[s_bin];   // after the last level: the keys equal to T
    top = sh;
    __syncthreads();
  }
  if (tid == 0) {
    // the eq keys equal to T = kmin + hi close the gap
    const uint64_t xt = fix(kmin + hi);
    const uint64_t need = target - above_m;   // > 0 by construction
    uint64_t e = xt > 0 ? (need + xt - 1) / xt : (uint64_t)eq;
    if (e < 1) e = 1;
    if (e > eq) e = eq;
    mba_out[row] = (int32_t)(above_c + e);
  }
}

// Workgroup sum of int64 over kThreads threads (all threads get it).
template <int kThreads>
__device__ int64_t block_sum_i64(int64_t x, int64_t* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  if (kThreads == kWave) return x;   // one wave: no exchange needed
  if (lane == 0) scratch[wid] = x;
  __syncthreads();
  int64_t t = 0;
  for (int i = 0; i < kThreads / kWave; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

// One thread per layer: kThreads = 64 (a single wave, no workgroup barriers
// in the sums) up to 64 layers, kAllocThreads beyond.
template <int kThreads>
__global__ __launch_bounds__(kThreads) void allocate_kernel(const int32_t* mba, int L, int Hkv, int64_t total,
                                                            int floor_l, int cap, int32_t* budgets) {
  __shared__ int64_t s_rem[kThreads];
  __shared__ int s_free[kThreads];
  __shared__ int64_t scratch[kThreads / kWave];
  auto block_sum = [&](int64_t x) { return block_sum_i64<kThreads>(x, scratch); };

  const int l = threadIdx.x;
  const bool has = l < L;
  // M_l = sum of the layer's MBA over its KV heads, 8 loads in flight at a time
  int64_t M = 0;
  if (has)
    for (int g0 = 0; g0 < Hkv; g0 += 8) {
      int32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = g0 + e < Hkv ? mba[(int64_t)l * Hkv + g0 + e] : 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) M += v[e];
    }
  bool clamped = false;
  for (int iter = 0; iter <= L; ++iter) {
    const int64_t nclamped = block_sum(has && clamped ? 1 : 0);
    const int64_t R = total - (int64_t)L * floor_l - nclamped * (int64_t)(cap - floor_l);
    const bool fr = has && !clamped;
    const int64_t Wsum = block_sum(fr ? M : 0);
    const int64_t nfree = block_sum(fr ? 1 : 0);
    const int64_t w = fr ? (Wsum > 0 ? M : 1) : 0;
    const int64_t W = Wsum > 0 ? Wsum : nfree;
    int64_t q = 0, rem = 0;
    if (fr && W > 0) {
      q = (R * w) / W;
      rem = (R * w) % W;
    }
    const int64_t left = R - block_sum(q);
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
    const int64_t nover = block_sum(over ? 1 : 0);
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
  if (n <= 16 * kMbaThreads)
    KVC_LAUNCH("lmba_mba", mba_kernel<16>, dim3(L * Hkv), dim3(kMbaThreads), s, importance, n, mass, mba_buf);
  else
    KVC_LAUNCH("lmba_mba", mba_kernel<0>, dim3(L * Hkv), dim3(kMbaThreads), s, importance, n, mass, mba_buf);
  if (L <= kWave)
    KVC_LAUNCH("lmba_allocate", allocate_kernel<kWave>, dim3(1), dim3(kWave), s, mba_buf, L, Hkv, total_budget,
               floor_per_layer, capacity, budgets);
  else
    KVC_LAUNCH("lmba_allocate", allocate_kernel<kAllocThreads>, dim3(1), dim3(kAllocThreads), s, mba_buf, L, Hkv,
               total_budget, floor_per_layer, capacity, budgets);
  return KVC_OK;
}
