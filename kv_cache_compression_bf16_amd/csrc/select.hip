// kvc_select_topk: per-head top-k of the importance plus the recent window.
//
// Selection rule (ZigZagKV blog page, SnapKV and token-selection sections;
// Keyformer blog page, prompt phase): candidates are positions [0, c),
// c = min(S - w, S - recent); the k_top = budget - recent candidates first in
// (importance descending, position ascending) order are kept together with
// every position of [S - recent, S); kept positions are written ascending.
//
// Design: one 1024-thread workgroup per head runs an exact MSB-first radix
// select on order-preserving 32-bit keys of the fp32 scores, relative to the
// head's smallest key: d = key - min, and each level histograms the next (up
// to) 11 bits below the highest set bit of max - min.  Scores of one head
// usually span a narrow key range (similar exponents), so the first level
// already spreads them over the bins (few LDS-atomic collisions) and often
// two levels suffice.  Integer atomics are exact and order-independent.  The
// select yields the k_top-th key T and how many T-valued candidates must be
// taken.  Each wave owns a contiguous range of candidates loaded with
// coalesced 256-byte loads, 64 in flight per lane, and kept in registers
// across all levels; the ordered output transposes them through LDS so each
// thread owns 64 consecutive candidates, and the kept positions are staged
// in LDS and written out coalesced.
#include "common.h"

namespace kvc {
namespace {

#ifndef KVC_SEL_THREADS
#define KVC_SEL_THREADS 1024
#endif
constexpr int kSelThreads = KVC_SEL_THREADS;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBins = 2048;
constexpr int kBPT = kBins / kSelThreads;   // histogram bins per thread in the scan

// fp32 -> uint32 with the same order (-0 folded onto +0).
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; *total receives the sum of all x.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const uint32_t s = wsum[i];
    before += (i < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + v - x;
}

// Workgroup-wide (min, max); every thread receives the result.
__device__ __forceinline__ void block_min_max(uint32_t& lo, uint32_t& hi, uint32_t* wlo, uint32_t* whi) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor(lo, o));
    hi = max(hi, (uint32_t)__shfl_xor(hi, o));
  }
  if (lane == 0) {
    wlo[wid] = lo;
    whi[wid] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    lo = min(lo, wlo[i]);
    hi = max(hi, whi[i]);
  }
  __syncthreads();
}

// Candidates are handled in rounds of kRound = 32768: in round r, wave w owns
// the contiguous range [r*kRound + w*kSpan, +kSpan) and lane l holds
// candidates base + 64*i + l (i < kVPL), so every load instruction reads 256
// contiguous bytes and a lane keeps kVPL loads in flight.  With one round (up
// to 32768 candidates) the keys are loaded once and stay in registers for all
// radix levels and both emission passes.
constexpr int kVPL = 32768 / kSelThreads;          // candidates per lane per round
constexpr int kSpan = kVPL * kWave;                 // candidates per wave per round
constexpr int kRound = kSelWaves * kSpan;

__device__ __forceinline__ void load_round(const uint32_t* v, int c, int r, uint32_t (&key)[kVPL]) {
  const int base = r * kRound + (int)(threadIdx.x >> 6) * kSpan + (int)(threadIdx.x & 63);
  // Unconditional loads from a clamped address (then masked): a guarded load
  // would be a branch, and the wait at each branch merge would serialize them.
  uint32_t raw[kVPL];
#pragma unroll
  for (int i = 0; i < kVPL; ++i) {
    const int j = base + 64 * i;
    raw[i] = v[j < c ? j : c - 1];
  }
#pragma unroll
  for (int i = 0; i < kVPL; ++i) key[i] = (base + 64 * i < c) ? order_key(raw[i]) : 0u;
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(const float* imp, int64_t hs, int c,
                                                                 int k_top, int S, int recent, int budget,
                                                                 int32_t* out) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wsum[kSelWaves], wsum2[kSelWaves];
  __shared__ uint32_t s_digit, s_above;
  __shared__ uint32_t tr[kRound + kRound / 64];   // 130 KB: transposed keys, then kept positions

  const int g = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(imp + (int64_t)g * hs);
  int32_t* o = out + (int64_t)g * budget;

  for (int t = tid; t < recent; t += kSelThreads) o[k_top + t] = S - recent + t;
  if (k_top == 0) return;
  if (k_top >= c) {
    for (int j = tid; j < c; j += kSelThreads) o[j] = j;
    return;
  }

  const int rounds = (c + kRound - 1) / kRound;
  uint32_t key[kVPL];
  if (rounds == 1) load_round(v, c, 0, key);
  const int lbase = wave * kSpan + (tid & 63);   // candidate of key[0] in round 0

  // ---- key range of the candidates
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int r = 0; r < rounds; ++r) {
    if (rounds > 1) load_round(v, c, r, key);
    const int j0 = r * kRound + lbase;
#pragma unroll
    for (int i = 0; i < kVPL; ++i) {
      const bool in = j0 + 64 * i < c;
      kmin = min(kmin, in ? key[i] : 0xFFFFFFFFu);
      kmax = max(kmax, in ? key[i] : 0u);
    }
  }
  block_min_max(kmin, kmax, wsum, wsum2);

  // ---- radix select on d = key - kmin, MSB first.  Bits [top, 32) of the
  // k_top-th largest d are known (= hi); each level resolves up to 11 more.
  int top = 32 - __clz(kmax - kmin);   // 0 when every candidate has the same key
  uint32_t hi = 0, krem = (uint32_t)k_top;
  while (top > 0) {
    const int width = top < 11 ? top : 11;
    const int sh = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    const uint32_t hmask = top >= 32 ? 0u : (0xFFFFFFFFu << top);   // bits already resolved
    const uint32_t hval = top >= 32 ? 0u : (hi << top);
    for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
    if (tid == 0) {
      s_digit = 0;
      s_above = 0;
    }
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
      if (rounds > 1) load_round(v, c, r, key);
      const int j0 = r * kRound + lbase;
#pragma unroll
      for (int i = 0; i < kVPL; ++i) {
        const uint32_t d = key[i] - kmin;
        const bool live = j0 + 64 * i < c && (d & hmask) == hval;
        if (live) atomicAdd(&hist[(d >> sh) & dmask], 1u);
      }
    }
    __syncthreads();
    // suffix counts: thread tid owns bins [kBPT*rt, kBPT*rt + kBPT), rt = last - tid
    const int rt = kSelThreads - 1 - tid;
    uint32_t hb[kBPT], a = 0;
#pragma unroll
    for (int i = 0; i < kBPT; ++i) {
      hb[i] = hist[kBPT * rt + i];
      a += hb[i];
    }
    uint32_t tot;
    const uint32_t incl = block_excl_scan(a, wsum, &tot) + a;   // = count of bins >= kBPT*rt
    uint32_t below = 0;
#pragma unroll
    for (int i = 0; i < kBPT; ++i) {
      const uint32_t suf = incl - below;                          // = count of bins >= kBPT*rt + i
      if (suf >= krem && suf - hb[i] < krem) {
        s_digit = kBPT * rt + i;
        s_above = suf - hb[i];
      }
      below += hb[i];
    }
    __syncthreads();
    hi = (hi << width) | s_digit;
    krem -= s_above;
    top = sh;
    __syncthreads();
  }
  const uint32_t T = kmin + hi;   // k_top-th largest key; take krem of the keys equal to T

  // ---- ordered emission, round by round.  The round's keys are transposed
  // through LDS (word j at j + j/64: conflict-free both ways) so that thread t
  // owns the 64 consecutive candidates [64t, 64t + 64); per-thread counts and
  // two workgroup scans give each thread its output offset; the kept
  // positions go to LDS in order and then out with coalesced stores, so the
  // output is ascending without a sort.
  uint32_t eq_carry = 0, out_carry = 0;
  for (int r = 0; r < rounds; ++r) {
    if (rounds > 1) {
      __syncthreads();   // the previous round's copy-out is done with `tr`
      load_round(v, c, r, key);
    }
    const int j0 = r * kRound + lbase;
#pragma unroll
    for (int i = 0; i < kVPL; ++i) {
      const int jl = j0 - r * kRound + 64 * i;      // position within the round
      tr[jl + (jl >> 6)] = key[i];
    }
    __syncthreads();
    const int seg = tid * kVPL;                      // this thread's first position in the round
    const int valid = min(kVPL, max(0, c - r * kRound - seg));
    uint32_t mine[kVPL];
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int e = 0; e < kVPL; ++e) {
      mine[e] = tr[seg + e + ((seg + e) >> 6)];      // = position seg + e, padded
      n_gt += (e < valid && mine[e] > T) ? 1u : 0u;
      n_eq += (e < valid && mine[e] == T) ? 1u : 0u;
    }
    uint32_t eq_tot, take_tot;
    const uint32_t eq_b = block_excl_scan(n_eq, wsum, &eq_tot) + eq_carry;   // also orders tr reads before writes
    const uint32_t room = krem > eq_b ? krem - eq_b : 0u;
    const uint32_t n_take = n_gt + (n_eq < room ? n_eq : room);
    uint32_t pos = block_excl_scan(n_take, wsum, &take_tot);   // offset within this round's output
    uint32_t eq_left = n_eq < room ? n_eq : room;    // T-valued candidates this thread keeps
    const uint32_t jb = (uint32_t)(r * kRound + seg);
#pragma unroll
    for (int e = 0; e < kVPL; ++e) {
      const bool in = e < valid;
      const bool eq = in && mine[e] == T;
      const bool take = (in && mine[e] > T) || (eq && eq_left > 0);
      eq_left -= (eq && eq_left > 0) ? 1u : 0u;
      if (take) tr[pos] = jb + e;                    // pos < take_tot <= kRound
      pos += take ? 1u : 0u;
    }
    __syncthreads();
    const uint32_t n_out = min(take_tot, (uint32_t)k_top - min(out_carry, (uint32_t)k_top));
    for (uint32_t t = tid; t < n_out; t += kSelThreads) o[out_carry + t] = (int32_t)tr[t];
    eq_carry += eq_tot;
    out_carry += take_tot;
  }
}

}  // namespace
}  // namespace kvc

extern "C" size_t kvc_select_topk_workspace_size(int32_t Hkv, int32_t n) {
  (void)Hkv;
  (void)n;
  return 0;
}

extern "C" kvc_status kvc_select_topk(const float* importance, int64_t imp_head_stride, int32_t Hkv,
                                      int32_t S, int32_t w, int32_t recent, int32_t budget,
                                      int32_t* indices, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (Hkv < 1 || S < 2 || w < 1 || w >= S || recent < 0 || recent > S) return KVC_E_ARG;
  const int32_t n = S - w;
  const int32_t c = n < S - recent ? n : S - recent;
  if (budget < recent || budget - recent > c) return KVC_E_ARG;
  if (imp_head_stride < n && Hkv > 1) return KVC_E_SHAPE;
  if (!indices || (!importance && budget > recent)) return KVC_E_ARG;
  if ((reinterpret_cast<uintptr_t>(importance) & 3) || (reinterpret_cast<uintptr_t>(indices) & 3))
    return KVC_E_ARG;
  if (Hkv > 65535) return KVC_E_SHAPE;
  if (budget == 0) return KVC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  KVC_LAUNCH("select_topk", kvc::select_topk_kernel, dim3(Hkv), dim3(kvc::kSelThreads), s, importance,
             imp_head_stride, c, budget - recent, S, recent, budget, indices);
  return KVC_OK;
}
