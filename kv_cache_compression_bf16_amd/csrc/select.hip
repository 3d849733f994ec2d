// kvc_select_topk: per-head top-k of the importance plus the recent window.
//
// Selection rule (ZigZagKV blog page, SnapKV and token-selection sections;
// Keyformer blog page, prompt phase): candidates are positions [0, c),
// c = min(S - w, S - recent); the k_top = budget - recent candidates first in
// (importance descending, position ascending) order are kept together with
// every position of [S - recent, S); kept positions are written ascending.
//
// Design: one 512-thread workgroup per head runs an exact MSB-first radix
// select on order-preserving 32-bit keys of the fp32 scores (digits of 11, 11
// and 10 bits; LDS histograms with integer atomics, which are exact and
// order-independent).  That yields the k_top-th key T and how many T-valued
// candidates must be taken.  Each wave owns a contiguous range of candidates
// loaded with coalesced 256-byte loads, 64 in flight per lane, and kept in
// registers across all radix passes; the ordered output transposes them
// through LDS so each thread owns 64 consecutive candidates (see below).
#include "common.h"

namespace kvc {
namespace {

constexpr int kSelThreads = 512;
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

// Candidates are handled in rounds of kRound = 512 * 64: in round r, wave w
// owns the contiguous range [r*kRound + w*4096, +4096) and lane l holds
// candidates base + 64*i + l (i < 64), so every load instruction reads 256
// contiguous bytes and a lane keeps 64 loads in flight.  With one round (up to
// 32768 candidates) the keys are loaded once and stay in registers for all
// radix levels and both emission passes.
constexpr int kVPL = 64;
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
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t s_digit, s_above;
  __shared__ uint32_t tr[kRound + kRound / 64];   // 130 KB transpose buffer of one round

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

  // ---- radix select of the k_top-th largest key
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k_top;
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t width_mask = (pass == 2) ? 0x3FFu : 0x7FFu;
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
      for (int i = 0; i < kVPL; ++i)
        if (j0 + 64 * i < c && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> sh) & width_mask], 1u);
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
    prefix |= s_digit << sh;
    pmask |= width_mask << sh;
    krem -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;   // k_top-th largest key; take krem of the keys equal to T

  // ---- ordered emission, round by round.  The round's keys are transposed
  // through LDS (word j at j + j/64: conflict-free both ways) so that thread t
  // owns the 64 consecutive candidates [64t, 64t + 64); per-thread counts, two
  // workgroup scans for the offsets, then each thread writes its kept positions
  // in order: the output is ascending without a sort.
  uint32_t eq_carry = 0, out_carry = 0;
  for (int r = 0; r < rounds; ++r) {
    if (rounds > 1) {
      __syncthreads();   // the previous round's readers are done with `tr`
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
      mine[e] = tr[seg + e + tid];                   // = position seg + e, padded
      n_gt += (e < valid && mine[e] > T) ? 1u : 0u;
      n_eq += (e < valid && mine[e] == T) ? 1u : 0u;
    }
    uint32_t eq_tot, take_tot;
    const uint32_t eq_b = block_excl_scan(n_eq, wsum, &eq_tot) + eq_carry;
    const uint32_t room = krem > eq_b ? krem - eq_b : 0u;
    const uint32_t n_take = n_gt + (n_eq < room ? n_eq : room);
    uint32_t pos = block_excl_scan(n_take, wsum, &take_tot) + out_carry;
    uint32_t eq_left = n_eq < room ? n_eq : room;    // T-valued candidates this thread keeps
    const int jb = r * kRound + seg;
#pragma unroll
    for (int e = 0; e < kVPL; ++e) {
      const bool in = e < valid;
      const bool eq = in && mine[e] == T;
      const bool take = (in && mine[e] > T) || (eq && eq_left > 0);
      eq_left -= (eq && eq_left > 0) ? 1u : 0u;
      if (take && pos < (uint32_t)k_top) o[pos] = jb + e;
      pos += take ? 1u : 0u;
    }
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
